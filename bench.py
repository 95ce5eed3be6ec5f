"""Benchmark of the verified sparse-attention decode step on one MI355X.

A step is one vattn_decode call (predict, select, base, budget, gather,
combine) over one batch of the Llama-3-8B-shaped workload: 8 sequences of
32768 tokens, 32 query / 8 KV heads, head dim 128, bf16 paged KV cache,
rank-32 low-rank predictor, sinks 128, window 128, top-k 2.5%,
eps = delta = 0.05.  Inputs are synthetic and resident in HBM before timing.
Three copies of the caches are rotated so that no step finds its keys in the
last-level cache.  The sampling seed changes every step.

Prints one JSON line: heads*tokens/s (mean, and the median / p10 / p90 of the
per-step times), the roofline of the dominant kernel (per-kernel HIP events
over the timed steps; algorithmic bytes from the kernel's own token counts),
the whole step's algorithmic HBM rate, a plain device-copy ceiling, the
(eps, delta) violation rate over 1000 seeds against dense fp64 attention, the
same rate, step time and HBM rate for the other long-context workloads (flat
128K, ragged batch of 64, 70B-shaped 64K with an eps sweep), and the CPU oracle
timed on the host cores.
"""
import argparse
import ctypes as C
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "sparse decode heads·tokens/s at 32K ctx; achieved HBM GB/s; ε-violation rate"
HOST_CORE_CAP = 16  # the host CPU share of one GPU on the measurement boxes


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama8b_32k")
    ap.add_argument("--profile", action="store_true",
                    help="the headline steps only, few of them (for rocprofv3 runs)")
    ap.add_argument("--rate-seeds", type=int, default=1000,
                    help="seeds of the (eps, delta) rate of every workload")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other long-context workloads (flat 128K, ragged B64, 70B-shaped 64K)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--base-sweep", default="",
                    help="comma-separated workloads whose (eps, delta) rate, union density and step time "
                         "are also measured at base-sample rates of 5, 10 and 20%% of the tail")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the hash-predictor, output-level and host-resident K/V legs")
    ap.add_argument("--layout-leg", action="store_true",
                    help="also time the workload with its pages in a permuted block table (same tokens, results "
                         "compared bit for bit); opt-in so the default run's kernel trace holds the headline's "
                         "dispatches only")
    ap.add_argument("--pca-basis", action="store_true",
                    help="also time and rate-check the workload with per-KV-head PCA predictor bases")
    return ap.parse_args()


class HipEvents:
    """Raw hipEvent_t handles from the process's HIP runtime (the one torch loaded)."""

    def __init__(self, n):
        self.rt = C.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.rt.hipEventDestroy.argtypes = [C.c_void_p]
        self.ev = []
        for _ in range(n):
            h = C.c_void_p()
            if self.rt.hipEventCreate(C.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(h.value)

    def elapsed(self, a, b):
        ms = C.c_float()
        if self.rt.hipEventElapsedTime(C.byref(ms), C.c_void_p(self.ev[a]), C.c_void_p(self.ev[b])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for h in self.ev:
            self.rt.hipEventDestroy(C.c_void_p(h))


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def clopper_pearson(k, n, conf=0.95):
    """Two-sided exact binomial interval of a rate k / n."""
    from scipy.stats import beta
    a = (1.0 - conf) / 2
    lo = 0.0 if k == 0 else float(beta.ppf(a, k, n - k + 1))
    hi = 1.0 if k == n else float(beta.ppf(1 - a, k + 1, n - k))
    return lo, hi


class Device:
    """One workload on the device: queries, block table, lengths, basis and
    `copies` independent copies of the K, V and low-rank key caches."""

    def __init__(self, w, dev, copies):
        import torch
        import verified_sparse_attention_amd as vsa
        self.w = w
        self.q = w.q.to(dev)
        self.bt = w.block_table.to(dev)
        self.sl = w.seq_lens.to(dev)
        self.proj = w.proj.to(dev) if w.proj is not None else None
        k0, v0 = w.k_cache.to(dev), w.v_cache.to(dev)
        kt0 = vsa.project_keys(k0, self.proj) if w.cfg["predictor"] == 1 else None
        ks0 = vsa.sign_keys(k0, self.proj) if w.cfg["predictor"] == 2 else None
        self.inst = [(k0, v0, kt0, ks0)]
        for _ in range(copies - 1):
            self.inst.append(tuple(None if t is None else t.clone() for t in (k0, v0, kt0, ks0)))
        torch.cuda.synchronize()

    def decoders(self, cfg_dict=None, group_counts=False, workspace=None):
        import verified_sparse_attention_amd as vsa
        cfg = dict(self.w.cfg if cfg_dict is None else cfg_dict)
        out = []
        ws = workspace
        for (k, v, kt, ks) in self.inst:
            d = vsa.Decoder(self.q, k, v, self.bt, self.sl, vsa.Config.from_dict(cfg), max_seq_len=self.w.max_seq_len,
                            k_lowrank=kt, proj=self.proj, k_sig=ks, want_group_counts=group_counts, workspace=ws)
            ws = d.workspace
            out.append(d)
        return out


def time_steps(decs, steps, warm, seed0):
    """Mean ms per step over exactly `steps` decodes (one event before the first
    and after every step, so per-step times come from the same run)."""
    import numpy as np
    import torch
    n = len(decs)
    for s in range(warm):
        decs[s % n].set_seed(seed0 + 100_000 + s)
        decs[s % n]()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t_wall = time.perf_counter()
    ev[0].record()
    for s in range(steps):
        dd = decs[s % n]
        dd.set_seed(seed0 + s)
        dd()
        ev[s + 1].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    return ev[0].elapsed_time(ev[steps]) / steps, per, t_wall


def step_spread(per):
    import numpy as np
    return {"median_ms": round(float(np.median(per)), 5), "p10_ms": round(float(np.quantile(per, 0.1)), 5),
            "p90_ms": round(float(np.quantile(per, 0.9)), 5)}


def dense_reference(D):
    """Dense softmax attention in fp64 over every cached token (torch on the
    device, contiguous operands): the exact quantity the sparse step estimates.
    Returns lse [B, Hq] and out [B, Hq, d] as fp64 device tensors."""
    import math
    import torch
    w = D.w
    k, v = D.inst[0][0], D.inst[0][1]
    B, Hq, Hkv, d = w.B, w.Hq, w.Hkv, w.d
    G = Hq // Hkv
    lse = torch.full((B, Hq), -float("inf"), dtype=torch.float64, device=D.q.device)
    out = torch.zeros(B, Hq, d, dtype=torch.float64, device=D.q.device)
    with torch.no_grad():
        for b in range(B):
            L = int(w.seq_lens[b])
            if L == 0:
                continue
            pages = D.bt[b, :(L + 15) // 16].long()
            Kb = k[pages].permute(1, 0, 2, 3).reshape(Hkv, -1, d)[:, :L].double().contiguous()
            qb = (D.q[b].double() / math.sqrt(d)).view(Hkv, G, d).transpose(1, 2).contiguous()
            s = torch.bmm(Kb, qb).transpose(1, 2).contiguous()  # [Hkv, G, L]
            del Kb
            lse[b] = torch.logsumexp(s, dim=-1).reshape(Hq)
            p = torch.softmax(s, dim=-1)
            del s
            Vb = v[pages].permute(1, 0, 2, 3).reshape(Hkv, -1, d)[:, :L].double().contiguous()
            out[b] = torch.bmm(p, Vb).reshape(Hq, d)
            del p, Vb
    return lse, out


def rate_run(dec, lse_dense, out_dense, eps, seeds, seed0):
    """(eps, delta) violations of the denominator over `seeds` decodes, the
    output-level error and the mean budget and group-union size."""
    import numpy as np
    import torch
    w_shape = tuple(dec.lse.shape)
    dev = dec.lse.device
    lse_all = torch.empty((seeds,) + w_shape, dtype=torch.float32, device=dev)
    oerr = torch.empty((seeds,) + w_shape, dtype=torch.float64, device=dev)
    nerr = torch.empty((seeds,) + w_shape, dtype=torch.float64, device=dev)
    nsum = torch.zeros(w_shape, dtype=torch.float64, device=dev)
    usum = None
    dn = out_dense.norm(dim=-1)
    live = torch.isfinite(lse_dense)
    for s in range(seeds):
        dec.set_seed(seed0 + s)
        dec()
        lse_all[s].copy_(dec.lse)
        oerr[s] = (dec.out.double() - out_dense).norm(dim=-1) / dn
        # numerator N_hat against N, both in units of the dense denominator
        ratio = torch.exp(dec.lse.double() - lse_dense)
        nerr[s] = (dec.out.double() * ratio[..., None] - out_dense).norm(dim=-1) / dn
        nsum += dec.counts[..., 3].double()
        if dec.group_counts is not None:
            g = dec.group_counts[..., 0].double()
            usum = g if usum is None else usum + g
    torch.cuda.synchronize()
    rel = (torch.exp(lse_all.double() - lse_dense) - 1.0).abs()[:, live]
    viol = int((rel > eps).sum())
    trials = int(rel.numel())
    lo, hi = clopper_pearson(viol, trials)
    e = oerr[:, live].flatten().cpu().numpy()
    ne = nerr[:, live].flatten().cpu().numpy()
    res = {"eps": eps, "rate": round(viol / trials, 5), "violations": viol, "trials": trials, "seeds": seeds,
           "cp95": [round(lo, 5), round(hi, 5)],
           "mean_budget": round(float((nsum / seeds)[live].mean()), 1),
           "output_error": {"rate_above_eps": round(float((e > eps).mean()), 5),
                            "median": round(float(np.median(e)), 5), "p99": round(float(np.quantile(e, 0.99)), 5)},
           "numerator_error": {"rate_above_eps": round(float((ne > eps).mean()), 5),
                               "median": round(float(np.median(ne)), 5)}}
    return res, (None if usum is None else usum / seeds)


def algorithmic_bytes(w, U):
    """Bytes one step must move: the predictor stream (K~ rows or signatures,
    plus the page ids) and the K and V rows of each group's union."""
    import numpy as np
    L = w.seq_lens.numpy().astype(np.float64)[:, None]
    row = w.d * w.k_cache.element_size()
    pred = w.cfg["predictor"]
    pred_row = w.cfg["rank"] * 2 if pred == 1 else 4 if pred == 2 else row
    pred_bytes = float(w.Hkv * (L[:, 0] * pred_row + np.ceil(L[:, 0] / 16) * 4).sum())
    return pred_bytes, pred_bytes + float((U * 2 * row).sum())


def workload_leg(name, mk, eps_list, steps, warm, seeds, dev):
    """Step time, HBM rate and (eps, delta) rates of one more workload."""
    import numpy as np
    import torch
    t0 = time.perf_counter()
    w = mk()
    D = Device(w, dev, 3)
    log("%s: B=%d Hq=%d Hkv=%d L<=%d (inputs %.1f s)" % (name, w.B, w.Hq, w.Hkv, w.max_seq_len,
                                                          time.perf_counter() - t0))
    lse_d, out_d = dense_reference(D)
    res = {"batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "seq_len": w.max_seq_len,
           "total_tokens": int(w.seq_lens.sum()), "heads_tokens_per_step": w.heads_tokens(),
           "eps_sweep": []}
    L = w.seq_lens.numpy().astype(np.float64)[:, None]
    for eps in (eps_list or [w.cfg["eps"]]):
        cfg = dict(w.cfg, eps=eps)
        decs = D.decoders(cfg)
        ms, per, _ = time_steps(decs, steps, warm, 0)
        gdec = D.decoders(cfg, group_counts=True, workspace=decs[0].workspace)[0]
        r, U = rate_run(gdec, lse_d, out_d, eps, seeds, 1_000_000)
        pred_b, step_b = algorithmic_bytes(w, U.cpu().numpy())
        gbs = step_b / (ms * 1e-3) / 1e9
        r.update({"ms_per_step": round(ms, 5), **step_spread(per),
                  "heads_tokens_per_s": round(w.heads_tokens() / (ms * 1e-3), 1),
                  "step_hbm": {"algorithmic_bytes": round(step_b), "achieved_GBps": round(gbs, 1),
                               "frac": round(gbs / HBM_PEAK_GBS, 4)},
                  "union_density": round(float((U.cpu().numpy() / L).mean()), 4)})
        res["eps_sweep"].append(r)
        log("%s eps=%g: %.4f ms/step (%.0f GB/s), union density %.3f, violations %d / %d = %.4f, delta %g"
            % (name, eps, ms, gbs, r["union_density"], r["violations"], r["trials"], r["rate"], w.cfg["delta"]))
        del decs, gdec
    res["delta"] = w.cfg["delta"]
    del D
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode step's (batch, KV head) groups are "
              "independent, so N GPUs would each run this same single-GPU step on their own shard; "
              "run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic
    import verified_sparse_attention_amd as vsa

    dev = torch.device("cuda:0")
    w = synthetic.WORKLOADS[args.workload]()
    G = w.Hq // w.Hkv
    d = w.d
    esize = w.k_cache.element_size()
    r = w.cfg["rank"]
    log("workload %s: B=%d Hq=%d Hkv=%d d=%d L=%d kv=%s" % (w.name, w.B, w.Hq, w.Hkv, d,
                                                            w.max_seq_len, w.k_cache.dtype))
    n_inst = 3
    D = Device(w, dev, n_inst)
    q, bt, sl, proj = D.q, D.bt, D.sl, D.proj
    k0, v0, kt0 = D.inst[0][0], D.inst[0][1], D.inst[0][2]
    decs = D.decoders()
    ws = decs[0].workspace
    pdecs = D.decoders(group_counts=True, workspace=ws)

    steps, warm = (min(args.steps, 5), min(args.warmup, 2)) if args.profile else (args.steps, args.warmup)
    if args.profile:
        # a plain device copy of known size, the last copy before the decode steps:
        # calibrates the HBM byte counters
        from verified_sparse_attention_amd import profile_summary
        cal_src = torch.empty(profile_summary.CALIBRATION_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        cal_dst = torch.empty_like(cal_src)
        cal_dst.copy_(cal_src)
        torch.cuda.synchronize()
        del cal_src, cal_dst

    # ---- timed region: exactly `steps` decode steps
    ms_per_step, per_step, t_wall = time_steps(decs, steps, warm, 0)
    heads_tokens = w.heads_tokens()
    value = heads_tokens / (ms_per_step * 1e-3)
    log("%.4f ms/step, %.4g heads*tokens/s (wall %.4f ms/step)" % (ms_per_step, value, t_wall * 1e3 / steps))

    # ---- per-kernel durations with events on the launch stream, same steps and
    # launches as the timed ones; then the same seeds once more with the group
    # counts (|U_g|, |B_g|) the byte accounting needs
    nst = vsa.NUM_STAGES
    ev = HipEvents((nst + 1) * steps)
    stage_ms = np.zeros(nst)
    gsum = torch.zeros(w.B, w.Hkv, 2, dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    for s in range(steps):
        dd = decs[s % n_inst]
        dd.set_seed(s)
        dd.profiled(ev.ev[(nst + 1) * s:(nst + 1) * (s + 1)])
    torch.cuda.synchronize()
    for s in range(steps):
        dd = pdecs[s % n_inst]
        dd.set_seed(s)
        dd()
        gsum += dd.group_counts
    torch.cuda.synchronize()
    for s in range(steps):
        for k in range(nst):
            stage_ms[k] += ev.elapsed((nst + 1) * s + k, (nst + 1) * s + k + 1)
    ev.close()
    stage_ms /= steps
    gmean = gsum.double().cpu().numpy() / steps  # mean |U_g|, |B_g| per group per step
    U = gmean[..., 0]
    Bc = gmean[..., 1]
    L = w.seq_lens.numpy().astype(np.float64)[:, None]

    # ---- algorithmic bytes per launch (mean over the timed steps)
    ncg = (w.max_seq_len + 1023) // 1024
    row = d * esize
    pred_bytes, step_bytes = algorithmic_bytes(w, U)
    base_bytes = float((Bc * row + Bc * G * 4).sum())
    # V rows of the union, K rows not scored by the base pass, cached scores,
    # chunk partials written
    gather_bytes = float((U * row + (U - Bc) * row + Bc * G * 4).sum()
                         + w.B * w.Hq * ncg * (d + 2) * 4)
    per_kernel_bytes = {"predict": pred_bytes, "base": base_bytes, "gather": gather_bytes}
    names = vsa.STAGES
    dom = int(np.argmax(stage_ms))
    dom_name = names[dom]
    # the timed step requests no index set, so its emit stage is empty (the
    # event pair alone) and is left out
    stages = {names[k]: round(float(stage_ms[k]) * 1e3, 2) for k in range(nst) if names[k] != "emit"}
    log("stage us: %s" % stages)
    log("mean |U_g| %.0f (density %.3f), |B_g| %.0f" % (U.mean(), (U / L).mean(), Bc.mean()))
    dom_bytes = per_kernel_bytes.get(dom_name)
    achieved = dom_bytes / (stage_ms[dom] * 1e-3) / 1e9 if dom_bytes else None
    kernel_frac = {}
    for k_, b_ in per_kernel_bytes.items():
        t_ = stage_ms[names.index(k_)] * 1e-3
        kernel_frac[k_] = round(b_ / t_ / 1e9 / HBM_PEAK_GBS, 4) if t_ > 0 else None

    # HBM bytes per launch from the committed counter summary, if it was taken
    # with the current kernel sources
    traffic = None
    pmc_file = os.path.join(ROOT, "profiles", "hbm_traffic_%s.json" % w.name)
    if os.path.exists(pmc_file):
        from verified_sparse_attention_amd import build as vbuild
        with open(pmc_file) as f:
            pmc = json.load(f)
        if pmc.get("source_hash") == vbuild.source_hash():
            traffic = pmc.get("kernels", {}).get("k_" + dom_name, {}).get("hbm_bytes_per_launch")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1) if achieved else None,
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
                "traffic": traffic, "kernel": "k_" + dom_name,
                "algorithmic_bytes_per_launch": round(dom_bytes) if dom_bytes else None,
                "kernel_us": round(float(stage_ms[dom]) * 1e3, 2)}
    step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9

    # ---- a plain device copy (read + write of 1 GiB): the box's practical ceiling
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(3)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 10 * 2 * src.numel() / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del dst
    # ---- a plain read of the same 1 GiB (vattn_read_probe: 16-byte
    # non-temporal loads, as the decode's streams): the ceiling of a read-only
    # stream, which a copy understates
    import verified_sparse_attention_amd as vsa
    sink = torch.zeros(vsa.READ_PROBE_SINK, dtype=torch.int32, device=dev)
    vsa.read_probe(src, sink)
    torch.cuda.synchronize()
    c0.record()
    for _ in range(10):
        vsa.read_probe(src, sink)
    c1.record()
    torch.cuda.synchronize()
    read_gbs = 10 * src.numel() / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, sink
    torch.cuda.empty_cache()
    log("device copy %.0f GB/s (read + write), read %.0f GB/s" % (copy_gbs, read_gbs))

    result = {"metric": METRIC, "value": round(value, 1), "unit": "heads·tokens/s", "n_gpus": 1,
              "steps": steps, "warmup": warm, "ms_per_step": round(ms_per_step, 5),
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
              "data": "synthetic",
              "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                         "head_dim": d, "seq_len": w.max_seq_len,
                         "kv_dtype": "bf16" if esize == 2 else "f32", "predictor_rank": r,
                         "sinks": w.cfg["sinks"], "window": w.cfg["window"],
                         "topk_ppm": w.cfg["topk_ppm"], "base_ppm": w.cfg["base_ppm"],
                         "eps": w.cfg["eps"], "delta": w.cfg["delta"],
                         "cache_copies_rotated": n_inst},
              "step_time": step_spread(per_step),
              "roofline": roofline,
              "step_hbm": {"algorithmic_bytes": round(step_bytes), "achieved_GBps": round(step_gbs, 1),
                           "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                           "union_density": round(float((U / L).mean()), 4),
                           "kernel_frac": kernel_frac},
              "copy_ceiling_GBps": round(copy_gbs, 1),
              "read_ceiling_GBps": round(read_gbs, 1),
              "stage_us": stages}

    # ---- key-side maintenance: append each sequence's newest token (K, V and
    # its low-rank key row).  Rewriting the current newest token with its own
    # values keeps the caches unchanged.
    if kt0 is not None and not args.profile:
        pos = (sl - 1).to(torch.int32)
        rows = [int(w.block_table[b, (int(w.seq_lens[b]) - 1) // 16]) for b in range(w.B)]
        pages = torch.tensor(rows, device=dev).long()
        slots = (pos.long() % 16)
        k_new = k0[pages, :, slots].contiguous()
        v_new = v0[pages, :, slots].contiguous()
        n_app = 200
        vsa.append_kv(k_new, v_new, pos, bt, k0, v0, k_lowrank=kt0, proj=proj)  # checks the arguments once
        torch.cuda.synchronize()
        lib = vsa.load()
        cargs = (C.c_void_p(k_new.data_ptr()), C.c_void_p(v_new.data_ptr()), C.c_void_p(pos.data_ptr()),
                 C.c_void_p(bt.data_ptr()), w.B, bt.shape[1], C.c_void_p(k0.data_ptr()), C.c_void_p(v0.data_ptr()),
                 C.c_void_p(kt0.data_ptr()), C.c_void_p(proj.data_ptr()), vsa.BF16 if esize == 2 else vsa.F32,
                 k0.shape[0], w.Hkv, d, r, 1 if proj.dim() == 2 else w.Hkv,
                 C.c_void_p(torch.cuda.current_stream().cuda_stream))
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(n_app):
            if lib.vattn_append_kv(*cargs) != 0:
                raise RuntimeError("vattn_append_kv failed")
        a1.record()
        torch.cuda.synchronize()
        app_us = a0.elapsed_time(a1) / n_app * 1e3
        app_bytes = w.B * w.Hkv * (4 * d * esize + r * 2)
        result["key_append"] = {"us": round(app_us, 2), "algorithmic_bytes": app_bytes,
                                "note": "one new token per sequence: K, V and its low-rank key row"}
        log("append %.2f us per call" % app_us)

    # ---- calibration, not part of the decode step: the keys' Gram matrices per
    # KV head (the second moments a per-head predictor basis is taken from), a
    # dense contraction over every cached token on the matrix cores
    if k0.dtype == torch.bfloat16 and not args.profile:
        gram = vsa.key_gram(k0, bt, sl, w.max_seq_len)
        gws = torch.empty(int(vsa.load().vattn_key_gram_workspace_size(w.B, w.Hkv, d, w.max_seq_len)) + 256,
                          dtype=torch.uint8, device=dev)
        vsa.key_gram(k0, bt, sl, w.max_seq_len, gram=gram, workspace=gws)
        torch.cuda.synchronize()
        n_g = 20
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(n_g):
            vsa.key_gram(k0, bt, sl, w.max_seq_len, gram=gram, workspace=gws)
        g1.record()
        torch.cuda.synchronize()
        g_us = g0.elapsed_time(g1) / n_g * 1e3
        tokens = int(w.seq_lens.sum())
        g_bytes = tokens * w.Hkv * d * esize
        g_flops = 2 * tokens * w.Hkv * d * d
        result["key_gram"] = {"us": round(g_us, 1), "bytes": g_bytes, "GBps": round(g_bytes / g_us / 1e3, 1),
                              "TFLOPs": round(g_flops / g_us / 1e6, 1),
                              "note": "calibration of per-KV-head predictor bases, not part of the decode step"}
        log("key gram %.1f us (%.0f GB/s)" % (g_us, g_bytes / g_us / 1e3))
        del gram, gws

    if not args.no_legs and not args.profile and args.workload == "llama8b_32k":
        # ---- host-resident K/V: the caches in pinned, device-mapped host memory,
        # read by the kernels over the host link (the low-rank keys and the
        # workspace stay in HBM).  Compared with moving the whole K/V over the
        # same link, measured as a plain host-to-device copy.  The first two
        # sequences of the workload (a launch of its own, so a kernel trace
        # tells these steps from the headline's).
        hw = synthetic.WORKLOADS[args.workload](B=2)
        hD = Device(hw, dev, 1)
        kh = hw.k_cache.pin_memory()
        vh = hw.v_cache.pin_memory()
        rt = C.CDLL("libamdhip64.so.7")
        rt.hipHostGetDevicePointer.argtypes = [C.POINTER(C.c_void_p), C.c_void_p, C.c_uint]
        for t_ in (kh, vh):  # the kernels read the host addresses: the device must map them alike
            a_ = C.c_void_p()
            if rt.hipHostGetDevicePointer(C.byref(a_), C.c_void_p(t_.data_ptr()), 0) != 0 or a_.value != t_.data_ptr():
                raise RuntimeError("pinned host memory is not mapped at the same device address")
        hdec = vsa.Decoder(hD.q, kh, vh, hD.bt, hD.sl, vsa.Config.from_dict(hw.cfg), max_seq_len=hw.max_seq_len,
                           k_lowrank=hD.inst[0][2], proj=hD.proj, workspace=ws, want_group_counts=True)
        hdec.set_seed(7)
        hdec()
        torch.cuda.synchronize()
        hU = hdec.group_counts[..., 0].double().cpu().numpy()
        n_h = 5
        h0, h1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        h0.record()
        for s in range(n_h):
            hdec.set_seed(s)
            hdec()
        h1.record()
        torch.cuda.synchronize()
        host_ms = h0.elapsed_time(h1) / n_h
        kv_bytes = 2 * hw.k_cache.numel() * esize
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dst = torch.empty_like(hD.inst[0][1])
        dst.copy_(vh, non_blocking=True)
        torch.cuda.synchronize()
        c0.record()
        for _ in range(3):
            dst.copy_(vh, non_blocking=True)
        c1.record()
        torch.cuda.synchronize()
        link_gbs = 3 * vh.numel() * esize / (c0.elapsed_time(c1) * 1e-3) / 1e9
        dense_ms = kv_bytes / (link_gbs * 1e9) * 1e3
        union_bytes = float((hU * 2 * row).sum())
        result["host_kv"] = {
            "batch": hw.B, "ms_per_step": round(host_ms, 3),
            "value": round(hw.heads_tokens() / (host_ms * 1e-3), 1),
            "unit": "heads·tokens/s", "link_copy_GBps": round(link_gbs, 1),
            "kv_bytes_over_link": round(union_bytes), "dense_kv_bytes": kv_bytes,
            "dense_kv_transfer_ms": round(dense_ms, 3), "speedup_vs_dense_transfer": round(dense_ms / host_ms, 2),
            "note": "the first %d sequences of the workload with K/V in pinned host memory read in place by the "
                    "kernels (low-rank keys in HBM), against moving the whole K/V over the same link" % hw.B}
        log("host-resident KV (B=%d): %.3f ms/step, link %.1f GB/s, dense K/V transfer %.3f ms"
            % (hw.B, host_ms, link_gbs, dense_ms))
        del hdec, kh, vh, dst, hD

    if args.layout_leg and not args.profile and args.workload == "llama8b_32k":
        # ---- the same workload with a globally shuffled block table: the same
        # tokens in pages scattered over the cache, so only the physical
        # layout differs (and the results must not)
        sw = synthetic.repaged(w, seed=5)
        sD = Device(sw, dev, n_inst)
        sdecs = sD.decoders(workspace=ws)
        s_ms, s_per, _ = time_steps(sdecs, steps, warm, 0)
        sev = HipEvents((nst + 1) * steps)
        for s_ in range(steps):
            sdecs[s_ % n_inst].set_seed(s_)
            sdecs[s_ % n_inst].profiled(sev.ev[(nst + 1) * s_:(nst + 1) * (s_ + 1)])
        torch.cuda.synchronize()
        s_stage = np.zeros(nst)
        for s_ in range(steps):
            for k_ in range(nst):
                s_stage[k_] += sev.elapsed((nst + 1) * s_ + k_, (nst + 1) * s_ + k_ + 1)
        sev.close()
        s_stage /= steps
        same = []
        for dd_ in (decs[0], sdecs[0]):
            dd_.set_seed(11)
            dd_()
            torch.cuda.synchronize()
            same.append((dd_.out.clone(), dd_.lse.clone()))
        identical = bool(torch.equal(same[0][0], same[1][0]) and torch.equal(same[0][1], same[1][1]))
        result["shuffled_pages"] = {
            "ms_per_step": round(s_ms, 5), "value": round(sw.heads_tokens() / (s_ms * 1e-3), 1),
            "unit": "heads·tokens/s", "step_time": step_spread(s_per), "outputs_identical": identical,
            "stage_us": {names[k_]: round(float(s_stage[k_]) * 1e3, 2) for k_ in range(nst) if names[k_] != "emit"},
            "note": "the headline workload with its pages in a globally permuted block table"}
        log("shuffled block table: %.4f ms/step, outputs identical to the identity layout: %s; stage us %s"
            % (s_ms, identical, result["shuffled_pages"]["stage_us"]))
        del sdecs, sD, same

    if not args.profile:
        # ---- (eps, delta): denominator relative error against dense fp64 attention
        lse_dense, out_dense = dense_reference(D)
        er, _ = rate_run(decs[0], lse_dense, out_dense, w.cfg["eps"], args.rate_seeds, 1_000_000)
        result["eps_violation"] = {k_: er[k_] for k_ in ("rate", "violations", "trials", "seeds", "cp95")}
        result["eps_violation"]["mean_budget"] = er["mean_budget"]
        result["eps_violation"].update({"delta": w.cfg["delta"], "reference": "dense attention in fp64"})
        result["output_error"] = dict(er["output_error"], note="the budget bounds the denominator only; "
                                      "this is the measured relative L2 error of the outputs against dense fp64")
        log("eps violations %d / %d = %.4f (95%% CI %s); output rel. error median %.4f"
            % (er["violations"], er["trials"], er["rate"], er["cp95"], er["output_error"]["median"]))

        # ---- the other long-context workloads: throughput, HBM rate and the
        # (eps, delta) rate at full size (the 70B-shaped one over an eps sweep)
        if not args.no_configs and args.workload == "llama8b_32k":
            result["workloads"] = {}
            legs = [("flat_128k", synthetic.flat_128k, None), ("ragged_b64", synthetic.ragged_b64, None),
                    ("wide_gqa_64k", synthetic.wide_gqa_64k, [0.01, 0.02, 0.05, 0.1])]
            for name, mk, eps_list in legs:
                result["workloads"][name] = workload_leg(name, mk, eps_list, max(10, steps // 2), warm,
                                                         args.rate_seeds, dev)
        # ---- the base-sample rate: 5, 10, 20% of the tail
        for name in [x for x in args.base_sweep.split(",") if x]:
            sweep = []
            for bp in (50000, 100000, 200000):
                mk = synthetic.WORKLOADS[name]
                res = workload_leg("%s base %d%%" % (name, bp // 10000), lambda mk=mk, bp=bp: mk(base_ppm=bp),
                                   None, 20, warm, args.rate_seeds, dev)
                sweep.append(dict(res["eps_sweep"][0], base_ppm=bp))
            result.setdefault("base_sweep", {})[name] = sweep

        # ---- the same workload with a per-KV-head PCA predictor basis (the r
        # leading eigenvectors of each head's key Gram matrix over the first half
        # of every sequence, as a basis fitted at prefill; host eigensolve).
        # Context only; the headline value above uses the workload's random basis.
        if args.pca_basis and kt0 is not None and k0.dtype == torch.bfloat16:
            gram = vsa.key_gram(k0, bt, (sl // 2).contiguous(), w.max_seq_len)
            _, evec = torch.linalg.eigh(gram.double().cpu())
            p_pca = evec[:, :, -r:].flip(-1).float().contiguous().to(dev)  # [Hkv, d, r], descending
            pca_decs = []
            for (k, v, _, _) in D.inst:
                pca_decs.append(vsa.Decoder(q, k, v, bt, sl, vsa.Config.from_dict(w.cfg), max_seq_len=w.max_seq_len,
                                            k_lowrank=vsa.project_keys(k, p_pca), proj=p_pca,
                                            want_group_counts=True, workspace=ws))
            pca_ms, pper, _ = time_steps(pca_decs, steps, warm, 30_000)
            pr, Up = rate_run(pca_decs[0], lse_dense, out_dense, w.cfg["eps"], args.rate_seeds, 1_000_000)
            result["pca_basis"] = {
                "ms_per_step": round(pca_ms, 5), "value": round(heads_tokens / (pca_ms * 1e-3), 1),
                "unit": "heads·tokens/s", "union_density": round(float((Up.cpu().numpy() / L).mean()), 4),
                "eps_violation": {k_: pr[k_] for k_ in ("rate", "violations", "trials", "seeds", "cp95")},
                "output_error": pr["output_error"],
                "note": "same workload with a per-KV-head basis: the %d leading eigenvectors of vattn_key_gram "
                        "over the first half of each sequence (a Loki-style basis fitted at prefill)" % r}
            log("pca basis: %.4f ms/step, eps violations %d / %d" % (pca_ms, pr["violations"], pr["trials"]))
            del pca_decs

        # ---- the same workload with the hash-signature predictor (32 sign
        # bits per key under the workload's random directions, 4 bytes per
        # token instead of a rank-r row).  Context only.
        if not args.no_legs and proj is not None and r == 32:
            hcfg = vsa.Config.from_dict(dict(w.cfg, predictor=vsa.PRED_HASH, rank=32))
            hdecs = [vsa.Decoder(q, k, v, bt, sl, hcfg, max_seq_len=w.max_seq_len, proj=proj,
                                 k_sig=vsa.sign_keys(k, proj), want_group_counts=True, workspace=ws)
                     for (k, v, _, _) in D.inst]
            hash_ms, hper, _ = time_steps(hdecs, steps, warm, 50_000)
            hev = HipEvents((nst + 1) * steps)
            hst = np.zeros(nst)
            for s in range(steps):
                hdecs[s % n_inst].set_seed(50_000 + s)
                hdecs[s % n_inst].profiled(hev.ev[(nst + 1) * s:(nst + 1) * (s + 1)])
            torch.cuda.synchronize()
            for s in range(steps):
                for k in range(nst):
                    hst[k] += hev.elapsed((nst + 1) * s + k, (nst + 1) * s + k + 1)
            hev.close()
            hst /= steps
            hr, Uh = rate_run(hdecs[0], lse_dense, out_dense, w.cfg["eps"], args.rate_seeds, 2_000_000)
            hpred_bytes = float(w.Hkv * (L[:, 0] * 4 + np.ceil(L[:, 0] / 16) * 4).sum())
            result["hash_predictor"] = {
                "ms_per_step": round(hash_ms, 5), "value": round(heads_tokens / (hash_ms * 1e-3), 1),
                "unit": "heads·tokens/s", "union_density": round(float((Uh.cpu().numpy() / L).mean()), 4),
                "stage_us": {names[k]: round(float(hst[k]) * 1e3, 2) for k in range(nst) if names[k] != "emit"},
                "predict_bytes": hpred_bytes,
                "eps_violation": {k_: hr[k_] for k_ in ("rate", "violations", "trials", "seeds", "cp95")},
                "output_error": hr["output_error"],
                "note": "same workload, top-k from 32-bit random-hyperplane key signatures "
                        "(vattn_sign_keys) scored by shared bits"}
            log("hash predictor: %.4f ms/step, eps violations %d / %d" % (hash_ms, hr["violations"], hr["trials"]))
            del hdecs

    if not args.profile and not args.no_legs and args.workload == "llama8b_32k":
        # ---- the output-level guarantee (numerator and denominator) against the
        # denominator-only budget: union density, budget, step time, the
        # denominator and numerator (eps, delta) rates and the output error.  On
        # the tiny workload as stated (zero-mean values) and with values of a
        # shared direction, and on the 32K workload with such values.
        legs = [("tiny_1k", lambda: synthetic.tiny(), 1000),
                ("tiny_1k_value_mean_3", lambda: synthetic.tiny(v_mean=3.0), 1000),
                ("llama8b_32k_value_mean_3", lambda: synthetic.WORKLOADS[args.workload](v_mean=3.0),
                 max(100, args.rate_seeds // 5))]
        og = {}
        for name, mk, seeds in legs:
            ow = mk()
            oD = Device(ow, dev, 1)
            lse_o, out_o = dense_reference(oD)
            Lo = ow.seq_lens.numpy().astype(np.float64)[:, None]
            og[name] = {"seeds": seeds}
            for gname, gval in (("denominator", 0), ("output", 1)):
                od = oD.decoders(dict(ow.cfg, guarantee=gval), group_counts=True)[0]
                oms, _, _ = time_steps([od], 20, 3, 70_000)
                res_o, Uo = rate_run(od, lse_o, out_o, ow.cfg["eps"], seeds, 3_000_000)
                og[name][gname] = {
                    "ms_per_step": round(oms, 5), "union_density": round(float((Uo.cpu().numpy() / Lo).mean()), 4),
                    "mean_budget": res_o["mean_budget"],
                    "denominator_violation": {"rate": res_o["rate"], "cp95": res_o["cp95"]},
                    "numerator_error": res_o["numerator_error"], "output_error": res_o["output_error"]}
                log("%s %s: %.4f ms/step, density %.3f, denominator viol %.4f, numerator above eps %.4f, "
                    "output above eps %.4f" % (name, gname, oms, og[name][gname]["union_density"], res_o["rate"],
                                               res_o["numerator_error"]["rate_above_eps"],
                                               res_o["output_error"]["rate_above_eps"]))
                del od
            og[name]["eps"] = ow.cfg["eps"]
            del oD
        og["note"] = ("guarantee=1 holds the numerator sum_i w_i e^{s_i} V_i to the same CLT bound as the "
                      "denominator and takes the larger budget; numerator_error is |N_hat - N| / |N|")
        result["output_guarantee"] = og
        torch.cuda.empty_cache()

    if not args.profile and not args.no_cpu_baseline:
        import oracle
        cores = min(len(os.sched_getaffinity(0)), HOST_CORE_CAP)
        model = "unknown"
        try:
            with open("/proc/cpuinfo") as f:
                model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
        except OSError:
            pass
        arrays = w.oracle_arrays()
        cpu_cfg = dict(w.cfg, seed=0)
        t = time.perf_counter()
        oracle.decode(**arrays, cfg=cpu_cfg, nthreads=cores, want_idx=False)
        dt = time.perf_counter() - t
        # single thread on a sample of the groups (the per-group work is uniform here)
        n1 = 4
        grp = [(b, g) for b in range(w.B) for g in range(w.Hkv)][:n1]
        t = time.perf_counter()
        oracle.decode(**arrays, cfg=cpu_cfg, nthreads=1, want_idx=False, groups=grp)
        dt1 = (time.perf_counter() - t) * (w.B * w.Hkv) / n1
        result["cpu_baseline"] = {"value": round(heads_tokens / dt, 1), "unit": "heads·tokens/s",
                                  "cores": cores, "kind": "oracle",
                                  "sample": "one full decode step of %s (all %d (batch, KV head) groups, seed 0), "
                                            "%.2f s wall on %d threads (the host's affinity set, capped at %d, "
                                            "the CPU share of one GPU)" % (w.name, w.B * w.Hkv, dt, cores,
                                                                           HOST_CORE_CAP),
                                  "cpu_model": model, "host_threads_available": len(os.sched_getaffinity(0)),
                                  "single_thread": {"value": round(heads_tokens / dt1, 1),
                                                    "sample": "%d of %d groups on one thread, %.2f s, scaled to "
                                                              "the whole step" % (n1, w.B * w.Hkv, dt1 * n1 /
                                                                                  (w.B * w.Hkv))}}
        log("cpu oracle %.2f s on %d threads, %.2f s on one (%s)" % (dt, cores, dt1, model))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
