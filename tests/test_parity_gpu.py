"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Index sets, counts and fixed-point statistics must be bit-identical; out and
lse within max-abs 1e-5 (fp32 KV) or 2e-3 (bf16 KV).  Small cases span several
predictor chunks, gather chunks and ragged tails; the full-size workloads run in
the benchmark's launch configuration and are compared on sampled (b, KV head)
groups that the oracle evaluates one by one.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synthetic

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3}


def _gpu():
    from tests.gpu_run import GpuCase, log
    return GpuCase, log


def compare(w, g, o, groups=None, tag=""):
    """Bit-exact discrete outputs, tolerance on out/lse, for the given groups."""
    G = w.Hq // w.Hkv
    tol = TOL["bf16" if w.k_cache.dtype.is_floating_point and w.k_cache.element_size() == 2 else "f32"]
    assert g["z32"] == o["z32"]
    if groups is None:
        groups = [(b, kv) for b in range(w.B) for kv in range(w.Hkv)]
    for (b, kv) in groups:
        for h in range(kv * G, (kv + 1) * G):
            ctx = "%s b=%d h=%d" % (tag, b, h)
            assert np.array_equal(g["counts"][b, h], o["counts"][b, h]), \
                (ctx, g["counts"][b, h], o["counts"][b, h])
            assert np.array_equal(g["stats"][b, h], o["stats"][b, h]), (ctx, g["stats"][b, h], o["stats"][b, h])
            if "num_stats" in g:  # output-level mode: fp64 sums in one order on both sides
                assert np.array_equal(g["num_stats"][b, h], o["num_stats"][b, h]), \
                    (ctx, g["num_stats"][b, h], o["num_stats"][b, h])
            if "idx" in g and "idx" in o:
                assert np.array_equal(g["idx"][b, h], o["idx"][b, h]), ctx
            L = int(w.seq_lens[b])
            if L == 0:
                assert np.all(g["out"][b, h] == 0) and np.isneginf(g["lse"][b, h]), ctx
                continue
            err_o = np.max(np.abs(g["out"][b, h].astype(np.float64) - o["out"][b, h]))
            err_l = abs(float(g["lse"][b, h]) - o["lse"][b, h])
            assert err_o <= tol and err_l <= tol, (ctx, err_o, err_l)
        # the group's union of index sets, counted by the gather blocks of every
        # chunk (atomics from blocks spread over all the device's dies)
        if "gcounts" in g and "idx" in o:
            sets = [o["idx"][b, h][o["idx"][b, h] >= 0] for h in range(kv * G, (kv + 1) * G)]
            nu = np.unique(np.concatenate(sets)).size
            assert int(g["gcounts"][b, kv, 0]) == nu, (tag, b, kv, int(g["gcounts"][b, kv, 0]), nu)


def run_both(w, seeds=(None,), groups=None, want_idx=True, tag=""):
    GpuCase, log = _gpu()
    log("[parity] %s %s B=%d Hq=%d Hkv=%d d=%d L=%s" % (tag, w.name, w.B, w.Hq, w.Hkv, w.d,
                                                       list(w.seq_lens.tolist())[:8]))
    case = GpuCase(w, want_idx=want_idx)
    arrays = w.oracle_arrays()
    for s in seeds:
        cfg = dict(w.cfg)
        if s is not None:
            cfg["seed"] = s
        g = case.run(cfg["seed"])
        o = oracle.decode(**arrays, cfg=cfg, groups=groups, want_idx=want_idx, nthreads=8)
        compare(w, g, o, groups, tag="%s seed=%s" % (tag, cfg["seed"]))
    return case


SMALL_CASES = {
    "gqa4_bf16_ragged": lambda: synthetic.make(
        name="gqa4_bf16_ragged", B=3, Hq=16, Hkv=4, d=128, seq_lens=(5000, 2500, 777),
        kv_dtype="bf16", recipe="outlier", predictor=1, rank=32, sinks=32, window=64,
        topk_ppm=25000, shuffle=True, data_seed=11),
    "gqa8_lowrank_3chunks": lambda: synthetic.make(
        name="gqa8_lowrank_3chunks", B=2, Hq=16, Hkv=2, d=128, seq_lens=(9000, 4100),
        kv_dtype="bf16", recipe="lowrank", predictor=1, rank=32, sinks=128, window=128,
        topk_ppm=25000, eps=0.02, data_seed=12),
    "gqa2_d64_f32_r16": lambda: synthetic.make(
        name="gqa2_d64_f32_r16", B=2, Hq=4, Hkv=2, d=64, seq_lens=(3000, 1500), kv_dtype="f32",
        recipe="planted", predictor=1, rank=16, sinks=8, window=16, topk_ppm=20000, data_seed=13),
    "exact_bf16_d128_g2": lambda: synthetic.make(
        name="exact_bf16_d128_g2", B=1, Hq=4, Hkv=2, d=128, seq_lens=(2000,), kv_dtype="bf16",
        recipe="planted", predictor=0, sinks=16, window=16, topk_abs=40, data_seed=14),
    "r64_g1_2chunks": lambda: synthetic.make(
        name="r64_g1_2chunks", B=1, Hq=2, Hkv=2, d=128, seq_lens=(33000,), kv_dtype="bf16",
        recipe="outlier", predictor=1, rank=64, sinks=64, window=64, topk_ppm=25000,
        data_seed=15),
    "flat_small": lambda: synthetic.make(
        name="flat_small", B=1, Hq=8, Hkv=2, d=128, seq_lens=(6000,), kv_dtype="bf16",
        recipe="flat", q_std=0.3, k_std=0.3, predictor=1, rank=32, sinks=128, window=128,
        topk_ppm=10000, eps=0.02, data_seed=16),
    "flat_crowded_bucket": lambda: synthetic.make(
        name="flat_crowded_bucket", B=1, Hq=8, Hkv=2, d=128, seq_lens=(20000,), kv_dtype="bf16",
        recipe="flat", q_std=0.3, k_std=0.3, predictor=1, rank=32, sinks=16, window=16,
        topk_ppm=25000, eps=0.02, data_seed=18),
    # one sequence, few heads, 20 predictor chunks: the chunk candidates are
    # pre-merged in 8 uneven parts before the per-head select
    "premerge_parts": lambda: synthetic.make(
        name="premerge_parts", B=1, Hq=4, Hkv=1, d=128, seq_lens=(40000,), kv_dtype="bf16",
        recipe="outlier", predictor=1, rank=32, sinks=64, window=64, topk_ppm=25000, data_seed=19),
    # one predictor basis per KV head (4 groups, each with its own P_g)
    "per_head_bases": lambda: synthetic.make(
        name="per_head_bases", B=2, Hq=16, Hkv=4, d=128, seq_lens=(5000, 2100), kv_dtype="bf16",
        recipe="outlier", predictor=1, rank=32, sinks=32, window=64, topk_ppm=25000,
        proj_per_head=True, data_seed=20),
    # per-head bases with G = 8 and the pre-merge (one 40K sequence, 16 heads)
    "per_head_g8_premerge": lambda: synthetic.make(
        name="per_head_g8_premerge", B=1, Hq=16, Hkv=2, d=128, seq_lens=(40000,), kv_dtype="bf16",
        recipe="lowrank", predictor=1, rank=32, sinks=64, window=64, topk_ppm=20000,
        proj_per_head=True, data_seed=21),
    # kernel instances the cases above leave out: d = 64 with bf16 and G = 8,
    # fp32 at d = 128 with G = 8 (exact predictor) and G = 4 (low rank), and a
    # rank equal to the head dim
    "d64_bf16_g8": lambda: synthetic.make(
        name="d64_bf16_g8", B=2, Hq=16, Hkv=2, d=64, seq_lens=(3000, 1700), kv_dtype="bf16",
        recipe="outlier", predictor=1, rank=16, sinks=16, window=32, topk_ppm=25000, data_seed=22),
    "d128_f32_g8_exact": lambda: synthetic.make(
        name="d128_f32_g8_exact", B=1, Hq=8, Hkv=1, d=128, seq_lens=(2500,), kv_dtype="f32",
        recipe="planted", predictor=0, sinks=8, window=16, topk_abs=50, data_seed=23),
    "d128_f32_g4_lowrank": lambda: synthetic.make(
        name="d128_f32_g4_lowrank", B=2, Hq=8, Hkv=2, d=128, seq_lens=(3100, 900), kv_dtype="f32",
        recipe="outlier", predictor=1, rank=32, sinks=16, window=16, topk_ppm=25000, data_seed=24),
    "d64_bf16_rank_eq_d": lambda: synthetic.make(
        name="d64_bf16_rank_eq_d", B=1, Hq=2, Hkv=2, d=64, seq_lens=(4000,), kv_dtype="bf16",
        recipe="normal", predictor=1, rank=64, sinks=8, window=8, topk_ppm=20000, data_seed=25),
    # the hash-signature predictor: 32-bit key signatures, scores 0..32 with
    # many ties (ranked by index), every group size, both dtypes and head
    # dims, one hyperplane set per KV head, and the pre-merge path
    "hash_g4_bf16_ragged": lambda: synthetic.make(
        name="hash_g4_bf16_ragged", B=3, Hq=16, Hkv=4, d=128, seq_lens=(5000, 2500, 777),
        kv_dtype="bf16", recipe="outlier", predictor=2, rank=32, sinks=32, window=64,
        topk_ppm=25000, shuffle=True, data_seed=40),
    "hash_g8_per_head_premerge": lambda: synthetic.make(
        name="hash_g8_per_head_premerge", B=1, Hq=16, Hkv=2, d=128, seq_lens=(40000,), kv_dtype="bf16",
        recipe="planted", predictor=2, rank=32, sinks=64, window=64, topk_ppm=20000,
        proj_per_head=True, data_seed=41),
    "hash_d64_f32_g2": lambda: synthetic.make(
        name="hash_d64_f32_g2", B=2, Hq=4, Hkv=2, d=64, seq_lens=(3000, 1500), kv_dtype="f32",
        recipe="planted", predictor=2, rank=32, sinks=8, window=16, topk_ppm=20000, data_seed=42),
    "hash_g1_d64_bf16": lambda: synthetic.make(
        name="hash_g1_d64_bf16", B=2, Hq=2, Hkv=2, d=64, seq_lens=(9000, 33), kv_dtype="bf16",
        recipe="normal", predictor=2, rank=32, sinks=8, window=8, topk_ppm=25000, data_seed=43),
    "mixed_ragged_shuffled": lambda: synthetic.make(
        name="mixed_ragged_shuffled", B=4, Hq=8, Hkv=2, d=128, seq_lens=(1100, 3333, 2048, 1500),
        kv_dtype="bf16", recipe="mixed", predictor=1, rank=32, sinks=64, window=64,
        topk_ppm=20000, eps=0.05, delta=0.1, shuffle=True, data_seed=17),
}


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_parity_small(name):
    run_both(SMALL_CASES[name](), seeds=(0, 1, 977), tag=name)


def test_parity_tiny_1000_seeds():
    w = synthetic.tiny()
    GpuCase, log = _gpu()
    log("[parity] tiny_1k x 1000 seeds")
    case = GpuCase(w)
    arrays = w.oracle_arrays()
    for s in range(1000):
        cfg = dict(w.cfg, seed=s)
        g = case.run(s)
        o = oracle.decode(**arrays, cfg=cfg)
        compare(w, g, o, tag="tiny seed=%d" % s)


EDGE_CASES = {
    "empty_one_short_seqs": lambda: synthetic.make(
        B=4, Hq=2, Hkv=1, d=64, seq_lens=(0, 1, 20, 50), kv_dtype="f32", predictor=0, sinks=2,
        window=2, topk_abs=4),
    "tail_1_and_2": lambda: synthetic.make(
        B=2, Hq=2, Hkv=1, d=64, seq_lens=(13, 14), kv_dtype="f32", predictor=0, sinks=2,
        window=2, topk_abs=8),
    "k_covers_middle": lambda: synthetic.make(
        B=1, Hq=2, Hkv=1, d=64, seq_lens=(300,), kv_dtype="bf16", predictor=0, sinks=2, window=2,
        topk_abs=1000),
    "pure_sampling": lambda: synthetic.make(
        B=1, Hq=4, Hkv=2, d=128, seq_lens=(3000,), kv_dtype="bf16", recipe="flat", q_std=0.3,
        k_std=0.3, predictor=1, rank=32, sinks=0, window=0, topk_abs=0),
    "forced_full": lambda: synthetic.make(
        B=2, Hq=4, Hkv=2, d=128, seq_lens=(2000, 1234), kv_dtype="bf16", recipe="outlier",
        predictor=1, rank=32, sinks=16, window=16, force_budget=10 ** 9),
    "forced_small": lambda: synthetic.make(
        B=1, Hq=4, Hkv=1, d=64, seq_lens=(1500,), kv_dtype="f32", predictor=0, sinks=4, window=4,
        topk_abs=16, force_budget=7),
    "forced_zero": lambda: synthetic.make(
        B=1, Hq=2, Hkv=1, d=64, seq_lens=(700,), kv_dtype="f32", predictor=0, sinks=4, window=4,
        topk_abs=16, force_budget=0),
    "tiny_eps_dense": lambda: synthetic.make(
        B=1, Hq=4, Hkv=1, d=128, seq_lens=(2500,), kv_dtype="bf16", recipe="outlier", predictor=1,
        rank=32, sinks=8, window=8, eps=1e-4),
    "base_ppm_max": lambda: synthetic.make(
        B=1, Hq=2, Hkv=2, d=64, seq_lens=(900,), kv_dtype="f32", predictor=0, sinks=4, window=4,
        topk_abs=10, base_ppm=1000000),
    # keys outside the predictor's span with scaled scores of 40 against ~4 for
    # the fixed set and a 2-token base sample: every chunk holding one takes
    # its weights against its own maximum (the rescale fallback), through the
    # K rows and, for the key in head 1's top-k, through the cached scores
    "hidden_rescale": lambda: synthetic.make(
        name="hidden_rescale", B=2, Hq=4, Hkv=2, d=128, seq_lens=(3000, 2100), kv_dtype="bf16",
        recipe="hidden", predictor=1, rank=32, sinks=4, window=4, topk_abs=4, base_ppm=1,
        force_budget=10 ** 9, data_seed=31),
    # pre-merged parts with fewer candidates than k (kept whole) and more
    "premerge_keep_all": lambda: synthetic.make(
        name="premerge_keep_all", B=1, Hq=2, Hkv=1, d=64, seq_lens=(36000,), kv_dtype="f32",
        predictor=0, sinks=8, window=8, topk_abs=5000, data_seed=20),
    "page_unaligned_regions": lambda: synthetic.make(
        B=2, Hq=8, Hkv=1, d=128, seq_lens=(1037, 4099), kv_dtype="bf16", recipe="planted",
        predictor=1, rank=32, sinks=5, window=27, topk_abs=33, shuffle=True),
}


@pytest.mark.parametrize("name", list(EDGE_CASES))
def test_parity_edge_cases(name):
    run_both(EDGE_CASES[name](), seeds=(0, 5), tag=name)


@pytest.mark.parametrize("name", ["gqa4_bf16_ragged", "gqa2_d64_f32_r16", "exact_bf16_d128_g2"])
def test_parity_host_kv(name):
    """K and V in pinned host memory, read by the kernels over the host link
    (the low-rank keys stay in HBM): the same results as the oracle."""
    w = SMALL_CASES[name]()
    GpuCase, log = _gpu()
    log("[parity] host-resident KV %s" % name)
    case = GpuCase(w, kv_host=True)
    assert not case.k.is_cuda and case.k.is_pinned() and case.v.is_pinned()
    arrays = w.oracle_arrays()
    for s in (0, 4):
        g = case.run(s)
        o = oracle.decode(**arrays, cfg=dict(w.cfg, seed=s), want_idx=True, nthreads=8)
        compare(w, g, o, tag="%s host kv seed=%d" % (name, s))


def test_full_budget_matches_dense():
    w = EDGE_CASES["forced_full"]()
    GpuCase, log = _gpu()
    log("[parity] forced_full vs dense")
    g = GpuCase(w).run()
    o = oracle.decode(**w.oracle_arrays(), cfg=w.cfg, want_dense=True)
    assert np.max(np.abs(g["out"] - o["out_dense"])) <= 2e-3
    assert np.max(np.abs(g["lse"] - o["lse_dense"])) <= 2e-3


def test_project_keys_bit_exact():
    import torch
    import verified_sparse_attention_amd as vsa
    _, log = _gpu()
    for (d, r, dt) in ((128, 32, torch.bfloat16), (64, 16, torch.float32), (128, 64, torch.bfloat16),
                       (64, 32, torch.float32), (128, 16, torch.float32)):
        log("[parity] project_keys d=%d r=%d %s" % (d, r, dt))
        gen = torch.Generator().manual_seed(d * 1000 + r)
        k = (torch.randn(37, 3, 16, d, generator=gen) * 2.0).to(dt)
        P = synthetic.orthonormal(d, r, gen)
        kt = vsa.project_keys(k.cuda(), P.cuda()).cpu().numpy().view(np.uint16)
        rows = k.float().reshape(-1, d).numpy()
        want = oracle.project_rows(rows, P.numpy()).reshape(kt.shape)
        assert np.array_equal(kt, want)
    # one basis per KV head: head g's rows use P_g
    for (d, r, dt) in ((128, 32, torch.bfloat16), (64, 16, torch.float32), (128, 64, torch.bfloat16)):
        log("[parity] project_keys per head d=%d r=%d %s" % (d, r, dt))
        gen = torch.Generator().manual_seed(d * 3000 + r)
        k = (torch.randn(29, 4, 16, d, generator=gen) * 2.0).to(dt)
        Ph = torch.stack([synthetic.orthonormal(d, r, gen) for _ in range(4)])
        kt = vsa.project_keys(k.cuda(), Ph.cuda()).cpu().numpy().view(np.uint16)
        for g in range(4):
            rows = k[:, g].float().reshape(-1, d).numpy()
            want = oracle.project_rows(rows, Ph[g].numpy()).reshape(kt[:, g].shape)
            assert np.array_equal(kt[:, g], want), g


def test_sign_keys_bit_exact():
    import torch
    import verified_sparse_attention_amd as vsa
    _, log = _gpu()
    for (d, dt, per_head) in ((128, torch.bfloat16, False), (64, torch.float32, False),
                              (128, torch.float32, True), (64, torch.bfloat16, True)):
        log("[parity] sign_keys d=%d %s per_head=%s" % (d, dt, per_head))
        gen = torch.Generator().manual_seed(d * 5000 + int(per_head))
        Hkv = 3
        k = (torch.randn(37, Hkv, 16, d, generator=gen) * 2.0).to(dt)
        k[0, 0, 0] = 0.0  # a zero key: no bit set
        P = (torch.stack([synthetic.orthonormal(d, 32, gen) for _ in range(Hkv)]) if per_head
             else synthetic.orthonormal(d, 32, gen))
        ks = vsa.sign_keys(k.cuda(), P.cuda()).cpu().numpy().view(np.uint32)
        assert ks.shape == (37, Hkv, 16)
        for g in range(Hkv):
            rows = k[:, g].float().reshape(-1, d).numpy()
            want = oracle.sign_rows(rows, (P[g] if per_head else P).numpy()).reshape(37, 16)
            assert np.array_equal(ks[:, g], want), g
        assert ks[0, 0, 0] == 0


def test_append_kv_sig_bit_exact():
    """The newest token's K and V rows land at their page slot and its
    signature equals the oracle's; every other word is untouched."""
    import torch
    import verified_sparse_attention_amd as vsa
    _, log = _gpu()
    for (d, dt, per_head) in ((128, torch.bfloat16, False), (64, torch.float32, True)):
        log("[parity] append_kv_sig d=%d %s per_head=%s" % (d, dt, per_head))
        gen = torch.Generator().manual_seed(9000 + d)
        B, Hkv, max_blocks = 5, 3, 6
        nb = B * max_blocks + 4
        bt = torch.randperm(nb, generator=gen)[:B * max_blocks].reshape(B, max_blocks).to(torch.int32)
        pos = torch.tensor([0, 17, 95, -1, 40], dtype=torch.int32)
        k_cache = torch.randn(nb, Hkv, 16, d, generator=gen).to(dt)
        v_cache = torch.randn(nb, Hkv, 16, d, generator=gen).to(dt)
        k_new = (torch.randn(B, Hkv, d, generator=gen) * 2.0).to(dt)
        v_new = torch.randn(B, Hkv, d, generator=gen).to(dt)
        P = (torch.stack([synthetic.orthonormal(d, 32, gen) for _ in range(Hkv)]) if per_head
             else synthetic.orthonormal(d, 32, gen))
        ks0 = torch.randint(-2 ** 31, 2 ** 31 - 1, (nb, Hkv, 16), generator=gen, dtype=torch.int32)
        kc, vc, ks = k_cache.cuda(), v_cache.cuda(), ks0.cuda()
        vsa.append_kv_sig(k_new.cuda(), v_new.cuda(), pos.cuda(), bt.cuda(), kc, vc, ks, P.cuda())
        torch.cuda.synchronize()
        want_k, want_v, want_s = k_cache.clone(), v_cache.clone(), ks0.numpy().view(np.uint32).copy()
        for b in range(B):
            p = int(pos[b])
            if p < 0:
                continue
            page, slot = int(bt[b, p // 16]), p % 16
            want_k[page, :, slot] = k_new[b]
            want_v[page, :, slot] = v_new[b]
            for g in range(Hkv):
                Pg = (P[g] if per_head else P).numpy()
                want_s[page, g, slot] = oracle.sign_rows(k_new[b, g:g + 1].float().numpy(), Pg)[0]
        assert torch.equal(kc.cpu(), want_k) and torch.equal(vc.cpu(), want_v)
        assert np.array_equal(ks.cpu().numpy().view(np.uint32), want_s)


def test_append_kv_bit_exact():
    """The newest token of each sequence lands at its page slot in K and V, and
    its low-rank row equals the oracle's projection; other rows are untouched."""
    import torch
    import verified_sparse_attention_amd as vsa
    _, log = _gpu()
    for (d, r, dt, with_lr, per_head) in ((128, 32, torch.bfloat16, True, False), (64, 16, torch.float32, True, False),
                                          (128, 64, torch.bfloat16, True, False), (64, 32, torch.bfloat16, False, False),
                                          (128, 32, torch.bfloat16, True, True), (64, 16, torch.float32, True, True)):
        log("[parity] append_kv d=%d r=%d %s lowrank=%s per_head=%s" % (d, r, dt, with_lr, per_head))
        gen = torch.Generator().manual_seed(7000 + d + r)
        B, Hkv, max_blocks = 5, 3, 6
        nb = B * max_blocks + 4
        bt = torch.randperm(nb, generator=gen)[:B * max_blocks].reshape(B, max_blocks).to(torch.int32)
        pos = torch.tensor([0, 17, 95, -1, 40], dtype=torch.int32)  # -1: no new token
        k_cache = torch.randn(nb, Hkv, 16, d, generator=gen).to(dt)
        v_cache = torch.randn(nb, Hkv, 16, d, generator=gen).to(dt)
        k_new = (torch.randn(B, Hkv, d, generator=gen) * 2.0).to(dt)
        v_new = torch.randn(B, Hkv, d, generator=gen).to(dt)
        P = (torch.stack([synthetic.orthonormal(d, r, gen) for _ in range(Hkv)]) if per_head
             else synthetic.orthonormal(d, r, gen))
        kt0 = torch.randint(-30000, 30000, (nb, Hkv, 16, r), generator=gen, dtype=torch.int16)
        kc, vc, kt = k_cache.cuda(), v_cache.cuda(), kt0.cuda()
        vsa.append_kv(k_new.cuda(), v_new.cuda(), pos.cuda(), bt.cuda(), kc, vc,
                      k_lowrank=kt if with_lr else None, proj=P.cuda() if with_lr else None)
        torch.cuda.synchronize()
        want_k, want_v, want_t = k_cache.clone(), v_cache.clone(), kt0.numpy().view(np.uint16).copy()
        for b in range(B):
            p = int(pos[b])
            if p < 0:
                continue
            page, slot = int(bt[b, p // 16]), p % 16
            want_k[page, :, slot] = k_new[b]
            want_v[page, :, slot] = v_new[b]
            if with_lr and per_head:
                for g in range(Hkv):
                    want_t[page, g, slot] = oracle.project_rows(k_new[b, g:g + 1].float().numpy(), P[g].numpy())[0]
            elif with_lr:
                want_t[page, :, slot] = oracle.project_rows(k_new[b].float().numpy(), P.numpy())
        assert torch.equal(kc.cpu(), want_k) and torch.equal(vc.cpu(), want_v)
        assert np.array_equal(kt.cpu().numpy().view(np.uint16), want_t)


def test_deterministic_repeat():
    w = SMALL_CASES["gqa4_bf16_ragged"]()
    GpuCase, log = _gpu()
    log("[parity] determinism")
    case = GpuCase(w)
    a = case.run(3)
    b = case.run(3)
    for key in ("idx", "counts", "stats", "out", "lse"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("pair", [("gqa4_bf16_ragged", "flat_small"), ("hash_g4_bf16_ragged", "flat_small")])
def test_concurrent_streams(pair):
    """Two decodes with their own workspaces, launched alternately on two
    streams so their kernels can overlap, give exactly what each gives alone:
    the library keeps no state between or across calls (also with a low-rank
    and a hash-signature decode side by side)."""
    import torch
    GpuCase, log = _gpu()
    log("[parity] two streams %s + %s" % pair)
    ca = GpuCase(SMALL_CASES[pair[0]]())
    cb = GpuCase(SMALL_CASES[pair[1]]())
    ref_a, ref_b = ca.run(5), cb.run(9)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    main = torch.cuda.current_stream()
    sa.wait_stream(main)
    sb.wait_stream(main)
    for _ in range(3):
        ca.dec.set_seed(5)
        ca.dec(sa)
        cb.dec.set_seed(9)
        cb.dec(sb)
    torch.cuda.synchronize()
    for case, ref in ((ca, ref_a), (cb, ref_b)):
        got = dict(out=case.dec.out.cpu().numpy(), lse=case.dec.lse.cpu().numpy(),
                   counts=case.dec.counts.cpu().numpy(), idx=case.dec.idx.cpu().numpy(),
                   stats=case.dec.stats.cpu().numpy().view(np.uint64))
        for key in ("idx", "counts", "stats", "out", "lse"):
            assert np.array_equal(got[key], ref[key]), key


# ---------------------------------------------------------------------------
# Output-level mode (guarantee = 1): the numerator statistics TR and NN
# bit-identical to the oracle's (fp64 sums in one order), budgets and index
# sets bit-exact, out/lse within tolerance.  Values with a shared direction
# (v_mean) so the budgets stay below the tail.
# ---------------------------------------------------------------------------
OUTPUT_CASES = {
    "out_tiny": lambda: synthetic.tiny(guarantee=1, v_mean=3.0),
    "out_gqa4_bf16_ragged": lambda: synthetic.make(
        name="out_gqa4_bf16_ragged", B=3, Hq=16, Hkv=4, d=128, seq_lens=(5000, 2500, 777), kv_dtype="bf16",
        recipe="outlier", predictor=1, rank=32, sinks=32, window=64, topk_ppm=25000, shuffle=True, data_seed=11,
        guarantee=1, v_mean=2.0),
    "out_g8_lowrank": lambda: synthetic.make(
        name="out_g8_lowrank", B=2, Hq=16, Hkv=2, d=128, seq_lens=(9000, 4100), kv_dtype="bf16", recipe="lowrank",
        predictor=1, rank=32, sinks=128, window=128, topk_ppm=25000, eps=0.05, data_seed=12, guarantee=1,
        v_mean=3.0),
    "out_d64_f32_g2": lambda: synthetic.make(
        name="out_d64_f32_g2", B=2, Hq=4, Hkv=2, d=64, seq_lens=(3000, 1500), kv_dtype="f32", recipe="planted",
        predictor=1, rank=16, sinks=8, window=16, topk_ppm=20000, data_seed=13, guarantee=1, v_mean=3.0),
    "out_hash_g4": lambda: synthetic.make(
        name="out_hash_g4", B=2, Hq=8, Hkv=2, d=128, seq_lens=(4000, 2222), kv_dtype="bf16", recipe="outlier",
        predictor=2, rank=32, sinks=32, window=32, topk_ppm=25000, data_seed=40, guarantee=1, v_mean=2.0),
    "out_premerge": lambda: synthetic.make(
        name="out_premerge", B=1, Hq=4, Hkv=1, d=128, seq_lens=(40000,), kv_dtype="bf16", recipe="outlier",
        predictor=1, rank=32, sinks=64, window=64, topk_ppm=25000, data_seed=19, guarantee=1, v_mean=3.0),
    "out_zero_mean_dense": lambda: synthetic.make(
        name="out_zero_mean", B=2, Hq=8, Hkv=2, d=128, seq_lens=(3000, 1234), kv_dtype="bf16", recipe="outlier",
        predictor=1, rank=32, sinks=16, window=16, data_seed=24, guarantee=1),
    "out_forced_small": lambda: synthetic.make(
        name="out_forced_small", B=1, Hq=4, Hkv=1, d=64, seq_lens=(1500,), kv_dtype="f32", predictor=0,
        sinks=4, window=4, topk_abs=16, force_budget=7, guarantee=1, v_mean=2.0),
    "out_short_seqs": lambda: synthetic.make(
        name="out_short", B=4, Hq=2, Hkv=1, d=64, seq_lens=(0, 1, 20, 50), kv_dtype="f32", predictor=0, sinks=2,
        window=2, topk_abs=4, guarantee=1, v_mean=1.0),
}


@pytest.mark.parametrize("name", list(OUTPUT_CASES))
def test_parity_output_mode(name):
    run_both(OUTPUT_CASES[name](), seeds=(0, 1, 977), tag=name)


def test_parity_output_mode_tiny_200_seeds():
    w = synthetic.tiny(guarantee=1, v_mean=3.0)
    GpuCase, log = _gpu()
    log("[parity] tiny output mode x 200 seeds")
    case = GpuCase(w)
    arrays = w.oracle_arrays()
    flagged = 0
    for s in range(200):
        cfg = dict(w.cfg, seed=s)
        g = case.run(s)
        o = oracle.decode(**arrays, cfg=cfg)
        compare(w, g, o, tag="tiny output seed=%d" % s)
        flagged += int(np.sum(o["counts"][..., 5] & 8 > 0))
    assert flagged > 0  # the numerator's budget decided some heads


# ---------------------------------------------------------------------------
# Full-size workloads in the benchmark's launch configuration, sampled groups.
# ---------------------------------------------------------------------------
FULL = {
    "llama8b_32k": (lambda: synthetic.llama8b_32k(), [(0, 0), (3, 5), (7, 7)]),
    "flat_128k": (lambda: synthetic.flat_128k(), [(0, 0), (0, 6)]),
    "ragged_b64": (lambda: synthetic.ragged_b64(), [(0, 1), (17, 4), (40, 0), (63, 7)]),
    "wide_gqa_64k": (lambda: synthetic.wide_gqa_64k(), [(1, 2), (3, 7)]),
    "llama8b_32k_output_mode": (lambda: synthetic.llama8b_32k(name="llama8b_32k_output", guarantee=1, v_mean=3.0),
                                [(0, 0), (6, 5)]),
    "llama8b_32k_hash": (lambda: synthetic.llama8b_32k(name="llama8b_32k_hash", predictor=2),
                         [(0, 0), (5, 3)]),
    # one query head per KV head at 2^20 tokens: predictor chunks of 32768
    # tokens, the largest one block takes (eight slot iterations per thread,
    # sample words drawn again for the counting sort)
    "g1_1m_chunk32k": (lambda: synthetic.make(
        name="g1_1m_chunk32k", B=1, Hq=8, Hkv=8, d=64, seq_lens=(1 << 20,), kv_dtype="bf16",
        recipe="outlier", predictor=1, rank=32, sinks=64, window=64, topk_ppm=2500, eps=0.05,
        data_seed=33), [(0, 0), (0, 5)]),
    # the longest sequence the library takes (2^20 tokens): 256 predictor
    # chunks pre-merged in parts, 1024 gather chunks, 32 emission passes
    "max_seq_1m": (lambda: synthetic.make(
        name="max_seq_1m", B=1, Hq=4, Hkv=1, d=64, seq_lens=(1 << 20,), kv_dtype="bf16",
        recipe="outlier", predictor=1, rank=32, sinks=64, window=64, topk_ppm=2500, eps=0.05,
        data_seed=31), [(0, 0)]),
}


@pytest.mark.parametrize("name", list(FULL))
def test_parity_full_size_sampled(name):
    mk, groups = FULL[name]
    w = mk()
    case = run_both(w, seeds=(0,), groups=groups, want_idx=True, tag=name)
    if name == "wide_gqa_64k":
        arrays = w.oracle_arrays()
        for eps in (0.01, 0.02, 0.1):
            cfg = dict(w.cfg, eps=eps)
            case.dec.cfg.eps = eps
            case.dec._ccfg.eps = eps
            g = case.run(0)
            o = oracle.decode(**arrays, cfg=cfg, groups=groups[:1], nthreads=8)
            compare(w, g, o, groups[:1], tag="%s eps=%g" % (name, eps))


# ---------------------------------------------------------------------------
# (eps, delta) on the GPU against the oracle's dense fp64 lse.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,mk", [
    ("tiny", lambda: synthetic.tiny()),
    ("flat_gqa", lambda: synthetic.make(name="flat_gqa", B=1, Hq=16, Hkv=4, d=128, seq_lens=(8192,),
                                        kv_dtype="bf16", recipe="flat", q_std=0.3, k_std=0.3,
                                        predictor=1, rank=32, sinks=128, window=128,
                                        topk_ppm=10000, eps=0.02, data_seed=21)),
    ("peaked_gqa", lambda: synthetic.make(name="peaked_gqa", B=1, Hq=16, Hkv=4, d=128,
                                          seq_lens=(8192,), kv_dtype="bf16", recipe="outlier",
                                          predictor=1, rank=32, sinks=128, window=128,
                                          topk_ppm=25000, eps=0.05, data_seed=22)),
])
def test_gpu_eps_delta_rate(name, mk):
    w = mk()
    GpuCase, log = _gpu()
    log("[rate] %s x 1000 seeds" % name)
    case = GpuCase(w, want_idx=False)
    dense = oracle.decode(**w.oracle_arrays(), cfg=w.cfg, want_dense=True, want_idx=False,
                          nthreads=8)["lse_dense"]
    viol = trials = 0
    for s in range(1000):
        g = case.run(s)
        rel = np.abs(np.exp(g["lse"].astype(np.float64) - dense) - 1.0)
        viol += int((rel > w.cfg["eps"]).sum())
        trials += rel.size
    rate = viol / trials
    from scipy.stats import beta
    ub = float(beta.ppf(0.95, viol + 1, trials - viol)) if viol < trials else 1.0
    log("[rate] %s: %d / %d = %.4f (95%% CP upper %.4f), delta %.3f"
        % (name, viol, trials, rate, ub, w.cfg["delta"]))
    assert rate <= w.cfg["delta"]


# ---------------------------------------------------------------------------
# Key Gram matrices (calibration of a per-head predictor basis).
# ---------------------------------------------------------------------------
def _host_keys(w):
    """fp64 keys per (b, KV head) through the block table, as the decode reads them."""
    import torch
    kc = w.k_cache.double()
    out = []
    for b in range(w.B):
        L = int(w.seq_lens[b])
        pages = w.block_table[b, :(L + 15) // 16].long()
        out.append(kc[pages].permute(1, 0, 2, 3).reshape(w.Hkv, -1, w.d)[:, :L].numpy())
    return out


def _gram_ref(w):
    """The oracle's fp64 key Gram and its |K| |K|^T scale (oracle.key_gram)."""
    return oracle.key_gram(**w.oracle_arrays())


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (3 << 20) + 16 * 37])
def test_read_probe_checksum(nbytes):
    """vattn_read_probe XORs every 32-bit word of the buffer into the sink's
    words: their XOR against numpy's XOR of the same words (sizes with a
    ragged tail)."""
    import torch
    import verified_sparse_attention_amd as vsa
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(vsa.READ_PROBE_SINK, dtype=torch.int32, device="cuda")
    vsa.read_probe(buf, sink)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(host)


@pytest.mark.parametrize("name,mk", [
    ("d128_ragged_shuffled", lambda: synthetic.make(
        name="gram_d128", B=3, Hq=8, Hkv=2, d=128, seq_lens=(5000, 777, 4096), kv_dtype="bf16",
        recipe="outlier", predictor=1, rank=32, shuffle=True, data_seed=51)),
    ("d64_one_empty", lambda: synthetic.make(
        name="gram_d64", B=3, Hq=8, Hkv=4, d=64, seq_lens=(9000, 0, 100), kv_dtype="bf16",
        recipe="normal", predictor=1, rank=16, data_seed=52)),
])
def test_key_gram_matches_fp64(name, mk):
    """gram[g] = sum_t K_t K_t^T against the oracle's fp64 sums: bf16 products are
    exact in fp32 and the sums are fp32, so each entry is within 1e-5 (about 170
    fp32 ulps) of the sum of the products' magnitudes of the fp64 value."""
    import torch
    import verified_sparse_attention_amd as vsa
    _, log = _gpu()
    w = mk()
    log("[parity] key_gram %s" % name)
    gram = vsa.key_gram(w.k_cache.cuda(), w.block_table.cuda(), w.seq_lens.cuda(), w.max_seq_len)
    torch.cuda.synchronize()
    g, a = _gram_ref(w)
    got = gram.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - g) <= 1e-5 * a + 1e-30), float(np.max(np.abs(got - g) / (a + 1e-30)))
    again = vsa.key_gram(w.k_cache.cuda(), w.block_table.cuda(), w.seq_lens.cuda(), w.max_seq_len)
    assert torch.equal(gram, again)  # fixed summation order


def test_pca_bases_from_the_gram():
    """Keys K = Z U_g^T + N(0, 0.1^2) with a 24-dimensional U_g per KV head: the
    second moments are n (U_g U_g^T + 0.01 I), so the Gram's 24th eigenvalue
    exceeds the 25th about 100-fold.  Its 32 leading eigenvectors per head then
    serve as per-head predictor bases: the decode stays bit-exact against the
    oracle, and the predicted top-k tracks the exact-score top-k far better than
    with random bases (the keys' residual outside the 24 dimensions still
    reorders near ties)."""
    import torch
    import verified_sparse_attention_amd as vsa
    GpuCase, log = _gpu()
    w = synthetic.make(name="pca_bases", B=2, Hq=16, Hkv=2, d=128, seq_lens=(6000, 3000), kv_dtype="bf16",
                       recipe="lowrank", lowrank_dim=24, lowrank_noise=0.1, predictor=1, rank=32,
                       sinks=32, window=32, topk_ppm=25000, data_seed=53)
    log("[parity] pca bases")
    gram = vsa.key_gram(w.k_cache.cuda(), w.block_table.cuda(), w.seq_lens.cuda(), w.max_seq_len)
    G = gram.cpu().numpy().astype(np.float64)
    bases = []
    for g in range(w.Hkv):
        lam, vec = np.linalg.eigh(G[g])  # ascending
        lam, vec = lam[::-1], vec[:, ::-1]
        assert lam[23] > 20 * lam[24], (g, lam[22:26])
        bases.append(vec[:, :32])
    pca = torch.tensor(np.stack(bases), dtype=torch.float32)
    w_pca = dataclasses.replace(w, proj=pca)
    run_both(w_pca, seeds=(0,), tag="pca bases")
    # predicted top-k against the exact-score top-k (oracle predictor scores)
    arrays = w.oracle_arrays()
    keys = _host_keys(w)
    q = arrays["q"].astype(np.float64)
    Gq = w.Hq // w.Hkv

    def overlap(P):
        o = oracle.decode(**dict(arrays, proj=P), cfg=w.cfg, want_pred=True)
        tot, hit = 0, 0
        for b in range(w.B):
            for h in range(w.Hq):
                pred = o["pred"][b, h]
                mid = np.nonzero(~np.isnan(pred))[0]
                k = int(o["counts"][b, h, 0]) - 64
                exact = keys[b][h // Gq][mid] @ q[b, h]
                top_p = set(mid[np.argsort(-pred[mid], kind="stable")[:k]])
                top_e = set(mid[np.argsort(-exact, kind="stable")[:k]])
                tot += k
                hit += len(top_p & top_e)
        return hit / tot
    ov_pca = overlap(np.stack(bases).astype(np.float32))
    ov_rand = overlap(w.proj.numpy())
    log("   top-k overlap with exact scores: pca %.3f, random %.3f" % (ov_pca, ov_rand))
    assert ov_pca > 0.7 and ov_pca > ov_rand + 0.3  # measured on the CPU: 0.81 against 0.19


@pytest.mark.parametrize("name", ["gqa4_bf16_ragged", "hash_g4_bf16_ragged"])
def test_graph_replay(name):
    """A decode captured in a HIP graph (no allocation, no memset inside) and
    replayed with new queries written into the same buffer gives, on every
    replay, exactly the eager result for those queries.  The configuration,
    seed included, is part of the captured launch.  Low-rank and hash-signature
    predictors."""
    import torch
    GpuCase, log = _gpu()
    log("[parity] graph replay %s" % name)
    case = GpuCase(SMALL_CASES[name]())
    gen = torch.Generator().manual_seed(77)
    qs = [torch.randn(case.q.shape, generator=gen).cuda() for _ in range(3)]
    keys = ("idx", "counts", "stats", "out", "lse")

    def outputs():
        d = case.dec
        return dict(out=d.out.cpu().numpy(), lse=d.lse.cpu().numpy(), counts=d.counts.cpu().numpy(),
                    idx=d.idx.cpu().numpy(), stats=d.stats.cpu().numpy().view(np.uint64))
    eager = []
    for qn in qs:
        case.q.copy_(qn)
        case.run(11)
        eager.append(outputs())
    case.q.copy_(qs[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        case.dec()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        case.dec()
    torch.cuda.synchronize()
    for rep in range(2):
        for i, qn in enumerate(qs):
            case.q.copy_(qn)
            graph.replay()
            torch.cuda.synchronize()
            got = outputs()
            for key in keys:
                assert np.array_equal(got[key], eager[i][key]), (rep, i, key)
            case.q.copy_(qs[(i + 1) % len(qs)])  # eager work between the replays
            case.run(11)


def test_page_layout_does_not_change_results():
    """The same tokens in pages moved to other physical ids (block table
    rewritten to match): the decode's index sets, counts, statistics and
    outputs are bit-identical to the identity layout's."""
    GpuCase, log = _gpu()
    w = synthetic.make(name="layout", B=2, Hq=16, Hkv=4, d=128, seq_lens=(9000, 5000), kv_dtype="bf16",
                       recipe="outlier", predictor=1, rank=32, sinks=64, window=64, topk_ppm=25000, data_seed=61)
    log("[parity] page layout")
    a = GpuCase(w).run(seed=4)
    b = GpuCase(synthetic.repaged(w, seed=9)).run(seed=4)
    for key in ("idx", "counts", "stats", "out", "lse"):
        assert np.array_equal(a[key], b[key]), key
