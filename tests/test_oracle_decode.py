"""Pins of the oracle's decode step against what the pages and mathematics fix.

* Exact reduction: when the sample covers the whole tail every weight is 1, so
  the output must equal dense softmax attention (torch SDPA in fp64 on the CPU).
* The index set always holds sinks and window; its top-k part is the k best
  predictor scores (checked against an fp64 recomputation and numpy lexsort);
  its sampled part is the first n tail tokens in (Philox word, index) order.
* The sampler includes each tail token with probability n / N_t (chi-square).
* At a fixed budget the denominator and numerator estimates are unbiased and
  the denominator's variance is the textbook without-replacement variance.
* The budget equals the CLT expression evaluated in exact rationals.
* The empirical rate of denominator relative error above eps is <= delta.
* Degenerate inputs: empty and one-token sequences, tails of 0, 1, 2 tokens,
  k covering the whole middle, no sinks/window.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic


def run(w, **kw):
    return oracle.decode(**w.oracle_arrays(), cfg=w.cfg, **kw)


def dense_sdpa_fp64(w):
    """Reference dense attention per (b, h) with torch in float64 on the CPU."""
    a = w.oracle_arrays()
    q = torch.from_numpy(a["q"]).double()
    B, Hq, d = q.shape
    G = Hq // w.Hkv
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    kc = w.k_cache.double()
    vc = w.v_cache.double()
    for b in range(B):
        L = int(w.seq_lens[b])
        if L == 0:
            lse[b] = -np.inf
            continue
        pages = w.block_table[b, :(L + 15) // 16].long()
        K = kc[pages].permute(1, 0, 2, 3).reshape(w.Hkv, -1, d)[:, :L]
        V = vc[pages].permute(1, 0, 2, 3).reshape(w.Hkv, -1, d)[:, :L]
        Kq = K.repeat_interleave(G, 0).unsqueeze(0)
        Vq = V.repeat_interleave(G, 0).unsqueeze(0)
        qq = q[b].view(1, Hq, 1, d)
        o = torch.nn.functional.scaled_dot_product_attention(qq, Kq.contiguous(), Vq.contiguous())
        out[b] = o[0, :, 0].numpy()
        s = (qq @ Kq.transpose(-1, -2).contiguous())[0, :, 0] / math.sqrt(d)
        lse[b] = torch.logsumexp(s, dim=-1).numpy()
    return out, lse


SMALL = [
    lambda **k: synthetic.tiny(**k),
    lambda **k: synthetic.make(name="gqa_bf16", B=2, Hq=8, Hkv=2, d=128, seq_lens=(700, 333),
                               kv_dtype="bf16", recipe="outlier", predictor=1, rank=32,
                               sinks=16, window=16, topk_ppm=25000, **k),
    lambda **k: synthetic.make(name="ragged_shuffled", B=3, Hq=4, Hkv=1, d=64,
                               seq_lens=(257, 40, 129), kv_dtype="bf16", recipe="planted",
                               predictor=1, rank=16, sinks=4, window=8, topk_ppm=50000,
                               shuffle=True, **k),
]


@pytest.mark.parametrize("mk", SMALL)
def test_full_budget_reduces_to_dense_sdpa(mk):
    w = mk(force_budget=10 ** 9)
    r = run(w, want_dense=True)
    ref_out, ref_lse = dense_sdpa_fp64(w)
    assert np.all(r["counts"][..., 3] == r["counts"][..., 1])  # n == N_t
    assert np.max(np.abs(r["out"] - ref_out)) < 1e-12
    assert np.max(np.abs(r["lse"] - ref_lse)) < 1e-12
    assert np.max(np.abs(r["out_dense"] - ref_out)) < 1e-12
    assert np.max(np.abs(r["lse_dense"] - ref_lse)) < 1e-12
    # every token is in the index set
    for b in range(w.B):
        L = int(w.seq_lens[b])
        for h in range(w.Hq):
            assert list(r["idx"][b, h, :L]) == list(range(L))


def test_short_sequence_is_dense_without_forcing():
    w = synthetic.make(B=2, Hq=2, Hkv=1, d=64, seq_lens=(36, 20), kv_dtype="f32", predictor=0,
                       sinks=4, window=32, topk_abs=8)
    r = run(w, want_dense=True)
    ref_out, ref_lse = dense_sdpa_fp64(w)
    assert np.max(np.abs(r["out"] - ref_out)) < 1e-12
    assert np.max(np.abs(r["lse"] - ref_lse)) < 1e-12
    assert np.all(r["counts"][..., 1] == 0)


def _structure_check(w, r):
    cfg = w.cfg
    d = w.d
    G = w.Hq // w.Hkv
    for b in range(w.B):
        L = int(w.seq_lens[b])
        for h in range(w.Hq):
            g = h // G
            if L == 0:      # no step runs: all counts zero, empty index set
                assert np.all(r["counts"][b, h] == 0) and np.all(r["idx"][b, h] == -1)
                continue
            n_fixed, NT, nb, n, cnt, flags = (int(x) for x in r["counts"][b, h])
            I = r["idx"][b, h]
            I = I[I >= 0]
            assert len(I) == cnt == n_fixed + n
            assert np.all(np.diff(I) > 0)                      # sorted, unique
            sp = min(cfg["sinks"], L)
            wp = min(cfg["window"], L - sp)
            lo, hi = sp, L - wp
            Iset = set(I.tolist())
            assert set(range(sp)) <= Iset and set(range(hi, L)) <= Iset   # sinks, window
            nM = hi - lo
            k = cfg["topk_abs"] if cfg["topk_abs"] >= 0 else -(-L * cfg["topk_ppm"] // 10 ** 6)
            k = min(k, nM)
            assert n_fixed == sp + wp + k and NT == nM - k
            # top-k: numpy lexsort on (-score, index) over the middle
            mid = np.arange(lo, hi)
            sc = r["pred"][b, h, lo:hi].astype(np.float64)
            order = np.lexsort((mid, -sc))
            T = set(mid[order[:k]].tolist())
            assert T <= Iset
            tail = np.array(sorted(set(mid.tolist()) - T), dtype=np.int64)
            assert len(tail) == NT
            # sample: first n of the tail in (Philox word, index) order
            u = oracle.token_keys(cfg["seed"], b, g, max(L, 1))[tail] if NT else np.zeros(0)
            rho = tail[np.lexsort((tail, u))] if NT else tail
            S = set(rho[:n].tolist())
            assert Iset - set(range(sp)) - set(range(hi, L)) - T == S
            if NT:
                want_nb = min(NT, max(2, -(-NT * cfg["base_ppm"] // 10 ** 6)))
                assert nb == want_nb
                if cfg["force_budget"] < 0:
                    assert nb <= n <= NT
                    assert set(rho[:nb].tolist()) <= S        # base sample nested in the final
            assert bool(flags & 1) == (n == NT)


@pytest.mark.parametrize("mk", SMALL)
@pytest.mark.parametrize("seed", [0, 1, 12345])
def test_index_set_structure(mk, seed):
    w = mk(seed=seed)
    r = run(w, want_pred=True)
    _structure_check(w, r)


def test_predictor_scores_vs_fp64_and_topk_gap():
    for w in (synthetic.tiny(), SMALL[1]()):
        r = run(w, want_pred=True)
        a = w.oracle_arrays()
        d = w.d
        G = w.Hq // w.Hkv
        scale = np.float32(1.0 / math.sqrt(d))
        for b in range(w.B):
            L = int(w.seq_lens[b])
            pages = w.block_table[b, :(L + 15) // 16].long()
            Kall = w.k_cache.float()[pages].permute(1, 0, 2, 3).reshape(w.Hkv, -1, d)[:, :L].numpy()
            for h in range(w.Hq):
                g = h // G
                qs = (a["q"][b, h] * scale).astype(np.float32)
                pred = r["pred"][b, h, :L]
                mid = ~np.isnan(pred)
                if w.cfg["predictor"] == 1:
                    Kt = oracle.project_rows(Kall[g], a["proj"])
                    Ktf = (Kt.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                    qt = qs.astype(np.float64) @ a["proj"].astype(np.float64)
                    ref = Ktf @ qt
                    mag = np.abs(Ktf) @ (np.abs(qs.astype(np.float64)) @ np.abs(a["proj"]))
                    tol = (d + w.cfg["rank"] + 2) * 2.0 ** -24 * mag * 1.5
                else:
                    ref = Kall[g].astype(np.float64) @ qs.astype(np.float64)
                    tol = (d + 2) * 2.0 ** -24 * (np.abs(Kall[g]) @ np.abs(qs))
                assert np.all(np.abs(pred[mid] - ref[mid]) <= tol[mid])
                # top-k by fp64 scores agrees except within the rounding band
                k = r["counts"][b, h, 0] - min(w.cfg["sinks"], L) - min(w.cfg["window"], L - min(w.cfg["sinks"], L))
                I = set(r["idx"][b, h][r["idx"][b, h] >= 0].tolist())
                midx = np.nonzero(mid)[0]
                srt = np.sort(ref[midx])[::-1]
                kth = srt[k - 1]
                band = 2 * tol[midx].max()
                for i in midx:
                    if ref[i] > kth + band:
                        assert i in I


def test_planted_heavy_hitters_are_kept():
    w = synthetic.tiny()
    r = run(w)
    per_head = {}
    for (b, h, pos) in w.meta["plants"]:
        I = set(r["idx"][b, h][r["idx"][b, h] >= 0].tolist())
        per_head.setdefault(h, []).append(pos in I)
    assert len(per_head) == 4
    for h, hits in per_head.items():
        assert sum(hits) >= 7, (h, hits)


def _tiny_tail_workload(seed, n_force, L=160):
    return synthetic.make(B=1, Hq=2, Hkv=1, d=64, seq_lens=(L,), kv_dtype="f32",
                          recipe="normal", predictor=0, sinks=4, window=4, topk_abs=8,
                          force_budget=n_force, seed=seed, data_seed=77, k_std=1.5)


def test_sampler_inclusion_is_uniform():
    n_force, seeds = 30, 3000
    counts = None
    for s in range(seeds):
        w = _tiny_tail_workload(s, n_force)
        r = run(w)
        if counts is None:
            base = [set(r["idx"][0, h][r["idx"][0, h] >= 0].tolist()) for h in range(2)]
            NT = int(r["counts"][0, 0, 1])
            counts = np.zeros((2, 160))
        for h in range(2):
            I = r["idx"][0, h]
            counts[h, I[I >= 0]] += 1
    for h in range(2):
        fixed = counts[h] == seeds
        tail = counts[h][~fixed & (np.arange(160) >= 4) & (np.arange(160) < 156)]
        # the tail is everything in the middle that is not always present
        NT = int(r["counts"][0, h, 1])
        assert tail.size == NT
        expect = seeds * n_force / NT
        chi2 = float(((tail - expect) ** 2 / (expect * (1 - n_force / NT))).sum())
        # dof = NT - 1 (about 143); far-tail rejection only
        assert 0.5 * NT < chi2 < 1.6 * NT, chi2


def test_fixed_budget_estimates_are_unbiased():
    n_force, seeds = 20, 4000
    Dhat, Nhat = [], []
    for s in range(seeds):
        w = _tiny_tail_workload(s, n_force)
        r = run(w, want_dense=True)
        ratio = np.exp(r["lse"][0] - r["lse_dense"][0])             # D_hat / D
        Dhat.append(ratio)
        Nhat.append(r["out"][0] * ratio[:, None])                   # N_hat / D
        if s == 0:
            out_dense = r["out_dense"][0]
            NT = int(r["counts"][0, 0, 1])
    Dhat = np.array(Dhat)
    Nhat = np.array(Nhat)
    se = Dhat.std(axis=0, ddof=1) / math.sqrt(seeds)
    assert np.all(np.abs(Dhat.mean(axis=0) - 1.0) < 4.5 * se), (Dhat.mean(axis=0), se)
    seN = Nhat.std(axis=0, ddof=1) / math.sqrt(seeds)
    z = np.abs(Nhat.mean(axis=0) - out_dense) / seN
    assert z.max() < 5.0, z.max()

    # variance of D_hat: N_t^2 (1 - n/N_t) S^2 / n with S^2 the tail's variance
    w = _tiny_tail_workload(0, 10 ** 9)
    r = run(w, want_dense=True)
    a = w.oracle_arrays()
    K = a["k_cache"][:, 0].reshape(-1, 64)[:160].astype(np.float64)
    for h in range(2):
        q = a["q"][0, h].astype(np.float64)
        sig = K @ q / 8.0
        lse_d = r["lse_dense"][0, h]
        e = np.exp(sig - lse_d)                                    # e_i / D
        I_f = set(range(4)) | set(range(156, 160))
        rr = run(_tiny_tail_workload(0, n_force), want_pred=True)
        mid = np.arange(4, 156)
        order = np.lexsort((mid, -rr["pred"][0, h, 4:156].astype(np.float64)))
        I_f |= set(mid[order[:8]].tolist())
        tail = np.array([e[i] for i in range(160) if i not in I_f])
        assert tail.size == NT
        S2 = tail.var(ddof=1)
        var_theory = NT ** 2 * (1 - n_force / NT) * S2 / n_force
        v = Dhat[:, h].var(ddof=1)
        m4 = ((Dhat[:, h] - Dhat[:, h].mean()) ** 4).mean()
        se_v = math.sqrt(max(m4 - v * v, 1e-30) / seeds)
        assert abs(v - var_theory) < 5 * se_v, (v, var_theory, se_v)


def _exact_budget(z32, eps, NT, nb, SF, S1, S2):
    M2 = nb * S2 - S1 * S1
    Y = nb * SF + NT * S1
    val = Fraction(z32) ** 2 * NT * NT * M2 * nb / ((nb - 1) * Fraction(eps) ** 2 * Y * Y)
    if val >= NT:
        return NT, val
    n = math.ceil(val)
    return max(n, nb), val


@pytest.mark.parametrize("mk,seeds", [(SMALL[0], range(40)), (SMALL[1], range(8)),
                                      (SMALL[2], range(8))])
def test_budget_equals_exact_rational_clt_bound(mk, seeds):
    checked = 0
    for s in seeds:
        w = mk(seed=s)
        r = run(w)
        z32 = r["z32"]
        eps = w.cfg["eps"]
        for b in range(w.B):
            for h in range(w.Hq):
                n_fixed, NT, nb, n, cnt, flags = (int(x) for x in r["counts"][b, h])
                SF, S1, S2hi, S2lo = (int(x) for x in r["stats"][b, h])
                S2 = (S2hi << 64) | S2lo
                if NT == 0:
                    assert n == 0 and nb == 0
                    continue
                if nb == NT:
                    assert n == NT
                    continue
                want, val = _exact_budget(z32, eps, NT, nb, SF, S1, S2)
                near = abs(val - round(val)) < Fraction(1, 10 ** 9) * max(1, val)
                if not near:
                    assert n == want, (b, h, n, want, float(val))
                    checked += 1
                # the fixed-point sums are consistent with the sizes
                assert SF <= n_fixed * 2 ** 40 and S1 <= nb * 2 ** 40 and S2 <= S1 * 2 ** 40
    assert checked > 0


def _violation_rate(make_w, seeds):
    viol = trials = 0
    for s in seeds:
        w = make_w(s)
        r = run(w, want_dense=True, want_idx=False)
        rel = np.abs(np.exp(r["lse"] - r["lse_dense"]) - 1.0)
        viol += int((rel > w.cfg["eps"]).sum())
        trials += rel.size
    return viol, trials


def _clopper_pearson_upper(k, n, conf=0.95):
    from scipy.stats import beta
    return 1.0 if k == n else float(beta.ppf(conf, k + 1, n - k))


@pytest.mark.parametrize("name,make_w", [
    ("tiny", lambda s: synthetic.tiny(seed=s)),
    ("flat", lambda s: synthetic.make(B=1, Hq=4, Hkv=2, d=64, seq_lens=(2048,), kv_dtype="bf16",
                                      recipe="flat", q_std=0.3, k_std=0.3, predictor=1, rank=16,
                                      sinks=16, window=16, topk_ppm=10000, eps=0.02,
                                      delta=0.05, seed=s, data_seed=31)),
    ("peaked_gqa", lambda s: synthetic.make(B=1, Hq=4, Hkv=1, d=64, seq_lens=(1536,),
                                            kv_dtype="bf16", recipe="outlier", predictor=1,
                                            rank=16, sinks=8, window=16, topk_ppm=25000,
                                            eps=0.05, delta=0.1, seed=s, data_seed=32)),
])
def test_eps_delta_violation_rate(name, make_w):
    viol, trials = _violation_rate(make_w, range(1000))
    delta = make_w(0).cfg["delta"]
    rate = viol / trials
    ub = _clopper_pearson_upper(viol, trials)
    print("%s: violations %d / %d = %.4f (95%% CP upper %.4f), delta %.3f"
          % (name, viol, trials, rate, ub, delta))
    assert trials >= 1000 * 4
    assert rate <= delta


def test_degenerate_inputs():
    # L = 0, L = 1, ragged with an empty sequence
    w = synthetic.make(B=3, Hq=2, Hkv=1, d=64, seq_lens=(0, 1, 50), kv_dtype="f32",
                       predictor=0, sinks=2, window=2, topk_abs=4)
    r = run(w, want_dense=True, want_pred=True)
    assert np.all(r["out"][0] == 0) and np.all(np.isneginf(r["lse"][0]))
    assert np.all(r["counts"][0] == 0) and np.all(r["idx"][0] == -1)
    assert np.all(r["counts"][1, :, 4] == 1)
    ref_out, ref_lse = dense_sdpa_fp64(w)
    assert np.max(np.abs(r["out"][1] - ref_out[1])) < 1e-12
    _structure_check(w, r)
    # tails of 1 and 2 tokens are taken whole; k covering the whole middle
    for L, k, NT in ((13, 8, 1), (14, 8, 2), (30, 100, 0)):
        w = synthetic.make(B=1, Hq=2, Hkv=1, d=64, seq_lens=(L,), kv_dtype="f32", predictor=0,
                           sinks=2, window=2, topk_abs=k)
        r = run(w, want_dense=True, want_pred=True)
        assert np.all(r["counts"][0, :, 1] == NT) and np.all(r["counts"][0, :, 3] == NT)
        assert np.max(np.abs(r["lse"] - r["lse_dense"])) < 1e-12
        _structure_check(w, r)
    # no sinks, no window, no top-k: pure sampling over the whole sequence
    w = synthetic.make(B=1, Hq=2, Hkv=1, d=64, seq_lens=(500,), kv_dtype="f32", predictor=0,
                       sinks=0, window=0, topk_abs=0, recipe="flat", q_std=0.3, k_std=0.3)
    r = run(w, want_pred=True)
    assert np.all(r["counts"][0, :, 0] == 0) and np.all(r["counts"][0, :, 1] == 500)
    _structure_check(w, r)


# ---------------------------------------------------------------------------
# One predictor basis per KV head: each group's low-rank query and keys use
# its own basis, and nothing else changes.
# ---------------------------------------------------------------------------
def _per_head_case():
    return synthetic.make(name="per_head_bases", B=2, Hq=8, Hkv=4, d=64, seq_lens=(900, 517),
                          kv_dtype="bf16", recipe="outlier", predictor=1, rank=16, sinks=8,
                          window=16, topk_ppm=30000, proj_per_head=True, data_seed=41)


def test_per_head_bases_equal_to_one_shared_basis_give_its_results():
    w = _per_head_case()
    a = w.oracle_arrays()
    P = a["proj"][1]
    shared = oracle.decode(**dict(a, proj=P), cfg=w.cfg)
    stacked = oracle.decode(**dict(a, proj=np.stack([P] * w.Hkv)), cfg=w.cfg)
    for key in ("idx", "counts", "stats", "out", "lse"):
        assert np.array_equal(shared[key], stacked[key]), key


def test_each_group_uses_its_own_basis():
    w = _per_head_case()
    a = w.oracle_arrays()
    assert a["proj"].shape == (w.Hkv, w.d, 16)
    full = oracle.decode(**a, cfg=w.cfg)
    G = w.Hq // w.Hkv
    differs = 0
    for g in range(w.Hkv):
        own = oracle.decode(**dict(a, proj=a["proj"][g]), cfg=w.cfg, groups=[(b, g) for b in range(w.B)])
        other = oracle.decode(**dict(a, proj=a["proj"][(g + 1) % w.Hkv]), cfg=w.cfg,
                              groups=[(b, g) for b in range(w.B)])
        hs = slice(g * G, (g + 1) * G)
        for key in ("idx", "counts", "stats", "out", "lse"):
            assert np.array_equal(full[key][:, hs], own[key][:, hs]), (g, key)
        differs += int(not np.array_equal(full["idx"][:, hs], other["idx"][:, hs]))
    assert differs > 0  # the bases matter: another head's basis selects other tokens


def test_results_do_not_depend_on_page_layout():
    """The pages of a cache moved to other physical ids (block table rewritten
    to match) hold the same tokens: index sets, counts, statistics and outputs
    are identical (a mixed-up page or token index would move them)."""
    for w in (synthetic.tiny(seed=0),
              synthetic.make(name="repage_lowrank", B=2, Hq=8, Hkv=2, d=64, seq_lens=(1500, 700),
                             kv_dtype="bf16", predictor=1, rank=16, sinks=8, window=16, topk_ppm=30000,
                             data_seed=77)):
        r = synthetic.repaged(w, seed=3)
        assert not np.array_equal(r.block_table.numpy(), w.block_table.numpy())
        a = oracle.decode(**w.oracle_arrays(), cfg=w.cfg)
        b = oracle.decode(**r.oracle_arrays(), cfg=r.cfg)
        for key in ("idx", "counts", "stats", "out", "lse"):
            assert np.array_equal(a[key], b[key]), key
