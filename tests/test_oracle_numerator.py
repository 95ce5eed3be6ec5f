"""Pins of the oracle's output-level mode (guarantee = 1): the numerator
N = sum_i e^{s_i - m} V_i held to the same central-limit bound as the
denominator (SkyLight post "vAttention Computation": guarantees on the
intermediate computations; edgentiq post "How vAttention Works": the
denominator-only budget is a relaxation of this).

* With every value V_i = (1, ..., 1) the numerator is the denominator in every
  channel, so its statistics are d times the exact integer ones and its budget
  is the denominator's.
* TR and NN equal an independent fp64 recomputation from rebuilt sets, and
  plausible mistakes (T1 over the final sample, NF without the top-k, the base
  sample in index order) fall far outside the bound.
* The budget is the larger of the two CLT expressions evaluated in exact
  rationals from the reported statistics.
* Zero-mean values make the estimated numerator small against its spread: the
  budget takes the whole tail and the output is exactly dense attention.
* Over 1000 seeds the numerator's relative L2 error exceeds eps in at most a
  fraction delta of the heads, and so does the denominator's.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic

U53 = 2.0 ** -53


def run(w, **kw):
    return oracle.decode(**w.oracle_arrays(), cfg=w.cfg, **kw)


def _ones(w):
    a = w.oracle_arrays()
    v = np.ones_like(a["v_cache"]) if a["v_cache"].dtype != np.uint16 else np.full_like(a["v_cache"], 0x3F80)
    return dict(a, v_cache=v)


CASES = [
    lambda **k: synthetic.tiny(guarantee=1, **k),
    lambda **k: synthetic.make(name="num_gqa_bf16", B=2, Hq=8, Hkv=2, d=128, seq_lens=(1500, 777), kv_dtype="bf16",
                               recipe="outlier", predictor=1, rank=32, sinks=16, window=16, topk_ppm=25000,
                               guarantee=1, data_seed=81, **k),
]


@pytest.mark.parametrize("mk", CASES)
def test_values_of_ones_reduce_to_the_denominator(mk):
    w = mk()
    d = w.d
    r = oracle.decode(**_ones(w), cfg=w.cfg)
    r0 = oracle.decode(**_ones(w), cfg=dict(w.cfg, guarantee=0))
    checked = 0
    for b in range(w.B):
        for h in range(w.Hq):
            n_fixed, NT, nb, n, cnt, flags = (int(x) for x in r["counts"][b, h])
            SF, S1, S2hi, S2lo = (int(x) for x in r["stats"][b, h])
            S2 = (S2hi << 64) | S2lo
            if NT == 0 or nb == NT:
                continue
            TR, NN = (float(x) for x in r["num_stats"][b, h])
            M2 = nb * S2 - S1 * S1
            Y = nb * SF + NT * S1
            assert abs(TR - d * M2) <= 1e-12 * d * nb * S2 + 1.0, (b, h, TR, d * M2)
            assert abs(NN - d * Y * Y) <= 1e-12 * d * Y * Y, (b, h, NN, d * Y * Y)
            # the same expression: the budget is the denominator's (one more
            # only where rounding puts the numerator's a hair above an integer)
            n0 = int(r0["counts"][b, h, 3])
            assert n in (n0, n0 + 1), (b, h, n, n0)
            checked += 1
    assert checked > 0


def _sets(w, r, b, h):
    cfg = w.cfg
    G = w.Hq // w.Hkv
    L = int(w.seq_lens[b])
    sp = min(cfg["sinks"], L)
    wp = min(cfg["window"], L - sp)
    lo, hi = sp, L - wp
    k = cfg["topk_abs"] if cfg["topk_abs"] >= 0 else -(-L * cfg["topk_ppm"] // 10 ** 6)
    k = min(k, hi - lo)
    mid = np.arange(lo, hi)
    T = mid[np.lexsort((mid, -r["pred"][b, h, lo:hi].astype(np.float64)))[:k]]
    fixed = np.sort(np.concatenate([np.arange(sp), np.arange(hi, L), T]).astype(np.int64))
    tail = np.setdiff1d(mid, T)
    NT = tail.size
    nb = 0 if NT == 0 else min(NT, max(2, -(-NT * cfg["base_ppm"] // 10 ** 6)))
    u = oracle.token_keys(cfg["seed"], b, h // G, L)[tail]
    rho = tail[np.lexsort((tail, u))]
    return dict(fixed=fixed, T=T, sb=np.sort(rho[:nb]), S=np.sort(rho[:int(r["counts"][b, h, 3])]),
                tail=tail, NT=NT, nb=nb, sw=np.concatenate([np.arange(sp), np.arange(hi, L)]))


def _rows(w, cache, b, g):
    L = int(w.seq_lens[b])
    pages = w.block_table[b, :(L + 15) // 16].long()
    return cache.float()[pages][:, g].reshape(-1, w.d)[:L].double().numpy()


def _tr_nn(E_of, V, fixed, sb, NT, nb):
    t1 = (E_of(sb)[:, None] * V[sb]).sum(0)
    t2 = ((E_of(sb)[:, None] * V[sb]) ** 2).sum(0)
    nf = (E_of(fixed)[:, None] * V[fixed]).sum(0)
    m2 = np.maximum(nb * t2 - t1 * t1, 0.0)
    yc = nb * nf + NT * t1
    return m2.sum(), (yc * yc).sum(), (np.abs(nb * t2) + t1 * t1).sum()


@pytest.mark.parametrize("mk", CASES)
def test_numerator_statistics_match_independent_fp64(mk):
    caught = {}
    for seed in range(3):
        w = mk(seed=seed, v_mean=2.0)
        r = run(w, want_pred=True)
        d = w.d
        G = w.Hq // w.Hkv
        for b in range(w.B):
            K = [_rows(w, w.k_cache, b, g) for g in range(w.Hkv)]
            V = [_rows(w, w.v_cache, b, g) for g in range(w.Hkv)]
            for h in range(w.Hq):
                st = _sets(w, r, b, h)
                if st["NT"] == 0 or st["nb"] == st["NT"]:
                    continue
                g = h // G
                qs = (w.q[b, h].numpy() * np.float32(1.0 / math.sqrt(d))).astype(np.float32).astype(np.float64)
                s = K[g] @ qs
                m = s[np.concatenate([st["fixed"], st["sb"]])].max()

                def E_of(idx, m=m, s=s):
                    return np.exp(s[idx] - m) * 2.0 ** 40
                TR, NN, mag = _tr_nn(E_of, V[g], st["fixed"], st["sb"], st["NT"], st["nb"])
                got_tr, got_nn = (float(x) for x in r["num_stats"][b, h])
                # scores to 2e-6 (the pinned fp32 arithmetic), so each E_i to 1e-5 relative
                assert abs(got_tr - TR) <= 1e-4 * mag + 1e-6 * abs(TR), (seed, b, h, got_tr, TR)
                assert abs(got_nn - NN) <= 1e-4 * NN, (seed, b, h, got_nn, NN)
                wrong = {"T1, T2 over the final sample": _tr_nn(E_of, V[g], st["fixed"], st["S"], st["NT"], st["nb"]),
                         "NF without the top-k": _tr_nn(E_of, V[g], st["sw"], st["sb"], st["NT"], st["nb"]),
                         "base sample in index order": _tr_nn(E_of, V[g], st["fixed"], st["tail"][:st["nb"]],
                                                              st["NT"], st["nb"])}
                for name, (tr2, nn2, _) in wrong.items():
                    if abs(tr2 - TR) > 1e-2 * mag or abs(nn2 - NN) > 1e-2 * NN:
                        caught[name] = caught.get(name, 0) + 1
    for name in ("T1, T2 over the final sample", "NF without the top-k", "base sample in index order"):
        assert caught.get(name, 0) > 0, (name, caught)


def _ceil_budget(val, NT, nb):
    if val >= NT:
        return NT
    return max(math.ceil(val), nb)


@pytest.mark.parametrize("mk", CASES)
def test_budget_is_the_larger_exact_rational_clt_bound(mk):
    checked = by_num = 0
    for seed in range(6):
        w = mk(seed=seed, v_mean=2.5)
        r = run(w)
        z = Fraction(r["z32"])
        eps = Fraction(w.cfg["eps"])
        for b in range(w.B):
            for h in range(w.Hq):
                n_fixed, NT, nb, n, cnt, flags = (int(x) for x in r["counts"][b, h])
                if NT == 0 or nb == NT:
                    continue
                SF, S1, S2hi, S2lo = (int(x) for x in r["stats"][b, h])
                S2 = (S2hi << 64) | S2lo
                TR, NN = (Fraction(float(x)) for x in r["num_stats"][b, h])
                vD = z * z * NT * NT * (nb * S2 - S1 * S1) * nb / ((nb - 1) * eps * eps * (nb * SF + NT * S1) ** 2)
                vN = z * z * NT * NT * TR * nb / ((nb - 1) * eps * eps * NN)
                near = any(abs(v - round(v)) < Fraction(1, 10 ** 9) * max(1, v) for v in (vD, vN))
                if near:
                    continue
                nD = _ceil_budget(vD, NT, nb)
                nN = NT if vN >= NT else math.ceil(vN)
                want = max(nD, nN)
                assert n == want, (seed, b, h, n, nD, nN)
                assert bool(flags & 8) == (nN > nD)
                by_num += int(nN > nD)
                checked += 1
    assert checked > 0 and by_num > 0


def test_zero_mean_values_take_the_whole_tail_and_are_dense():
    w = synthetic.tiny(guarantee=1)  # V ~ N(0, 1): the output nearly cancels
    r = run(w, want_dense=True)
    assert np.all(r["counts"][0, :, 3] == r["counts"][0, :, 1])
    assert np.max(np.abs(r["out"] - r["out_dense"])) < 1e-12
    assert np.max(np.abs(r["lse"] - r["lse_dense"])) < 1e-12


def test_denominator_mode_reports_no_numerator_statistics():
    w = synthetic.tiny(v_mean=2.0)
    r = run(w)
    assert np.all(r["num_stats"] == 0.0)
    assert not np.any(r["counts"][..., 5] & 8)


def test_numerator_eps_delta_rate():
    w = synthetic.tiny(guarantee=1, v_mean=3.0)
    a = w.oracle_arrays()
    eps, delta = w.cfg["eps"], w.cfg["delta"]
    vn = vd = trials = 0
    sparse = 0
    for s in range(1000):
        r = oracle.decode(**a, cfg=dict(w.cfg, seed=s), want_dense=True, want_idx=False)
        ratio = np.exp(r["lse"] - r["lse_dense"])                       # D_hat / D
        num_err = (np.linalg.norm(r["out"] * ratio[..., None] - r["out_dense"], axis=-1)
                   / np.linalg.norm(r["out_dense"], axis=-1))           # |N_hat - N| / |N|
        vn += int((num_err > eps).sum())
        vd += int((np.abs(ratio - 1.0) > eps).sum())
        trials += ratio.size
        sparse += int((r["counts"][..., 3] < r["counts"][..., 1]).sum())
    print("numerator violations %d / %d, denominator %d / %d" % (vn, trials, vd, trials))
    assert vn / trials <= delta and vd / trials <= delta
    assert sparse > trials // 2  # the mode still samples: most budgets stay below the tail
