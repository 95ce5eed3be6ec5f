"""Pin of the oracle's exact fixed-point statistics SF, S1, S2 (and the
maximum m they are taken against), independent of the oracle's own code.

The definition (edgentiq blog post "vAttention: a new approach to sparse
attention with guaranteed accuracy", section "How vAttention Works": the
denominator is estimated from the deterministic set plus a sample of the
tail): with exact scores s_i = q_s . K_i over the fixed set I_f (sinks, window,
top-k) and the base sample S_b (the first n_b tail tokens in (Philox word,
index) order), m = max of s_i over I_f and S_b, E_i = exp(s_i - m) * 2^40, and

    SF = sum over I_f of E_i,   S1 = sum over S_b of E_i,   S2 = sum over S_b of E_i^2.

This test rebuilds I_f and S_b from scratch (sinks and window from the
sequence length, the top-k by numpy lexsort on the oracle's predictor scores,
which are pinned against fp64 elsewhere; the tail order by lexsort on the
Philox words, which are pinned against rocRAND's engine), recomputes every s_i
in fp64 from q_s and the cached keys, and compares the oracle's integers with
the fp64 sums within the error bound of the pinned fp32 arithmetic: the
blocked dot product, the subtraction of m, the fp32 exp (2 ulp) and the
truncation to integers.  Plausible mistakes (m over I_f only, SF without the
top-k, S1 and S2 over the final sample instead of the base sample, the base
sample taken in index order) each move at least one head's statistic far
outside that bound; the test asserts this too, so it is known to catch them.
"""
import math

import numpy as np
import pytest

import oracle
import synthetic

U = 2.0 ** -24  # fp32 unit roundoff


def _keys(w, b, g):
    L = int(w.seq_lens[b])
    pages = w.block_table[b, :(L + 15) // 16].long()
    return w.k_cache.float()[pages][:, g].reshape(-1, w.d)[:L].double().numpy()


def _reference(w, r, b, h):
    """fp64 statistics of head (b, h) from independently rebuilt sets, and the
    error bound of each; None for a head with no tail decision."""
    cfg = w.cfg
    d = w.d
    G = w.Hq // w.Hkv
    g = h // G
    L = int(w.seq_lens[b])
    if L == 0:
        return None
    sp = min(cfg["sinks"], L)
    wp = min(cfg["window"], L - sp)
    lo, hi = sp, L - wp
    k = cfg["topk_abs"] if cfg["topk_abs"] >= 0 else -(-L * cfg["topk_ppm"] // 10 ** 6)
    k = min(k, hi - lo)
    mid = np.arange(lo, hi)
    pred = r["pred"][b, h, lo:hi].astype(np.float64)
    T = mid[np.lexsort((mid, -pred))[:k]]
    fixed = np.concatenate([np.arange(sp), np.arange(hi, L), T]).astype(np.int64)
    tail = np.setdiff1d(mid, T)
    NT = tail.size
    nb = 0 if NT == 0 else min(NT, max(2, -(-NT * cfg["base_ppm"] // 10 ** 6)))
    u = oracle.token_keys(cfg["seed"], b, g, L)[tail] if NT else np.zeros(0, np.uint32)
    rho = tail[np.lexsort((tail, u))] if NT else tail
    Sb = rho[:nb]
    n = int(r["counts"][b, h, 3])
    S = rho[:n]
    K = _keys(w, b, g)
    qs = (w.q[b, h].numpy() * np.float32(1.0 / math.sqrt(d))).astype(np.float32).astype(np.float64)
    s = K @ qs                                    # exact dot of the fp32 operands
    mag = np.abs(K) @ np.abs(qs)
    depth = 8 + int(math.log2(d // 8))           # fma chain of 8, then the pairwise tree
    err = 1.01 * depth * U * mag                  # |fl32 pdot - s|
    both = np.concatenate([fixed, Sb])
    m = s[both].max()
    err_m = err[both].max()

    def sums(idx, m_, err_m_):
        x = s[idx] - m_
        E = np.exp(x) * 2.0 ** 40
        dx = err[idx] + err_m_ + U * np.abs(x)   # score errors and the fp32 subtraction
        rel = np.expm1(dx) + 3 * U                # exp's argument error, then 2 ulp of fp32 exp
        tol = E * rel + 1.0                       # plus the truncation to an integer
        return E, tol

    Ef, tf = sums(fixed, m, err_m)
    Eb, tb = sums(Sb, m, err_m)
    ref = dict(SF=(Ef.sum(), tf.sum()), S1=(Eb.sum(), tb.sum()),
               S2=((Eb ** 2).sum(), ((Eb + tb) ** 2 - Eb ** 2).sum() + 1.0))
    # plausible mistakes, evaluated the same way
    m_if = s[fixed].max() if fixed.size else m
    Ef_wrong_m, _ = sums(fixed, m_if, 0.0)
    Eb_wrong_m, _ = sums(Sb, m_if, 0.0)
    sw = np.concatenate([np.arange(sp), np.arange(hi, L)]).astype(np.int64)
    Esw, _ = sums(sw, m, 0.0)
    ES, _ = sums(S, m, 0.0)
    Sb_index_order = np.sort(tail)[:nb]
    Ebi, _ = sums(Sb_index_order, m, 0.0)
    wrong = {"m over I_f only": dict(SF=Ef_wrong_m.sum(), S1=Eb_wrong_m.sum()),
             "SF without top-k": dict(SF=Esw.sum()),
             "S1, S2 over the final sample": dict(S1=ES.sum(), S2=(ES ** 2).sum()),
             "base sample in index order": dict(S1=Ebi.sum(), S2=(Ebi ** 2).sum())}
    return ref, wrong


CASES = {
    # exact-score top-k, fp32 keys, planted heavy hitters (the tiny workload)
    "tiny": lambda s: synthetic.tiny(seed=s),
    # no top-k and a 30% base sample: the maximum often lies in the base sample
    "max_in_base_sample": lambda s: synthetic.make(
        name="max_in_base", B=1, Hq=4, Hkv=2, d=64, seq_lens=(900,), kv_dtype="f32", recipe="planted",
        predictor=0, sinks=4, window=4, topk_abs=0, base_ppm=300000, seed=s, data_seed=61),
    # low-rank top-k over bf16 keys, small eps: final samples larger than the base sample
    "lowrank_bf16_small_eps": lambda s: synthetic.make(
        name="lowrank_small_eps", B=2, Hq=8, Hkv=2, d=128, seq_lens=(1500, 777), kv_dtype="bf16",
        recipe="outlier", predictor=1, rank=32, sinks=16, window=16, topk_ppm=25000, eps=0.01,
        seed=s, data_seed=62),
    # hash-signature top-k (integer scores with ties)
    "hash_bf16": lambda s: synthetic.make(
        name="hash_stats", B=1, Hq=4, Hkv=1, d=128, seq_lens=(1200,), kv_dtype="bf16", recipe="planted",
        predictor=2, rank=32, sinks=8, window=8, topk_ppm=20000, seed=s, data_seed=63),
}


def _check_case(name):
    """Asserts the oracle's statistics for every head of the case; returns how
    many heads each plausible mistake would have moved outside the bound."""
    caught = {}
    heads = 0
    for seed in range(3):
        w = CASES[name](seed)
        r = oracle.decode(**w.oracle_arrays(), cfg=w.cfg, want_pred=True)
        for b in range(w.B):
            for h in range(w.Hq):
                got = r["stats"][b, h]
                rr = _reference(w, r, b, h)
                if rr is None:
                    continue
                ref, wrong = rr
                vals = dict(SF=int(got[0]), S1=int(got[1]), S2=(int(got[2]) << 64) | int(got[3]))
                for key in ("SF", "S1", "S2"):
                    want, tol = ref[key]
                    assert abs(vals[key] - want) <= tol, (name, seed, b, h, key, vals[key], want, tol)
                heads += 1
                for mistake, alt in wrong.items():
                    for key, v in alt.items():
                        if abs(v - ref[key][0]) > 4 * ref[key][1]:
                            caught.setdefault(mistake, 0)
                            caught[mistake] += 1
    assert heads > 0
    return caught


@pytest.mark.parametrize("name", list(CASES))
def test_statistics_match_independent_fp64(name):
    _check_case(name)


def test_each_plausible_mistake_is_caught():
    """Every mistake listed in the module docstring moves some head's statistic
    by more than four times the tolerance in at least one of the cases."""
    caught = {}
    for name in CASES:
        for k, v in _check_case(name).items():
            caught[k] = caught.get(k, 0) + v
    for mistake in ("m over I_f only", "SF without top-k", "S1, S2 over the final sample",
                    "base sample in index order"):
        assert caught.get(mistake, 0) > 0, (mistake, caught)
