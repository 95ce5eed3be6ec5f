"""Pins of the oracle's signature predictor (CPU only).

The predictor ranks middle tokens by hash signatures, the scoring that
HashAttention uses (named as a top-k method in the edgentiq blog post
"vAttention: a new approach to sparse attention with guaranteed accuracy",
section "Performance and Efficiency"), with untrained random hyperplanes
(Charikar's SimHash) in place of learned hashes: bit j of a signature is set
when the vector's projection on column j of P is positive, and a token's score
is the number of bits its key signature shares with the query's.  These tests
pin that definition against closed forms and fp64 projections computed here
with numpy, never against the oracle's own formula.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import synthetic


def _coordinate_basis(d):
    P = np.zeros((d, 32), np.float32)
    P[np.arange(32), np.arange(32)] = 1.0
    return P


def _bits(mask_rows):
    """Pack a [n, 32] boolean array into uint32 words, bit j from column j."""
    w = np.zeros(mask_rows.shape[0], np.uint64)
    for j in range(32):
        w |= mask_rows[:, j].astype(np.uint64) << np.uint64(j)
    return w.astype(np.uint32)


def test_sign_rows_with_coordinate_hyperplanes():
    # P = the first 32 unit vectors: every projection is one coordinate exactly,
    # so the signature is the sign pattern of k[:, :32]; zeros of either sign
    # are not positive
    rng = np.random.default_rng(3)
    k = rng.standard_normal((40, 64)).astype(np.float32)
    k[0, :] = 0.0
    k[1, :] = -0.0
    k[2, 5] = 0.0
    k[3, 7] = -0.0
    got = oracle.sign_rows(k, _coordinate_basis(64))
    assert np.array_equal(got, _bits(k[:, :32] > 0))
    assert got[0] == 0 and got[1] == 0
    assert not (got[2] >> 5) & 1 and not (got[3] >> 7) & 1


def test_sign_rows_vs_fp64_projection():
    rng = np.random.default_rng(4)
    for d in (64, 128):
        k = rng.standard_normal((300, d)).astype(np.float32)
        P = np.linalg.qr(rng.standard_normal((d, 32)))[0].astype(np.float32)
        got = oracle.sign_rows(k, P)
        ref = k.astype(np.float64) @ P.astype(np.float64)
        band = (d + 2) * 2.0 ** -24 * (np.abs(k) @ np.abs(P)).astype(np.float64)
        sure = np.abs(ref) > band  # signs no fp32 summation order can flip
        assert sure.mean() > 0.99
        gbits = ((got[:, None] >> np.arange(32, dtype=np.uint32)) & 1).astype(bool)
        assert np.array_equal(gbits[sure], (ref > 0)[sure])


def _workload(**kw):
    base = dict(name="sig", B=2, Hq=4, Hkv=2, d=64, seq_lens=(700, 333), kv_dtype="f32",
                recipe="planted", predictor=2, rank=32, sinks=4, window=16, topk_ppm=25000,
                eps=0.05, delta=0.05, seed=11)
    base.update(kw)
    return synthetic.make(**base)


def _head_rows(w, b, g):
    L = int(w.seq_lens[b])
    pages = w.block_table[b, :(L + 15) // 16].long()
    return w.k_cache.float()[pages].permute(1, 0, 2, 3).reshape(w.Hkv, -1, w.d)[g, :L].numpy()


def test_scores_count_the_shared_signature_bits():
    w = _workload()
    a = w.oracle_arrays()
    r = oracle.decode(**a, cfg=w.cfg, want_pred=True)
    P = a["proj"].astype(np.float64)
    scale = np.float32(1.0 / math.sqrt(w.d))
    G = w.Hq // w.Hkv
    checked = 0
    for b in range(w.B):
        L = int(w.seq_lens[b])
        for h in range(w.Hq):
            K = _head_rows(w, b, h // G).astype(np.float64)
            qs = (a["q"][b, h] * scale).astype(np.float32).astype(np.float64)
            qp, kp = qs @ P, K @ P
            qband = (w.d + 2) * 2.0 ** -24 * (np.abs(qs) @ np.abs(P))
            kband = (w.d + 2) * 2.0 ** -24 * (np.abs(K) @ np.abs(P))
            sure = np.all(np.abs(kp) > kband, axis=1) & bool(np.all(np.abs(qp) > qband))
            ref = ((kp > 0) == (qp > 0)[None, :]).sum(axis=1).astype(np.float32)
            pred = r["pred"][b, h, :L]
            mid = ~np.isnan(pred)
            assert mid.sum() == L - min(4, L) - min(16, L - min(4, L))
            m = mid & sure
            assert np.array_equal(pred[m], ref[m])
            checked += int(m.sum())
            # the fixed set holds the k best middle tokens, the lower index
            # first among equal scores (a complete ranking when every sign is sure)
            if np.all(sure[mid]):
                k = r["counts"][b, h, 0] - min(4, L) - min(16, L - min(4, L))
                midx = np.nonzero(mid)[0]
                order = sorted(midx.tolist(), key=lambda i: (-ref[i], i))
                I = set(r["idx"][b, h][r["idx"][b, h] >= 0].tolist())
                assert set(order[:k]) <= I
    assert checked > 0.95 * sum(int(x) for x in w.seq_lens) * G


def test_a_key_along_the_query_scores_every_bit():
    w = _workload(B=1, Hq=2, Hkv=1, seq_lens=(500,), recipe="normal")
    a = w.oracle_arrays()
    qdir = a["q"][0, 0] / np.linalg.norm(a["q"][0, 0])
    # token 100 points along head 0's query, token 200 against it
    pg100, pg200 = a["block_table"][0, 100 // 16], a["block_table"][0, 200 // 16]
    a["k_cache"][pg100, 0, 100 % 16] = (3.0 * qdir).astype(np.float32)
    a["k_cache"][pg200, 0, 200 % 16] = (-3.0 * qdir).astype(np.float32)
    r = oracle.decode(**a, cfg=w.cfg, want_pred=True)
    assert r["pred"][0, 0, 100] == 32.0
    assert r["pred"][0, 0, 200] == 0.0
    assert 100 in set(r["idx"][0, 0].tolist())


def test_without_topk_the_predictor_does_not_matter():
    # k = 0: the fixed set is sinks + window only, so the signature predictor
    # and the exact one give the same decode
    w = _workload(topk_abs=0)
    a = w.oracle_arrays()
    sig = oracle.decode(**a, cfg=w.cfg)
    ex = oracle.decode(**dict(a, proj=None), cfg=dict(w.cfg, predictor=0, rank=0))
    for key in ("idx", "counts", "stats", "out", "lse"):
        assert np.array_equal(sig[key], ex[key]), key


def test_each_group_signs_with_its_own_hyperplanes():
    w = _workload(proj_per_head=True)
    a = w.oracle_arrays()
    assert a["proj"].shape == (w.Hkv, w.d, 32)
    full = oracle.decode(**a, cfg=w.cfg)
    G = w.Hq // w.Hkv
    for g in range(w.Hkv):
        own = oracle.decode(**dict(a, proj=a["proj"][g]), cfg=w.cfg, groups=[(b, g) for b in range(w.B)])
        hs = slice(g * G, (g + 1) * G)
        for key in ("idx", "counts", "stats", "out", "lse"):
            assert np.array_equal(full[key][:, hs], own[key][:, hs]), (g, key)


def test_signature_predictor_rejects_other_widths():
    w = _workload()
    with pytest.raises(ValueError):
        oracle.decode(**w.oracle_arrays(), cfg=dict(w.cfg, rank=16))
