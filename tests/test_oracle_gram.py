"""Pins of the oracle's key second moments (oracle.key_gram), the matrix whose
leading eigenvectors give a per-KV-head PCA predictor basis (pith.science page
"Loki: Low-rank Keys for Efficient Sparse Attention", abstract: keys lie near a
low-dimensional subspace).  Every case is a closed form with small-integer keys,
so the fp64 sums are exact and compared with ==."""
import numpy as np
import pytest

import oracle

PAGE = 16


def paged(rows, seq_lens, shuffle_seed=None, fill=None, dtype=np.float32):
    """rows[b]: [Hkv, L_b, d] keys -> (k_cache [nblk, Hkv, 16, d], block_table, seq_lens).
    Unused slots (past each sequence's end) hold `fill` (default 0)."""
    B = len(rows)
    Hkv, _, d = rows[0].shape
    mb = max(1, max((r.shape[1] + PAGE - 1) // PAGE for r in rows))
    nblk = B * mb
    cache = np.full((nblk, Hkv, PAGE, d), 0.0 if fill is None else fill, dtype=np.float32)
    perm = np.arange(nblk) if shuffle_seed is None else np.random.default_rng(shuffle_seed).permutation(nblk)
    bt = np.full((B, mb), -1, dtype=np.int32)
    for b, r in enumerate(rows):
        L = r.shape[1]
        for p in range(mb):
            page = int(perm[b * mb + p])
            bt[b, p] = page
            for t in range(PAGE):
                i = p * PAGE + t
                if i < L:
                    cache[page, :, t, :] = r[:, i, :]
    if dtype == np.uint16:  # bf16 bit patterns (the test keys are exact in bf16)
        c32 = cache.view(np.uint32)
        assert np.all((c32 & 0xFFFF) == 0)
        cache = (c32 >> 16).astype(np.uint16)
    return cache, bt, np.array([r.shape[1] for r in rows], dtype=np.int32)


def test_one_hot_keys_give_a_diagonal():
    """Key t of head g = c_t e_{j_t}: the Gram is diag(sum of c_t^2 per channel),
    each head with its own channels (a head or token index mixed up, or a token
    dropped, moves an entry)."""
    rng = np.random.default_rng(1)
    Hkv, d, L = 3, 16, 77
    keys = np.zeros((Hkv, L, d), dtype=np.float32)
    want = np.zeros((Hkv, d, d))
    for g in range(Hkv):
        for t in range(L):
            j = int(rng.integers(0, d // 2)) + (d // 2 if g % 2 else 0)
            c = float(rng.integers(-5, 6))
            keys[g, t, j] = c
            want[g, j, j] += c * c
    k, bt, sl = paged([keys], [L])
    gram, absg = oracle.key_gram(k_cache=k, block_table=bt, seq_lens=sl)
    assert np.array_equal(gram, want)
    assert np.array_equal(absg, want)


def test_rank_two_keys_closed_form():
    """K_t = a_t u + b_t v: Gram = (sum a^2) u u^T + (sum a b)(u v^T + v u^T) + (sum b^2) v v^T,
    over two sequences of different lengths."""
    rng = np.random.default_rng(2)
    d = 32
    u = rng.integers(-2, 3, size=d).astype(np.float32)
    v = rng.integers(-2, 3, size=d).astype(np.float32)
    rows, A2, AB, B2 = [], 0.0, 0.0, 0.0
    for L in (45, 130):
        a = rng.integers(-3, 4, size=L).astype(np.float32)
        bb = rng.integers(-3, 4, size=L).astype(np.float32)
        rows.append((a[:, None] * u[None, :] + bb[:, None] * v[None, :])[None])
        A2 += float(a @ a); AB += float(a @ bb); B2 += float(bb @ bb)
    want = A2 * np.outer(u, u) + AB * (np.outer(u, v) + np.outer(v, u)) + B2 * np.outer(v, v)
    k, bt, sl = paged(rows, [45, 130])
    gram, absg = oracle.key_gram(k_cache=k, block_table=bt, seq_lens=sl)
    assert np.array_equal(gram[0], want)
    assert np.all(absg[0] >= np.abs(gram[0]))


def test_paging_and_sequence_ends():
    """Physical page order does not matter, and slots past a sequence's end
    (here holding 1e6) are not read; a sequence of length 0 adds nothing."""
    rng = np.random.default_rng(3)
    Hkv, d = 2, 8
    rows = [rng.integers(-4, 5, size=(Hkv, L, d)).astype(np.float32) for L in (33, 0, 50)]
    k1, bt1, sl = paged(rows, None)
    k2, bt2, _ = paged(rows, None, shuffle_seed=7, fill=1e6)
    g1, _ = oracle.key_gram(k_cache=k1, block_table=bt1, seq_lens=sl)
    g2, _ = oracle.key_gram(k_cache=k2, block_table=bt2, seq_lens=sl)
    assert np.array_equal(g1, g2)
    want = sum(np.einsum("gti,gtj->gij", r.astype(np.float64), r.astype(np.float64)) for r in rows)
    assert np.array_equal(g1, want)  # small integers: every sum exact


def test_bf16_cache_reads_the_same_values():
    rng = np.random.default_rng(4)
    rows = [rng.integers(-8, 9, size=(2, 40, 16)).astype(np.float32)]
    kf, bt, sl = paged(rows, None)
    kb, _, _ = paged(rows, None, dtype=np.uint16)
    gf, _ = oracle.key_gram(k_cache=kf, block_table=bt, seq_lens=sl)
    gb, _ = oracle.key_gram(k_cache=kb, block_table=bt, seq_lens=sl)
    assert np.array_equal(gf, gb)


def test_non_finite_key_refused():
    rows = [np.ones((1, 20, 8), dtype=np.float32)]
    rows[0][0, 19, 3] = np.inf
    k, bt, sl = paged(rows, None)
    with pytest.raises(ValueError):
        oracle.key_gram(k_cache=k, block_table=bt, seq_lens=sl)
