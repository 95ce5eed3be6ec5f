"""Host emulation of the hash predictor's chunk top-k (integer scores 0..32):
the boundary score found by three probes per sweep on block-wide counts
(33 -> 9 -> 3 -> 1 candidate values), then every key above it and the ties at
it ranked by index through per-thread contiguous token ranges and one block
scan of (above, equal) counts packed in 16-bit halves.  The emulation follows
the kernel's integer arithmetic step by step and must emit exactly the k
best tokens by (score descending, index ascending) -- the top-k definition the
oracle uses -- over random score vectors and the edge cases: k equal to the
chunk, k = 1 with every score equal, the boundary at score 0 and at 32,
unaligned chunk starts, and the largest chunk one block holds (32768 tokens).
"""
import numpy as np
import pytest

NTHR = 1024  # threads of the predictor block


def boundary_score(scores, kp):
    """The search: [slo, shi) with count(>= slo) >= kp > count(>= shi)."""
    slo, shi = 0, 33
    for _ in range(3):
        probes = [slo + (shi - slo) * (j + 1) // 4 for j in range(3)]
        cnt = [int((scores >= m).sum()) for m in probes]
        nlo, nhi = slo, shi
        for m, c in zip(probes, cnt):
            if c >= kp:
                nlo = max(nlo, m)
            else:
                nhi = min(nhi, m)
        slo, shi = nlo, nhi
    return slo


def emulate(scores, kp, o0):
    """Tokens emitted for a chunk whose middle tokens are offsets [o0, o0 + n)
    of the block's key area (o0 need not be a multiple of 4)."""
    n = scores.size
    o1 = o0 + n
    oa = o0 & ~3
    span = (((o1 - oa) + NTHR - 1) // NTHR + 3) & ~3
    key = np.full(o1 + 4 * NTHR + span, -1, dtype=np.int64)
    key[o0:o1] = scores
    th = boundary_score(scores, kp)
    # per-thread counts in 16-bit halves
    packed = np.zeros(NTHR, dtype=np.uint64)
    for t in range(NTHR):
        my0, my1 = oa + t * span, min(oa + t * span + span, o1)
        seg = key[max(my0, o0):max(my1, max(my0, o0))] if my1 > my0 else key[0:0]
        a = int((seg > th).sum())
        e = int((seg == th).sum())
        assert a < 1 << 16 and e < 1 << 16
        packed[t] = a | (e << 16)
    ex = np.concatenate([[0], np.cumsum(packed)[:-1]]).astype(np.uint64)
    tot = int(packed.sum())
    assert (tot & 0xFFFF) < 1 << 16 and (tot >> 16) < 1 << 16  # the halves never carry
    need = kp - (tot & 0xFFFF)
    assert need >= 1
    out = np.full(kp, -1, dtype=np.int64)
    for t in range(NTHR):
        my0, my1 = oa + t * span, min(oa + t * span + span, o1)
        e_ = int(ex[t])
        pos = (e_ & 0xFFFF) + min(e_ >> 16, need)
        tie = e_ >> 16
        for o in range(my0, my1, 4):
            for e in range(4):
                if o + e < o0 or o + e >= o1:
                    continue
                k = key[o + e]
                take = k > th or (k == th and tie < need)
                if k == th:
                    tie += 1
                if take and pos < kp:
                    out[pos] = o + e - o0
                    pos += 1
    return out


def direct(scores, kp):
    idx = np.arange(scores.size)
    return idx[np.lexsort((idx, -scores))][:kp]


def check(scores, kp, o0):
    got = emulate(scores, kp, o0)
    assert np.all(got >= 0), "an output slot was left empty"
    assert sorted(got.tolist()) == sorted(direct(scores, kp).tolist())


@pytest.mark.parametrize("seed", range(12))
def test_random_chunks(seed):
    rng = np.random.default_rng(seed)
    for _ in range(4):
        n = int(rng.integers(1, 9000))
        kind = rng.integers(0, 4)
        if kind == 0:
            s = rng.integers(0, 33, n)
        elif kind == 1:  # concentrated around the middle, as equal-bit counts are
            s = np.clip(rng.binomial(32, 0.5, n), 0, 32)
        elif kind == 2:  # few distinct values
            s = rng.choice(rng.integers(0, 33, 3), n)
        else:
            s = np.clip(rng.binomial(32, 0.8, n), 0, 32)
        kp = int(rng.integers(1, n + 1))
        check(s.astype(np.int64), kp, int(rng.integers(0, 4)) + 4 * int(rng.integers(0, 3)))


def test_edge_cases():
    rng = np.random.default_rng(99)
    s = rng.integers(0, 33, 500)
    check(s, 500, 0)                                   # k covers the chunk
    check(s, 500, 3)
    check(np.full(777, 17), 1, 1)                      # k = 1, all scores equal
    check(np.full(777, 17), 777, 2)
    z = np.zeros(1000, dtype=np.int64)
    z[[5, 900]] = 3
    check(z, 10, 0)                                    # boundary at score 0
    t = np.full(1000, 32)
    t[:7] = 31
    check(t, 400, 1)                                   # boundary at score 32
    check(np.arange(33).repeat(3)[::-1].copy(), 50, 2)  # every score value present
    check(np.array([4]), 1, 3)                         # one token


def test_largest_chunk():
    rng = np.random.default_rng(7)
    s = np.clip(rng.binomial(32, 0.5, 32768), 0, 32)
    check(s, 820, 0)
    check(s, 32768, 0)
