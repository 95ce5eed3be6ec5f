"""CPU oracle for the verified sparse-attention decode step (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The HIP library never
imports, links or runs anything here, and nothing here imports the HIP library.

The arithmetic lives in ``vattn_oracle.c`` (plain C, fp64 outputs, pinned fp32
steps for every discrete decision).  This module only compiles it with gcc,
loads it and marshals numpy arrays.  One value is computed here rather than in
C: z = Phi^-1(1 - delta/2), from the standard library's inverse normal CDF,
rounded to fp32 (the failure-probability reading of (eps, delta) in the
edgentiq blog post "vAttention: a new approach to sparse attention with
guaranteed accuracy", section "Introducing vAttention").

Parity status per function: all functions are pinned by the CPU tests
(tests/test_oracle_*.py); nothing here is "parity unpinned".
"""
from __future__ import annotations

import ctypes as C
import os
import statistics
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vattn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# a separately built copy (the sanitizer build of the tests) may be named here
_LIB_OVERRIDE = os.environ.get("VATTN_ORACLE_LIB")
_lock = threading.Lock()
_lib = None


_CFLAGS = ["-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc"] + _CFLAGS + ["-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(path: str) -> str:
    """The same oracle under AddressSanitizer and UndefinedBehaviorSanitizer
    (every report fatal), for the tests; a process loading it must preload
    gcc's libasan (see tests/test_oracle_sanitized.py)."""
    subprocess.run(["gcc"] + _CFLAGS + ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                                        "-fno-sanitize-recover=all", "-o", path, _SRC, "-lm"], check=True)
    return path


class OrcCfg(C.Structure):
    _fields_ = [("sinks", C.c_int32), ("window", C.c_int32), ("topk_abs", C.c_int32),
                ("topk_ppm", C.c_int32), ("base_ppm", C.c_int32), ("force_budget", C.c_int32),
                ("predictor", C.c_int32), ("rank", C.c_int32), ("eps", C.c_double),
                ("delta", C.c_double), ("z32", C.c_double), ("seed", C.c_uint64), ("guarantee", C.c_int32)]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if _LIB_OVERRIDE:
                lib = C.CDLL(_LIB_OVERRIDE)
            else:
                if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                    build(force=True)
                lib = C.CDLL(_LIB)
            P = C.c_void_p
            lib.orc_decode.restype = C.c_int
            lib.orc_decode.argtypes = [C.POINTER(OrcCfg)] + [C.c_int] * 7 + [P] * 4 + [C.c_int] + \
                [P] * 3 + [C.c_int, C.c_int] + [P] * 5 + [C.c_int] + [P] * 4
            lib.orc_dense.restype = C.c_int
            lib.orc_dense.argtypes = [C.c_int] * 6 + [P] * 6 + [C.c_int, C.c_int, P, P]
            lib.orc_pdot.restype = C.c_float
            lib.orc_pdot.argtypes = [P, C.c_int, P, C.c_int, C.c_int]
            lib.orc_pexp.restype = C.c_float
            lib.orc_pexp.argtypes = [C.c_float]
            lib.orc_fixed_weight.restype = C.c_uint64
            lib.orc_fixed_weight.argtypes = [C.c_float]
            lib.orc_okey.restype = C.c_uint32
            lib.orc_okey.argtypes = [C.c_float]
            lib.orc_philox4x32_10.restype = None
            lib.orc_philox4x32_10.argtypes = [P, P, P]
            lib.orc_token_key.restype = C.c_uint32
            lib.orc_token_key.argtypes = [C.c_uint64, C.c_int, C.c_int, C.c_int]
            lib.orc_project_rows.restype = None
            lib.orc_project_rows.argtypes = [P, C.c_int64, C.c_int, P, C.c_int, P]
            lib.orc_sign_rows.restype = None
            lib.orc_sign_rows.argtypes = [P, C.c_int64, C.c_int, P, P]
            lib.orc_key_gram.restype = C.c_int
            lib.orc_key_gram.argtypes = [C.c_int] * 5 + [P] * 5
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def z_for_delta(delta: float) -> float:
    """z = Phi^-1(1 - delta/2) in fp64, rounded to fp32 (returned as a Python float)."""
    z = statistics.NormalDist().inv_cdf(1.0 - delta / 2.0)
    return float(np.float32(z))


# ---------------------------------------------------------------------------
# Pinned primitives (exported for the pins)
# ---------------------------------------------------------------------------

def pdot(a, b) -> np.float32:
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    assert a.shape == b.shape and a.ndim == 1
    return np.float32(_load().orc_pdot(_ptr(a), 1, _ptr(b), 1, a.shape[0]))


def pexp(x) -> np.float32:
    return np.float32(_load().orc_pexp(float(np.float32(x))))


def fixed_weight(x) -> int:
    return int(_load().orc_fixed_weight(float(np.float32(x))))


def okey(x) -> int:
    return int(_load().orc_okey(float(np.float32(x))))


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    o = np.zeros(4, dtype=np.uint32)
    _load().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(o))
    return o


def token_keys(seed: int, b: int, g: int, n: int) -> np.ndarray:
    lib = _load()
    return np.array([lib.orc_token_key(seed, b, g, i) for i in range(n)], dtype=np.uint32)


def project_rows(k_rows: np.ndarray, proj: np.ndarray) -> np.ndarray:
    """Low-rank keys as bf16 bit patterns: bf16(pdot(K_i, P[:, j]))."""
    k_rows = np.ascontiguousarray(k_rows, dtype=np.float32)
    proj = np.ascontiguousarray(proj, dtype=np.float32)
    n, d = k_rows.shape
    r = proj.shape[1]
    out = np.zeros((n, r), dtype=np.uint16)
    _load().orc_project_rows(_ptr(k_rows), n, d, _ptr(proj), r, _ptr(out))
    return out


def sign_rows(k_rows: np.ndarray, proj: np.ndarray) -> np.ndarray:
    """Key signatures: bit j set when pdot(K_i, P[:, j]) > 0, P of shape [d, 32]."""
    k_rows = np.ascontiguousarray(k_rows, dtype=np.float32)
    proj = np.ascontiguousarray(proj, dtype=np.float32)
    n, d = k_rows.shape
    assert proj.shape == (d, 32)
    out = np.zeros(n, dtype=np.uint32)
    _load().orc_sign_rows(_ptr(k_rows), n, d, _ptr(proj), _ptr(out))
    return out


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------

def decode(*, q, k_cache, v_cache, block_table, seq_lens, cfg: dict, proj=None,
           max_seq_len=None, groups=None, nthreads=1, want_idx=True, want_dense=False,
           want_pred=False):
    """Run the oracle.

    q: [B,Hq,d] float32.  k_cache/v_cache: [num_blocks,Hkv,16,d] float32, or
    uint16 holding bf16 bit patterns.  block_table [B,max_blocks] int32,
    seq_lens [B] int32, proj [d,r] float32 (low-rank or signature predictor; or [Hkv,d,r],
    one basis per KV head) or None.
    cfg keys: sinks, window, topk_abs, topk_ppm, base_ppm, force_budget,
    predictor (0 exact, 1 low-rank, 2 32-bit signatures with rank 32), rank, eps, delta, seed,
    guarantee (0 the denominator, default; 1 the denominator and the numerator).
    groups: iterable of (b, g) to evaluate (default all).  Returns a dict of
    numpy arrays (rows of groups not evaluated are zero / -1).
    """
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, Hq, d = q.shape
    kv_bf16 = k_cache.dtype == np.uint16
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    assert v_cache.dtype == k_cache.dtype
    Hkv = k_cache.shape[1]
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    max_blocks = block_table.shape[1]
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max()) if seq_lens.size else 0
    max_seq_len = max(int(max_seq_len), 1)
    proj_heads = 1
    if proj is not None:
        proj = np.ascontiguousarray(proj, dtype=np.float32)
        if proj.ndim == 3:  # one basis per KV head
            assert proj.shape[0] == Hkv
            proj_heads = Hkv
    c = OrcCfg(int(cfg["sinks"]), int(cfg["window"]), int(cfg.get("topk_abs", -1)),
               int(cfg.get("topk_ppm", 0)), int(cfg.get("base_ppm", 50000)),
               int(cfg.get("force_budget", -1)), int(cfg["predictor"]), int(cfg.get("rank", 0)),
               float(cfg["eps"]), float(cfg["delta"]), z_for_delta(float(cfg["delta"])),
               int(cfg["seed"]) & 0xFFFFFFFFFFFFFFFF, int(cfg.get("guarantee", 0)))
    out = np.zeros((B, Hq, d), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    lse_dense = np.zeros((B, Hq), dtype=np.float64) if want_dense else None
    out_dense = np.zeros((B, Hq, d), dtype=np.float64) if want_dense else None
    idx = np.full((B, Hq, max_seq_len), -1, dtype=np.int32) if want_idx else None
    counts = np.zeros((B, Hq, 6), dtype=np.int32)
    stats = np.zeros((B, Hq, 4), dtype=np.uint64)
    pred = np.full((B, Hq, max_seq_len), np.nan, dtype=np.float32) if want_pred else None
    nstats = np.zeros((B, Hq, 2), dtype=np.float64)
    if groups is None:
        garr, ng = None, 0
    else:
        garr = np.array([b * Hkv + g for (b, g) in groups], dtype=np.int32)
        ng = garr.shape[0]
    rc = _load().orc_decode(C.byref(c), B, Hq, Hkv, d, max_blocks, int(kv_bf16), max_seq_len,
                            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(proj), proj_heads, _ptr(block_table),
                            _ptr(seq_lens), _ptr(garr), ng, int(nthreads), _ptr(out), _ptr(lse),
                            _ptr(lse_dense), _ptr(out_dense), _ptr(idx), max_seq_len,
                            _ptr(counts), _ptr(stats), _ptr(pred), _ptr(nstats))
    if rc == 5:
        raise ValueError("oracle refused a non-finite input (q, the basis, or a cached K or V row)")
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)
    res = dict(out=out, lse=lse, counts=counts, stats=stats, z32=c.z32, num_stats=nstats)
    if want_idx:
        res["idx"] = idx
    if want_dense:
        res["lse_dense"] = lse_dense
        res["out_dense"] = out_dense
    if want_pred:
        res["pred"] = pred
    return res


def dense(*, q, k_cache, v_cache, block_table, seq_lens, groups=None, nthreads=1, want_out=True, **_):
    """Dense fp64 softmax attention over every cached token of every head (the
    exact target): returns dict(lse_dense [B, Hq], out_dense [B, Hq, d] or None).
    Takes the same arrays as decode (extra keys such as proj are ignored)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, Hq, d = q.shape
    kv_bf16 = k_cache.dtype == np.uint16
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    Hkv = k_cache.shape[1]
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    lse = np.zeros((B, Hq), dtype=np.float64)
    out = np.zeros((B, Hq, d), dtype=np.float64) if want_out else None
    if groups is None:
        garr, ng = None, 0
    else:
        garr = np.array([b * Hkv + g for (b, g) in groups], dtype=np.int32)
        ng = garr.shape[0]
    rc = _load().orc_dense(B, Hq, Hkv, d, block_table.shape[1], int(kv_bf16), _ptr(q), _ptr(k_cache),
                           _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), _ptr(garr), ng, int(nthreads),
                           _ptr(lse), _ptr(out))
    if rc == 5:
        raise ValueError("oracle refused a non-finite input (q, or a cached K or V row)")
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)
    return dict(lse_dense=lse, out_dense=out)


def key_gram(*, k_cache, block_table, seq_lens, **_):
    """Per KV head, sum over every cached token of K K^T in fp64 ([Hkv, d, d]),
    and the same sums of |K| |K|^T (the scale of an fp32 accumulation's error).
    Takes the same arrays as decode (extra keys are ignored)."""
    k_cache = np.ascontiguousarray(k_cache)
    kv_bf16 = k_cache.dtype == np.uint16
    _, Hkv, _, d = k_cache.shape
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B, max_blocks = block_table.shape
    gram = np.zeros((Hkv, d, d), dtype=np.float64)
    absg = np.zeros((Hkv, d, d), dtype=np.float64)
    rc = _load().orc_key_gram(B, Hkv, d, max_blocks, int(kv_bf16), _ptr(k_cache), _ptr(block_table),
                              _ptr(seq_lens), _ptr(gram), _ptr(absg))
    if rc == 5:
        raise ValueError("oracle refused a non-finite cached key")
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)
    return gram, absg
