"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: the tiny
workload, degenerate sequences (empty, one token, tails of one and two tokens,
k covering the middle), a ragged bf16 low-rank case and a hash-signature case
run in a child process that loads the sanitized build; any out-of-bounds
access, leak-free misuse or undefined operation aborts it.  Its results must be
bit-identical to the plain build's."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, %(root)r)
import numpy as np
import oracle, synthetic
from tests.test_oracle_sanitized import workloads
res = {}
for name, w in workloads():
    r = oracle.decode(**w.oracle_arrays(), cfg=w.cfg, want_dense=True, want_pred=True, nthreads=4)
    for k, v in r.items():
        if isinstance(v, np.ndarray):
            res[name + "/" + k] = v
np.savez(%(out)r, **res)
print("sanitized oracle ok", flush=True)
"""


def workloads():
    yield "tiny", synthetic.tiny(seed=3)
    yield "degenerate", synthetic.make(B=5, Hq=2, Hkv=1, d=64, seq_lens=(0, 1, 13, 14, 50), kv_dtype="f32",
                                       predictor=0, sinks=2, window=2, topk_abs=8)
    yield "k_covers_middle", synthetic.make(B=1, Hq=2, Hkv=1, d=64, seq_lens=(30,), kv_dtype="f32",
                                            predictor=0, sinks=2, window=2, topk_abs=100)
    yield "ragged_lowrank", synthetic.make(B=3, Hq=8, Hkv=2, d=128, seq_lens=(700, 33, 257), kv_dtype="bf16",
                                           recipe="outlier", predictor=1, rank=32, sinks=16, window=16,
                                           topk_ppm=25000, shuffle=True, data_seed=71)
    yield "hash", synthetic.make(B=1, Hq=4, Hkv=2, d=64, seq_lens=(600,), kv_dtype="bf16", recipe="planted",
                                 predictor=2, rank=32, sinks=4, window=8, topk_ppm=20000, data_seed=72)


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_oracle_clean_under_asan_ubsan(tmp_path):
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    out = str(tmp_path / "res.npz")
    env = dict(os.environ, VATTN_ORACLE_LIB=lib, LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([sys.executable, "-c", CHILD % dict(root=ROOT, out=out)], env=env, capture_output=True,
                       text=True, timeout=600, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-4000:]
    assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr, p.stderr[-4000:]
    got = np.load(out)
    for name, w in workloads():
        r = oracle.decode(**w.oracle_arrays(), cfg=w.cfg, want_dense=True, want_pred=True, nthreads=4)
        for k, v in r.items():
            if isinstance(v, np.ndarray):
                assert np.array_equal(got[name + "/" + k], v, equal_nan=True), (name, k)


def test_oracle_refuses_non_finite_inputs():
    w = synthetic.tiny()
    a = w.oracle_arrays()
    for key, where in (("q", (0, 1, 3)), ("k_cache", (5, 2, 3, 7)), ("v_cache", (40, 0, 0, 0))):
        bad = dict(a)
        arr = a[key].copy()
        arr[where] = np.nan if key != "v_cache" else np.inf
        bad[key] = arr
        with pytest.raises(ValueError, match="non-finite"):
            oracle.decode(**bad, cfg=w.cfg)
    # a non-finite key row beyond every sequence's end is never read: accepted
    w2 = synthetic.make(B=1, Hq=2, Hkv=1, d=64, seq_lens=(20,), kv_dtype="f32", predictor=0, sinks=2, window=2,
                        topk_abs=4)
    a2 = w2.oracle_arrays()
    k2 = a2["k_cache"].copy()
    k2[1, 0, 15] = np.nan  # token 31 of page 1; the sequence has 20 tokens
    oracle.decode(**dict(a2, k_cache=k2), cfg=w2.cfg)
    wl = synthetic.make(B=1, Hq=2, Hkv=1, d=64, seq_lens=(64,), kv_dtype="f32", predictor=1, rank=16,
                        sinks=2, window=2, topk_abs=4)
    al = wl.oracle_arrays()
    p = al["proj"].copy()
    p[3, 2] = np.inf
    with pytest.raises(ValueError, match="non-finite"):
        oracle.decode(**dict(al, proj=p), cfg=wl.cfg)
