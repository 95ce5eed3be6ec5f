"""Pins of the oracle's building blocks against things other than itself.

Philox   -> rocRAND's Philox4x32-10 engine (compiled here from its header, run on
            the host) plus a chi-square uniformity check.
pexp     -> math.exp, within 2 fp32 ulp on [-28, 0]; exact at 0.
E_i      -> exp(x) * 2^40 within the fp32 error of pexp; 0 below -28.
pdot     -> exact rational dot (fractions) within the standard fp32 error bound;
            exact on small-integer vectors.
okey     -> order of a sorted list of floats (incl. -0, +0, subnormals).
z        -> scipy.stats.norm.isf(delta / 2), rounded to fp32.
low-rank -> bf16 of an fp64 projection, within one bf16 ulp + fp32 dot error.
"""
import math
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND host reference")
    exe = str(tmp_path_factory.mktemp("rr") / "philox_ref")
    subprocess.run([hipcc, "-O1", "-o", exe, os.path.join(HERE, "helpers", "rocrand_philox_ref.cpp")],
                   check=True, capture_output=True)

    def run(queries):
        inp = "".join("%d %d %d %d\n" % q for q in queries)
        res = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True)
        return [int(x) for x in res.stdout.split()]
    return run


def test_philox_matches_rocrand(rocrand_ref):
    rng = np.random.default_rng(7)
    queries = [(0, 0, 0, 0), (0, 0, 0, 1), (0, 0, 0, 2), (0, 0, 0, 3),
               (2**64 - 1, 7, 5, 131071), (0xDEADBEEF12345678, 63, 7, 4)]
    for _ in range(400):
        queries.append((int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2)),
                        int(rng.integers(0, 64)), int(rng.integers(0, 16)),
                        int(rng.integers(0, 1 << 20))))
    ref = rocrand_ref(queries)
    import ctypes
    lib = oracle._load()
    mine = [int(lib.orc_token_key(ctypes.c_uint64(s), b, g, i)) for (s, b, g, i) in queries]
    assert mine == ref


def test_philox_uniform_chi2():
    # 65536 words, 256 bins: chi2 with 255 dof; reject only far in the tail.
    w = np.concatenate([oracle.token_keys(123, b, 0, 8192) for b in range(8)])
    hist = np.bincount(w >> 24, minlength=256)
    exp = w.size / 256
    chi2 = float(((hist - exp) ** 2 / exp).sum())
    assert 170 < chi2 < 360, chi2
    # distinct keys across (b, g) streams
    a = oracle.token_keys(1, 0, 0, 4096)
    b = oracle.token_keys(1, 0, 1, 4096)
    c = oracle.token_keys(2, 0, 0, 4096)
    assert (a != b).mean() > 0.999 and (a != c).mean() > 0.999


def _ulp32(x):
    x = np.float32(abs(x))
    return float(np.spacing(x))


def test_pexp_accuracy():
    assert oracle.pexp(0.0) == np.float32(1.0)
    xs = np.concatenate([np.linspace(-28, 0, 20001, dtype=np.float32),
                         -np.logspace(-12, 0, 2001).astype(np.float32),
                         np.array([-28.0, -1e-30, -0.34657359, -0.34657360, -10.3972], np.float32)])
    worst = 0.0
    for x in xs:
        got = float(oracle.pexp(x))
        true = math.exp(float(x))
        err = abs(got - true) / _ulp32(true)
        worst = max(worst, err)
    assert worst <= 2.0, worst


def test_fixed_weight():
    assert oracle.fixed_weight(0.0) == 1 << 40
    assert oracle.fixed_weight(-28.0001) == 0
    assert oracle.fixed_weight(-1e9) == 0
    prev = 0
    for x in np.linspace(-28, 0, 4001, dtype=np.float32):
        e = oracle.fixed_weight(x)
        assert e >= prev
        prev = e
        true = math.exp(float(x)) * 2 ** 40
        assert abs(e - true) <= 1 + 3e-7 * true


def test_pdot_error_bound_and_exact_cases():
    rng = np.random.default_rng(3)
    for n in (8, 16, 32, 64, 128, 256):
        for _ in range(50):
            a = rng.standard_normal(n).astype(np.float32)
            b = rng.standard_normal(n).astype(np.float32)
            got = Fraction(float(oracle.pdot(a, b)))
            exact = sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a, b))
            bound = Fraction(n + 1) * Fraction(1, 2 ** 24) * \
                sum(abs(Fraction(float(x)) * Fraction(float(y))) for x, y in zip(a, b))
            assert abs(got - exact) <= bound
        # small integers: every partial sum is exact
        a = rng.integers(-50, 50, n).astype(np.float32)
        b = rng.integers(-50, 50, n).astype(np.float32)
        assert float(oracle.pdot(a, b)) == float(np.dot(a.astype(np.int64), b.astype(np.int64)))
    # each element is used exactly once with its own partner
    a = np.zeros(128, np.float32)
    b = np.zeros(128, np.float32)
    for j in range(128):
        a[:] = 0
        b[:] = 0
        a[j] = 3.0
        b[j] = 5.0
        b[(j + 1) % 128] = 7.0
        assert float(oracle.pdot(a, b)) == 15.0


def test_okey_order():
    vals = np.array([-np.inf, -3e38, -1.5, -1.0, -1e-30, -1e-45, -0.0, 0.0, 1e-45, 1e-30, 0.5,
                     1.0, 2.0, 3e38, np.inf], dtype=np.float32)
    keys = [oracle.okey(v) for v in vals]
    assert keys == sorted(keys) and len(set(keys)) == len(keys)
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000)).astype(np.float32)
    order = np.argsort([oracle.okey(v) for v in x], kind="stable")
    assert np.all(np.diff(x[order].astype(np.float64)) >= 0)


def test_z_matches_scipy():
    from scipy.stats import norm
    for delta in (0.5, 0.2, 0.1, 0.05, 0.02, 0.01, 1e-3, 1e-6):
        assert oracle.z_for_delta(delta) == float(np.float32(norm.isf(delta / 2)))
    assert abs(oracle.z_for_delta(0.05) - 1.959964) < 1e-6


def test_lowrank_projection():
    rng = np.random.default_rng(5)
    K = rng.standard_normal((300, 128)).astype(np.float32)
    P = np.linalg.qr(rng.standard_normal((128, 32)))[0].astype(np.float32)
    kt = oracle.project_rows(K, P)
    as_f = (kt.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = K.astype(np.float64) @ P.astype(np.float64)
    # bf16 keeps 8 significant bits: half an ulp is 2^-8 relative, plus the dot error
    tol = np.abs(ref) * 2.0 ** -8 * 1.01 + 129 * 2.0 ** -24 * (np.abs(K) @ np.abs(P))
    assert np.all(np.abs(as_f - ref) <= tol)
