"""Pins of the oracle's scalar pieces against what the pages and libraries fix.

Element grid and steps: OptiTrain-FP4 README enumeration, Full-Stack FP4 sec. 2
and Appendix 7.  E4M3 / bfloat16: torch's CPU conversions (library routines).
Philox4x32-10: rocRAND's host implementation (library routine).  Hadamard:
scipy.linalg.hadamard and the Walsh-Hadamard recursion of the README.
"""
import os
import shutil
import struct
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


def nextafter32(x, d):
    return float(np.nextafter(np.float32(x), np.float32(d)))


def read_grid():
    vals, steps = [], None
    with open(os.path.join(GOLDEN, "e2m1_grid.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("steps"):
                steps = [float(t) for t in line.split()[1:]]
            else:
                e, m, v = line.split()
                vals.append((int(e), int(m), float(v)))
    return vals, steps


# ------------------------------------------------------------------ E2M1
def test_e2m1_decode_all_16_codes(oracle):
    grid, _ = read_grid()
    assert len(grid) == 8
    for e, m, v in grid:
        code = (e << 1) | m
        assert oracle.e2m1_value(code) == v
        neg = oracle.e2m1_value(8 | code)
        assert neg == -v and (v != 0.0 or np.signbit(neg))


def test_e2m1_steps_match_appendix7(oracle):
    _, steps = read_grid()
    pos = [oracle.e2m1_value(c) for c in range(8)]
    assert [b - a for a, b in zip(pos, pos[1:])] == steps


def test_e2m1_rne_ties_go_to_even_code(oracle):
    # The tie points between grid neighbours and the even-code winner under RNE.
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for t, code in ties.items():
        assert oracle.e2m1_rne(t) == code, t
        # one ulp either side leaves the tie and goes to the nearer neighbour
        lo, hi = nextafter32(t, 0.0), nextafter32(t, 10.0)
        below = [c for c in range(8) if oracle.e2m1_value(c) < t][-1]
        above = [c for c in range(8) if oracle.e2m1_value(c) > t][0]
        assert oracle.e2m1_rne(lo) == below
        assert oracle.e2m1_rne(hi) == above


def _threshold_form(u):
    # independent closed form of nearest-even onto the grid (a different formula)
    return int(u > 0.25) + int(u >= 0.75) + int(u > 1.25) + int(u >= 1.75) + \
        int(u > 2.5) + int(u >= 3.5) + int(u > 5.0)


def test_e2m1_rne_matches_threshold_form_dense(oracle):
    rng = np.random.default_rng(0)
    vals = list(rng.uniform(0, 8, 20000).astype(np.float32))
    vals += list((10.0 ** rng.uniform(-45, 38, 5000)).astype(np.float32))
    for t in [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1.0, 2.0, 3.0, 4.0]:
        x = np.float32(t)
        for _ in range(6):
            vals += [x]
            x = np.nextafter(x, np.float32(0))
        x = np.float32(t)
        for _ in range(6):
            x = np.nextafter(x, np.float32(10))
            vals += [x]
    for u in vals:
        assert oracle.e2m1_rne(float(u)) == _threshold_form(float(u)), u


def test_e2m1_rne_saturates(oracle):
    for u in [6.0, 6.5, 7.0, 100.0, 3.4e38, float("inf")]:
        assert oracle.e2m1_rne(u) == 7


def test_rtn_input_averaged_mse_is_delta2_over_12(oracle):
    # Appendix 7: averaged over u uniform in an interior bin, RTN MSE = Delta^2/12.
    pos = [oracle.e2m1_value(c) for c in range(8)]
    for k in range(7):
        lo, hi = pos[k], pos[k + 1]
        d = hi - lo
        us = lo + (np.arange(4000) + 0.5) / 4000 * d
        err = [(oracle.e2m1_value(oracle.e2m1_rne(u)) - u) ** 2 for u in us]
        assert abs(np.mean(err) - d * d / 12) < 1e-3 * d * d


# ------------------------------------------------------------------ stochastic rounding
def test_sr_exact_expectation_and_variance(oracle):
    # Appendix 7: up with probability d/Delta, conditional variance d(Delta - d).
    # Brute force over all 2^16 random draws gives the exact distribution.
    pos = [oracle.e2m1_value(c) for c in range(8)]
    r = np.arange(65536)
    for u in [0.1, 0.3, 0.49, 0.6, 1.2, 1.6, 2.2, 2.9, 3.3, 4.7, 5.99, 0.0, 1.0, 4.0]:
        u = f32(u)
        codes = np.array([oracle.e2m1_sr(u, int(x)) for x in r])
        vals = np.array([pos[c] for c in codes])
        k = max(c for c in range(8) if pos[c] <= u)
        if pos[k] == u:
            assert np.all(vals == u)
            continue
        lo, hi = pos[k], pos[k + 1]
        d, delta = u - lo, hi - lo
        assert set(np.unique(vals)) <= {lo, hi}
        mean = vals.mean()
        assert abs(mean - u) <= delta / 65536 + 1e-12          # unbiased up to 2^-16 Delta
        var = vals.var()
        assert abs(var - d * (delta - d)) <= 2 * delta * delta / 65536 + 1e-12


def test_sr_bin_average_variance_is_delta2_over_6(oracle):
    pos = [oracle.e2m1_value(c) for c in range(8)]
    rs = np.arange(0, 65536, 97)
    for k in range(7):
        lo, hi = pos[k], pos[k + 1]
        d = hi - lo
        vs = []
        for u in lo + (np.arange(64) + 0.5) / 64 * d:
            vals = np.array([pos[oracle.e2m1_sr(f32(u), int(x))] for x in rs])
            vs.append(vals.var())
        assert abs(np.mean(vs) - d * d / 6) < 0.02 * d * d


def test_sr_saturation_cell(oracle):
    for u in [6.0, 7.0, 1e30]:
        assert oracle.e2m1_sr(u, 0) == 7 and oracle.e2m1_sr(u, 65535) == 7


# ------------------------------------------------------------------ E4M3
def test_e4m3_matches_torch_float8_e4m3fn(oracle):
    rng = np.random.default_rng(1)
    vals = list(rng.uniform(0, 448, 3000)) + list(10.0 ** rng.uniform(-5, 2.65, 3000))
    # every representable value, every midpoint, and their float32 neighbours
    reps = sorted({oracle.e4m3_value(c) for c in range(0x7F)})
    mids = [(a + b) / 2 for a, b in zip(reps, reps[1:])]
    for v in reps + mids:
        vals += [v, nextafter32(v, 0.0), nextafter32(v, 1000.0)]
    vals = [f32(v) for v in vals if 0 <= v < 464]
    t = torch.tensor(vals, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
    ours = [oracle.e4m3_encode(v) for v in vals]
    assert ours == t.tolist()


def test_e4m3_decode_matches_torch_and_saturates(oracle):
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).tolist()
    assert [oracle.e4m3_value(c) for c in range(0x7F)] == ref
    assert oracle.e4m3_value(0x7E) == 448.0
    for v in [448.0, 460.0, 470.0, 1e6, float("inf")]:
        assert oracle.e4m3_encode(v) == 0x7E
    vals = [oracle.e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))          # monotonic


def test_bf16_matches_torch(oracle):
    rng = np.random.default_rng(2)
    vals = list(rng.standard_normal(4000) * 10.0 ** rng.uniform(-30, 30, 4000))
    for base in [1.0, 1.00390625, 3.0, 1e-20]:
        b = np.float32(base)
        # exact bf16 midpoints: keep 8 significant bits then set the next bit
        u = np.frombuffer(np.float32(b).tobytes(), dtype=np.uint32)[0]
        mid = (int(u) & 0xFFFF0000) | 0x8000
        vals.append(np.frombuffer(np.uint32(mid).tobytes(), dtype=np.float32)[0])
        vals.append(np.frombuffer(np.uint32(mid | 0x10000).tobytes(), dtype=np.float32)[0])
    vals = [f32(float(v)) for v in vals]
    ref = torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
    ref = [x & 0xFFFF for x in ref.tolist()]
    assert [oracle.bf16_rne(v) for v in vals] == ref


# ------------------------------------------------------------------ Philox4x32-10
KAT_SRC = os.path.join(os.path.dirname(__file__), "philox_rocrand_kat.cpp")


@pytest.fixture(scope="module")
def rocrand_kat():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc (needed to build rocRAND's host Philox) is not installed")
    d = tempfile.mkdtemp()
    exe = os.path.join(d, "kat")
    subprocess.check_call([hipcc, "-O1", KAT_SRC, "-o", exe], stderr=subprocess.DEVNULL)
    yield exe
    shutil.rmtree(d, ignore_errors=True)


def test_philox_matches_rocrand_host_engine(oracle, rocrand_kat):
    cases = [((0, 0), (0, 0, 0, 0)),
             # the helper reaches counter words 0-1 through a 64-bit offset * 4, so word 1
             # stays below 2^30 here
             ((0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0x3FFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF)),
             ((0x5EED4, 0), (12345, 0, 1, 0x53523136)),
             ((0xDEADBEEF, 0x01234567), (7, 3, 0, 0x52485431)),
             ((1, 2), (0x80000000, 0x2FFFFFFF, 5, 6))]
    for key, ctr in cases:
        args = [rocrand_kat] + [f"{v:x}" for v in (*key, *ctr)]
        ref = [int(t, 16) for t in subprocess.check_output(args).split()]
        assert oracle.philox4x32_10(ctr, key).tolist() == ref, (key, ctr)


def test_sr_bits_and_signs_layout(oracle):
    seed = 0x123456789ABCDEF
    key = (seed & 0xFFFFFFFF, seed >> 32)
    for j in [0, 1, 2, 7, 8, 13, 2 ** 33 + 5]:
        w = oracle.philox4x32_10(((j >> 3) & 0xFFFFFFFF, j >> 35, 1, 0x53523136), key)
        word = int(w[(j >> 1) & 3])
        want = (word >> 16) if j & 1 else (word & 0xFFFF)
        assert oracle.sr_bits(seed, 1, j) == want
    s = oracle.rht_signs(seed)
    w0 = int(oracle.philox4x32_10((0, 0, 0, 0x52485431), key)[0])
    assert s.tolist() == [-1.0 if (w0 >> i) & 1 else 1.0 for i in range(16)]
    assert not np.array_equal(oracle.rht_signs(1), oracle.rht_signs(2))


# ------------------------------------------------------------------ Hadamard
def test_wht16_equals_sylvester_hadamard(oracle):
    from scipy.linalg import hadamard
    H = hadamard(16)
    assert np.array_equal(H @ H.T, 16 * np.eye(16, dtype=H.dtype))      # H H^T = n I
    for i in range(16):
        e = np.zeros(16, dtype=np.float32)
        e[i] = 1.0
        assert np.array_equal(oracle.wht16(e), H[:, i].astype(np.float32))
    rng = np.random.default_rng(3)
    for _ in range(200):
        v = rng.standard_normal(16).astype(np.float32) * 10.0 ** rng.uniform(-3, 3)
        ref = H.astype(np.float64) @ v.astype(np.float64)
        got = oracle.wht16(v).astype(np.float64)
        bound = 4 * np.finfo(np.float32).eps * np.abs(v).astype(np.float64).sum()
        assert np.all(np.abs(got - ref) <= bound)


def test_rht_is_orthogonal_and_preserves_inner_products(oracle):
    from scipy.linalg import hadamard
    rng = np.random.default_rng(4)
    sgn = oracle.rht_signs(0x5EED4)
    T = 0.25 * hadamard(16) @ np.diag(sgn.astype(np.float64))
    assert np.allclose(T @ T.T, np.eye(16), atol=0)
    for _ in range(200):
        a = rng.standard_normal(16).astype(np.float32)
        b = rng.standard_normal(16).astype(np.float32)
        ta, tb = oracle.rht16_forward(a, sgn), oracle.rht16_forward(b, sgn)
        assert np.allclose(ta.astype(np.float64), T @ a.astype(np.float64), rtol=0, atol=1e-6)
        ip = float(np.dot(a.astype(np.float64), b.astype(np.float64)))
        ipt = float(np.dot(ta.astype(np.float64), tb.astype(np.float64)))
        assert abs(ip - ipt) <= 1e-5 * np.linalg.norm(a) * np.linalg.norm(b)
        back = oracle.rht16_inverse(ta, sgn)
        assert np.allclose(back, a, rtol=0, atol=1e-6)


def test_rht_spreads_an_outlier(oracle):
    # OptiTrain README: after the normalised transform an outlier of 100 spreads
    # to about 100/sqrt(N) on every entry; here N = 16, so 25 +- sum of the rest / 4.
    v = np.zeros(16, dtype=np.float32)
    v[:8] = [100.0, 0.2, 0.4, 0.1, 0.3, 0.5, 0.2, 0.1]
    t = oracle.rht16_forward(v, np.ones(16, dtype=np.float32))
    rest = float(np.abs(v[1:]).sum())
    assert np.all(np.abs(np.abs(t) - 25.0) <= rest / 4 + 1e-5)
