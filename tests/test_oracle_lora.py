"""Pins of the oracle's LoRA-SVD low-rank branch (Full-Stack FP4 sec. 3.2 eq. (1) and
Appendix 9): the down-projection T = BF16(beta X L1^T) and the GEMM that adds T L2^T to the
NVFP4 product.  The checks use no oracle arithmetic:
  * closed forms: unit-vector rows of L1 pick columns of X (exact for power-of-two beta);
    sums that land on BF16 midpoints round to the even neighbour;
  * random shapes: the binary64 value equals numpy's float64 matrix product, and the BF16
    result is that value rounded to nearest-even by a rounding written here;
  * the GEMM with T = 0 is the plain GEMM, bit for bit; with all-zero NVFP4 operands it
    is T L2^T as numpy computes it from the BF16 values.
"""
import math

import numpy as np
import torch

ONE = 0x3F80


def bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def bf16_vals(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(v):
    """Nearest-even BF16 of a binary64 value in the normal range (exact integer rounding)."""
    if v == 0.0:
        return 0.0
    m, e = math.frexp(abs(v))          # |v| = m 2^e, m in [0.5, 1)
    q = round(m * 256.0)               # 8 significant bits; Python rounds ties to even
    return math.copysign(math.ldexp(q, e - 8), v)


def test_unit_rows_pick_columns(oracle):
    rng = np.random.default_rng(0)
    x = bf16_vals(bf16_bits(rng.standard_normal((8, 48)))).astype(np.float32)
    cols = [5, 0, 47, 16]
    a = np.zeros((len(cols), 48), dtype=np.uint16)
    for j, k in enumerate(cols):
        a[j, k] = ONE
    for beta in (1.0, 0.25, -8.0):
        t, t64, tabs = oracle.lora_down(x, a, beta)
        want = beta * x[:, cols].astype(np.float64)
        assert np.array_equal(bf16_vals(t), want)
        assert np.array_equal(t64, want) and np.array_equal(tabs, np.abs(want))
    t, _, _ = oracle.lora_down(x, a, 0.0)
    assert np.all(bf16_vals(t) == 0.0)


def test_midpoints_round_to_even(oracle):
    # x a^T = v exactly; 1 + 2^-8 lies midway between 1 (even) and 1 + 2^-7 (odd)
    cases = [(1 + 2 ** -8, 0x3F80), (1 + 3 * 2 ** -8, 0x3F82), (-(1 + 2 ** -8), 0xBF80),
             (1 + 2 ** -8 + 2 ** -20, 0x3F81), (3 * 2 ** -9 + 2 ** -16, 0x3BC0),
             (3 * 2 ** -9 + 3 * 2 ** -16, 0x3BC2)]
    x = np.array([[v] for v, _ in cases], dtype=np.float32)
    a = np.array([[ONE]], dtype=np.uint16)
    t, _, _ = oracle.lora_down(x, a, 1.0)
    assert [int(b) for b in t[:, 0]] == [want for _, want in cases]


def test_down_projection_is_the_matrix_product(oracle):
    rng = np.random.default_rng(1)
    M, K, r = 40, 96, 32
    x = bf16_vals(bf16_bits(rng.standard_normal((M, K)) * 3)).astype(np.float32)
    a = bf16_bits(rng.standard_normal((r, K)) / np.sqrt(K))
    beta = 0.7
    t, t64, tabs = oracle.lora_down(x, a, beta)
    ref = np.float64(np.float32(beta)) * (x.astype(np.float64) @ bf16_vals(a).T)
    assert np.allclose(t64, ref, rtol=1e-13, atol=1e-300)
    assert np.allclose(tabs, abs(np.float32(beta)) * (np.abs(x.astype(np.float64)) @ np.abs(bf16_vals(a)).T),
                       rtol=1e-13)
    got = bf16_vals(t)
    want = np.vectorize(round_bf16)(ref)
    # the two binary64 sums may differ in the last bits; they round alike away from midpoints
    near_mid = np.zeros_like(ref, dtype=bool)
    for idx, v in np.ndenumerate(ref):
        m, e = math.frexp(abs(v))
        near_mid[idx] = abs(m * 256 - math.floor(m * 256) - 0.5) < 1e-9
    assert np.array_equal(got[~near_mid], want[~near_mid])
    assert near_mid.sum() < 3


def test_gemm_lora_reduces_to_gemm(oracle):
    rng = np.random.default_rng(2)
    M, N, K, r = 32, 48, 64, 16
    qa, _ = oracle.quantize(rng.standard_normal((M, K)).astype(np.float32))
    qb, _ = oracle.quantize(rng.standard_normal((N, K)).astype(np.float32))
    zt = np.zeros((M, r), dtype=np.uint16)
    b = bf16_bits(rng.standard_normal((N, r)))
    C0, ad0 = oracle.gemm_f64(qa, qb)
    C1, ad1 = oracle.gemm_lora_f64(qa, qb, zt, b)
    assert np.array_equal(C0, C1) and np.array_equal(ad0, ad1)
    em, en = np.array([0, 5, 31]), np.array([47, 0, 9])
    e1, a1 = oracle.gemm_lora_f64_entries(qa, qb, zt, b, em, en)
    assert np.array_equal(e1, C0[em, en]) and np.array_equal(a1, ad0[em, en])


def test_gemm_lora_with_zero_operands_is_the_low_rank_product(oracle):
    rng = np.random.default_rng(3)
    M, N, K, r = 24, 40, 32, 64
    qa, _ = oracle.quantize(np.zeros((M, K), dtype=np.float32))
    qb, _ = oracle.quantize(np.zeros((N, K), dtype=np.float32))
    t = bf16_bits(rng.standard_normal((M, r)))
    b = bf16_bits(rng.standard_normal((N, r)) * 0.02)
    C, ad = oracle.gemm_lora_f64(qa, qb, t, b)
    ref = bf16_vals(t) @ bf16_vals(b).T
    assert np.allclose(C, ref, rtol=1e-14, atol=1e-300)
    assert np.allclose(ad, np.abs(bf16_vals(t)) @ np.abs(bf16_vals(b)).T, rtol=1e-14)
    # and on top of a nonzero product the difference is the same low-rank term
    qa2, _ = oracle.quantize(rng.standard_normal((M, K)).astype(np.float32))
    qb2, _ = oracle.quantize(rng.standard_normal((N, K)).astype(np.float32))
    C2, _ = oracle.gemm_lora_f64(qa2, qb2, t, b)
    C20, _ = oracle.gemm_f64(qa2, qb2)
    assert np.allclose(C2 - C20, ref, rtol=1e-12, atol=1e-12 * np.abs(C20).max())


# ---------------------------------------------------------------- eq. (2) double quantization
def test_requantize_cols_of_a_representable_tensor_is_single_quantization(oracle):
    """When X already holds decoded NVFP4 values with one tensor scale, Q_1x16 returns the
    same values, so Q_16x1(H^T Q_1x16(X)) must equal Q_16x1(H^T X)."""
    rng = np.random.default_rng(12)
    x0 = (rng.standard_normal((64, 96)) * np.exp(rng.standard_normal((64, 1)))).astype(np.float32)
    q, _ = oracle.quantize(x0)
    x = oracle.dequantize(q)                     # representable values
    q2, _ = oracle.quantize(x)
    assert np.array_equal(oracle.dequantize(q2), x)   # the rowwise copy reproduces them
    for kw in (dict(), dict(rht_col=True, seed=5), dict(round_col=oracle.SR, seed=7),
               dict(rht_col=True, round_col=oracle.SR, seed=9)):
        got = oracle.requantize_cols(q2, **kw)
        _, want = oracle.quantize(x, rowwise=False, colwise=True, **kw)
        assert np.array_equal(got.codes, want.codes) and np.array_equal(got.scales, want.scales)
        assert got.sg == want.sg


def test_requantize_cols_differs_from_single_quantization(oracle):
    rng = np.random.default_rng(13)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    qr, _ = oracle.quantize(x)
    got = oracle.requantize_cols(qr, rht_col=True, seed=3)
    _, single = oracle.quantize(x, rowwise=False, colwise=True, rht_col=True, seed=3)
    assert not np.array_equal(got.codes, single.codes)   # the row rounding shows through
    assert got.codes.shape == single.codes.shape and got.scales.shape == single.scales.shape
