"""GPU parity of the LoRA-SVD low-rank branch (Full-Stack FP4 sec. 3.2 eq. (1), Appendix 9)
against the oracle.

nvfp4_gemm_lora: operands quantized by the oracle, BF16 factors seeded synthetic inputs;
the reference is the oracle's binary64 GEMM plus sum_j t l.  Tolerance as the plain GEMM's
(gpu_util.GEMM_TOL) with sum |terms| covering both parts: relative Frobenius error and
max |C - C64| / (sum_k |a b| + sum_j |t l|) <= 1e-5.  The kernel's roundings are the FP32
accumulations of both parts and the one FP32 scaling of the NVFP4 accumulator.
Full-size FFN-up (8192 x 9216 x 3072, rank 64) is checked on sampled entries.
"""
import numpy as np
import pytest
import torch

from gpu_util import GEMM_TOL, dev, gemm_errors, to_gpu_qtensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load_library()
    return nv


def operands(oracle, M, N, K, r, seed):
    from nvfp4_block_scaled_quantize_amd import synthetic
    a = synthetic.outlier_channels((M, K), seed).to(torch.bfloat16).float().numpy()
    b = synthetic.normal((N, K), seed + 1, 0.02).to(torch.bfloat16).float().numpy()
    qa, _ = oracle.quantize(a)
    qb, _ = oracle.quantize(b, block2d=True)
    t = synthetic.normal((M, r), seed + 2, 0.5).to(torch.bfloat16)
    lb = synthetic.normal((N, r), seed + 3, 0.02).to(torch.bfloat16)
    return qa, qb, t, lb


def bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("M,N,K,r", [(16, 16, 32, 16), (48, 80, 64, 32), (272, 400, 160, 64),
                                     (528, 272, 416, 48), (256, 256, 416, 64), (64, 96, 1024, 128),
                                     (304, 208, 192, 16)])
def test_gemm_lora_small_shapes(nv, oracle, M, N, K, r):
    print(f"gemm_lora case {M}x{N}x{K} rank {r}", flush=True)
    qa, qb, t, lb = operands(oracle, M, N, K, r, 10 + M + N + K + r)
    c = nv.nvfp4_gemm_lora(to_gpu_qtensor(nv, qa), to_gpu_qtensor(nv, qb), t.to(dev()), lb.to(dev()))
    torch.cuda.synchronize()
    ref, absdot = oracle.gemm_lora_f64(qa, qb, bits(t), bits(lb))
    fro, nw = gemm_errors(c.cpu().numpy(), ref, absdot)
    print(f"  frobenius {fro:.3e} normwise {nw:.3e}")
    assert fro <= GEMM_TOL and nw <= GEMM_TOL


def test_gemm_lora_full_size_sampled(nv, oracle):
    M, N, K, r = 8192, 9216, 3072, 64
    print(f"gemm_lora full-size FFN-up {M}x{N}x{K} rank {r}", flush=True)
    qa, qb, t, lb = operands(oracle, M, N, K, r, 77)
    c = nv.nvfp4_gemm_lora(to_gpu_qtensor(nv, qa), to_gpu_qtensor(nv, qb), t.to(dev()), lb.to(dev()))
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    em = np.concatenate([rng.integers(0, M, 4096), [0] * N, [M - 1] * N, np.arange(M), np.arange(M)])
    en = np.concatenate([rng.integers(0, N, 4096), np.arange(N), np.arange(N), [0] * M, [N - 1] * M])
    ref, absdot = oracle.gemm_lora_f64_entries(qa, qb, bits(t), bits(lb), em, en)
    fro, nw = gemm_errors(c.cpu().numpy()[em, en], ref, absdot)
    print(f"  sampled frobenius {fro:.3e} normwise {nw:.3e}")
    assert fro <= GEMM_TOL and nw <= GEMM_TOL


def test_gemm_lora_rank_zero_is_the_plain_gemm(nv, oracle):
    qa, qb, _, _ = operands(oracle, 96, 112, 128, 16, 3)
    ga, gb = to_gpu_qtensor(nv, qa), to_gpu_qtensor(nv, qb)
    empty_t = torch.empty((96, 0), dtype=torch.bfloat16, device=dev())
    empty_b = torch.empty((112, 0), dtype=torch.bfloat16, device=dev())
    c0 = nv.nvfp4_gemm(ga, gb)
    c1 = nv.nvfp4_gemm_lora(ga, gb, empty_t, empty_b)
    torch.cuda.synchronize()
    assert torch.equal(c0, c1)


def test_gemm_lora_rejects_bad_rank(nv, oracle):
    qa, qb, _, _ = operands(oracle, 32, 32, 64, 16, 4)
    ga, gb = to_gpu_qtensor(nv, qa), to_gpu_qtensor(nv, qb)
    t = torch.zeros((32, 8), dtype=torch.bfloat16, device=dev())
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_gemm_lora(ga, gb, t, t.clone())


# ---------------------------------------------------------------- fused down-projection
# nvfp4_quantize_lora: the NVFP4 copies must equal the oracle's bit for bit (the first pass
# computes the tensor amax too), and T = BF16(beta x a^T) is compared with the oracle's
# binary64 value: either the same BF16 value, or within half a BF16 ulp of the exact value
# plus the FP32 accumulation bound (cols + 1) 2^-24 |beta| sum |x a|; almost all elements
# must be the same value.
def bf16_to_np(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_vals(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def check_lora_t(t_gpu, t_or, t64, tabs, cols):
    got, want = bf16_vals(t_gpu), bf16_vals(t_or)
    same = got == want
    ulp = np.maximum(np.abs(want), 2.0 ** -126) * 2.0 ** -7
    bound = 0.5 * ulp + (cols + 1) * 2.0 ** -24 * tabs
    assert np.all(same | (np.abs(got - t64) <= bound)), "low-rank values outside the bound"
    assert same.mean() > 0.99, f"only {same.mean():.4f} of the low-rank values agree"


LORA_MODES = {
    "row": dict(rowwise=True),
    "row+colRHT": dict(rowwise=True, colwise=True, rht_col=True, seed=0x5EED4),
    "rowRHT+colRHT SR": dict(rowwise=True, colwise=True, rht_row=True, rht_col=True,
                            round_row=1, round_col=1, seed=0x5EED4),
    "rowRHT": dict(rowwise=True, rht_row=True, seed=11),
    "col": dict(rowwise=False, colwise=True),
}


@pytest.mark.parametrize("mode", list(LORA_MODES))
@pytest.mark.parametrize("R,C,r", [(64, 128, 16), (48, 256, 32), (272, 384, 64), (528, 640, 48)])
def test_quantize_lora_small(nv, oracle, mode, R, C, r):
    from nvfp4_block_scaled_quantize_amd import synthetic
    from gpu_util import assert_copy_equal
    print(f"quantize_lora {mode} {R}x{C} rank {r}", flush=True)
    x = synthetic.outlier_channels((R, C), R + C + r).to(torch.bfloat16)
    la = synthetic.normal((r, C), 7 + r, C ** -0.5).to(torch.bfloat16)
    beta = 0.5
    kw = LORA_MODES[mode]
    p = nv.quant_params(**kw)
    row, col, t = nv.nvfp4_quantize_lora(x.to(dev()), p, la.to(dev()), beta)
    torch.cuda.synchronize()
    xo = x.float().numpy()
    okw = dict(rowwise=kw.get("rowwise", True), colwise=kw.get("colwise", False),
               round_row=kw.get("round_row", 0), round_col=kw.get("round_col", 0),
               rht_row=kw.get("rht_row", False), rht_col=kw.get("rht_col", False),
               seed=kw.get("seed", 0))
    orow, ocol = oracle.quantize(xo, **okw)
    if okw["rowwise"]:
        assert_copy_equal(row, orow, "rowwise")
    if okw["colwise"]:
        assert_copy_equal(col, ocol, "colwise")
    t_or, t64, tabs = oracle.lora_down(xo, bf16_to_np(la), beta)
    check_lora_t(bf16_to_np(t), t_or, t64, tabs, C)


def test_quantize_lora_full_size_x(nv, oracle):
    """X 8192x3072 (row + column RHT copies) with the rank-64 down-projection of L1."""
    from nvfp4_block_scaled_quantize_amd import synthetic
    from gpu_util import assert_copy_equal
    print("quantize_lora full-size X 8192x3072 rank 64", flush=True)
    x = synthetic.ffn()["X"]
    lo = synthetic.lora()
    p = nv.quant_params(rowwise=True, colwise=True, rht_col=True, seed=0x5EED4)
    row, col, t = nv.nvfp4_quantize_lora(x.to(dev()), p, lo["L1"].to(dev()), lo["beta"])
    torch.cuda.synchronize()
    xo = x.float().numpy()
    orow, ocol = oracle.quantize(xo, rowwise=True, colwise=True, rht_col=True, seed=0x5EED4)
    assert_copy_equal(row, orow, "rowwise")
    assert_copy_equal(col, ocol, "colwise")
    rows = np.random.default_rng(3).choice(8192, 256, replace=False)
    t_or, t64, tabs = oracle.lora_down(xo[rows], bf16_to_np(lo["L1"]), lo["beta"])
    check_lora_t(bf16_to_np(t)[rows], t_or, t64, tabs, 3072)


def test_quantize_lora_limits(nv):
    x = torch.zeros((64, 128), dtype=torch.bfloat16, device=dev())
    p = nv.quant_params(rowwise=True)
    with pytest.raises(nv.Nvfp4Error):   # rank above 64
        nv.nvfp4_quantize_lora(x, p, torch.zeros((80, 128), dtype=torch.bfloat16, device=dev()), 1.0)
    with pytest.raises(nv.Nvfp4Error):   # cols not a multiple of 128
        nv.nvfp4_quantize_lora(torch.zeros((64, 96), dtype=torch.bfloat16, device=dev()), p,
                               torch.zeros((16, 96), dtype=torch.bfloat16, device=dev()), 1.0)
    # zero input: T = 0 and the copies of a zero tensor
    row, _, t = nv.nvfp4_quantize_lora(x, p, torch.ones((16, 128), dtype=torch.bfloat16, device=dev()), 1.0)
    torch.cuda.synchronize()
    assert torch.all(t == 0) and row.gscale.item() == 1.0


# ---------------------------------------------------------------- eq. (2) double quantization
# nvfp4_requantize_cols gets the oracle's rowwise copy and must reproduce the oracle's
# columnwise quantization of its decoded values bit for bit.
REQ_MODES = {
    "rne": dict(),
    "rht": dict(rht_col=True, seed=0x5EED4),
    "sr": dict(round_col=1, seed=21),
    "rht+sr": dict(rht_col=True, round_col=1, seed=0x5EED4),
    "rht+sr 4/6": dict(rht_col=True, round_col=1, seed=0x5EED4, scale46=True),
}


@pytest.mark.parametrize("mode", list(REQ_MODES))
@pytest.mark.parametrize("R,C", [(16, 16), (48, 80), (272, 400), (528, 160)])
def test_requantize_cols_small(nv, oracle, mode, R, C):
    from nvfp4_block_scaled_quantize_amd import synthetic
    from gpu_util import assert_copy_equal
    print(f"requantize_cols {mode} {R}x{C}", flush=True)
    x = synthetic.outlier_channels((R, C), 31 + R + C).to(torch.bfloat16).float().numpy()
    orow, _ = oracle.quantize(x)
    kw = REQ_MODES[mode]
    p = nv.quant_params(rowwise=False, colwise=True, **kw)
    col = nv.nvfp4_requantize_cols(to_gpu_qtensor(nv, orow), p)
    torch.cuda.synchronize()
    want = oracle.requantize_cols(orow, round_col=kw.get("round_col", 0),
                                  rht_col=kw.get("rht_col", False), seed=kw.get("seed", 0),
                                  scale46=kw.get("scale46", False))
    assert_copy_equal(col, want, "requantized columnwise")


def test_requantize_cols_full_size(nv, oracle):
    """X 8192x3072: the Wgrad operand of eq. (2) (column RHT, SR) from the rowwise copy."""
    from nvfp4_block_scaled_quantize_amd import synthetic
    from gpu_util import assert_copy_equal
    print("requantize_cols full-size X 8192x3072", flush=True)
    x = synthetic.ffn()["X"].float().numpy()
    orow, _ = oracle.quantize(x)
    p = nv.quant_params(rowwise=False, colwise=True, rht_col=True, round_col=1, seed=0x5EED4)
    col = nv.nvfp4_requantize_cols(to_gpu_qtensor(nv, orow), p)
    torch.cuda.synchronize()
    want = oracle.requantize_cols(orow, round_col=1, rht_col=True, seed=0x5EED4)
    assert_copy_equal(col, want, "requantized columnwise")


def test_requantize_cols_refuses_rowwise(nv):
    q = nv.QTensor.empty(32, 32, dev())
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_requantize_cols(q, nv.quant_params(rowwise=True, colwise=True))
