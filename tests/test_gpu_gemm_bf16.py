"""GPU parity of the bfloat16-output GEMM with tile maxima, and of the quantize that takes
its amax from caller-supplied partial maxima (the two halves of a single-read quantize of a
GEMM's output).

nvfp4_gemm_bf16 stores bf16_rne of the FP32 result that one workgroup per tile forms (its last
round, when at most half full after whole rounds, runs as half-width tiles whose elements see
the same MFMAs in the same order), so on every shape:
  * the output is bit for bit nvfp4_gemm's FP32 output with one workgroup per tile
    (NVFP4_GEMM_SK=0) rounded to bfloat16 by torch, and within the GEMM tolerance plus one
    bf16 rounding of the oracle's binary64 product;
  * each tile maximum equals the largest |C| over that 256 x 256 tile of the output.
nvfp4_quantize with amax_parts is bit for bit nvfp4_quantize of the same tensor whenever
the parts' maximum is the tensor's amax (tile maxima, per-row maxima, one value).
Shapes: 2000 x 4000 x 192 (one round, half full); 4112 x 4112 x 192 (one whole round, then 33
ragged tiles as half-width tiles, some right halves wholly past N); 4352 x 4096 x 320 (one
whole round, 16 half-width tile pairs on their XCDs, three K stages); 300 x 520 x 256 has
ragged tiles; K = 96 takes the generic staging path.  The FFN-up shape 8192 x 9216 x 3072
(four whole rounds, then 128 tiles as half-width tiles) is compared whole, twice in a row.
"""
import numpy as np
import pytest
import torch

from gpu_util import GEMM_TOL, dev, to_gpu_qtensor

pytestmark = pytest.mark.gpu

SHAPES = [(2000, 4000, 192), (4112, 4112, 192), (4352, 4096, 320), (300, 520, 256), (256, 512, 96)]
BF16_U = 2.0 ** -8   # unit roundoff of bfloat16 nearest-even (8 significant bits)


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load_library()
    return nv


@pytest.fixture(scope="module", params=SHAPES, ids=lambda s: "x".join(map(str, s)))
def operands(oracle, request):
    from nvfp4_block_scaled_quantize_amd import synthetic
    M, N, K = request.param
    a = synthetic.outlier_channels((M, K), 5501 + M).to(torch.bfloat16).float().numpy()
    b = synthetic.normal((N, K), 5502 + N, 0.02).to(torch.bfloat16).float().numpy()
    qa, _ = oracle.quantize(a)
    qb, _ = oracle.quantize(b)
    return qa, qb


def setenv(monkeypatch, **env):
    for k in ("NVFP4_GEMM_SK", "NVFP4_GEMM_SK_SPIN", "NVFP4_GEMM_SK_TEST"):
        monkeypatch.delenv(k, raising=False)
    for k, v in env.items():
        monkeypatch.setenv(k, str(v))


def tile_maxima(c):
    """Largest |c| per 256 x 256 tile, row-major over tiles (float32)."""
    M, N = c.shape
    a = c.float().abs()
    tm, tn = (M + 255) // 256, (N + 255) // 256
    pad = torch.zeros((tm * 256, tn * 256), dtype=torch.float32, device=c.device)
    pad[:M, :N] = a
    return pad.view(tm, 256, tn, 256).amax(dim=(1, 3)).reshape(-1)


def bits16(t):
    return t.view(torch.int16)


def test_bf16_is_the_fp32_result_rounded(nv, operands, monkeypatch):
    qa, qb = operands
    M, N = qa.shape[0], qb.shape[0]
    print(f"gemm bf16 {M}x{N}x{qa.shape[1]}", flush=True)
    ga, gb = to_gpu_qtensor(nv, qa), to_gpu_qtensor(nv, qb)
    setenv(monkeypatch, NVFP4_GEMM_SK=0)
    c32 = nv.nvfp4_gemm(ga, gb)
    setenv(monkeypatch)
    c16, tmax = nv.nvfp4_gemm_bf16(ga, gb)
    torch.cuda.synchronize()
    assert torch.equal(bits16(c16), bits16(c32.to(torch.bfloat16)))
    assert torch.equal(tmax.view(torch.int32), tile_maxima(c16).view(torch.int32))


def test_bf16_ffn_up_full_size(nv, monkeypatch):
    """8192 x 9216 x 3072 as the benchmark runs it (whole rounds, then half-width tiles): bit for
    bit the per-tile FP32 product rounded, and the tile maxima, on two calls in a row."""
    from nvfp4_block_scaled_quantize_amd import synthetic
    ffn = synthetic.ffn()
    print("gemm bf16 FFN-up 8192x9216x3072", flush=True)
    qx, _ = nv.nvfp4_quantize(ffn["X"].to(dev()), nv.quant_params(rowwise=True))
    qw, _ = nv.nvfp4_quantize(ffn["W_up"].to(dev()), nv.quant_params(rowwise=True, block2d=True))
    setenv(monkeypatch, NVFP4_GEMM_SK=0)
    ref = nv.nvfp4_gemm(qx, qw).to(torch.bfloat16)
    setenv(monkeypatch)
    out = torch.empty_like(ref)
    tmax = torch.full((nv.load_library().nvfp4_gemm_tiles(8192, 9216),), -1.0, device=dev())
    for rep in range(2):
        nv.nvfp4_gemm_bf16(qx, qw, out=out, tile_amax=tmax)
        torch.cuda.synchronize()
        assert torch.equal(bits16(out), bits16(ref)), f"call {rep}"
        assert torch.equal(tmax.view(torch.int32), tile_maxima(out).view(torch.int32)), f"call {rep}"


def test_bf16_vs_oracle(nv, oracle, operands, monkeypatch):
    """|c - ref| <= GEMM_TOL sum|a b| + 2^-8 (|ref| + GEMM_TOL sum|a b|) per entry: the FP32
    GEMM's bound, then one bf16 rounding."""
    qa, qb = operands
    setenv(monkeypatch)
    c16, _ = nv.nvfp4_gemm_bf16(to_gpu_qtensor(nv, qa), to_gpu_qtensor(nv, qb))
    ref, absdot = oracle.gemm_f64(qa, qb)
    c = c16.float().cpu().numpy().astype(np.float64)
    bound = GEMM_TOL * absdot + BF16_U * (np.abs(ref) + GEMM_TOL * absdot) + 1e-30
    err = np.abs(c - ref)
    print(f"  max err/bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound)


def test_bf16_graph_replays(nv, operands, monkeypatch):
    qa, qb = operands
    M, N = qa.shape[0], qb.shape[0]
    setenv(monkeypatch)
    ga, gb = to_gpu_qtensor(nv, qa), to_gpu_qtensor(nv, qb)
    ref, rmax = nv.nvfp4_gemm_bf16(ga, gb)
    d = dev()
    out = torch.empty((M, N), dtype=torch.bfloat16, device=d)
    tmax = torch.empty_like(rmax)
    s = torch.cuda.Stream(device=d)
    s.wait_stream(torch.cuda.current_stream(d))
    with torch.cuda.stream(s):
        nv.nvfp4_gemm_bf16(ga, gb, out=out, tile_amax=tmax)
    torch.cuda.current_stream(d).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv.nvfp4_gemm_bf16(ga, gb, out=out, tile_amax=tmax)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        tmax.fill_(-1.0)
        other, _ = nv.nvfp4_gemm_bf16(ga, gb)      # an eager launch in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits16(out), bits16(ref)), f"replay {rep}"
        assert torch.equal(tmax.view(torch.int32), rmax.view(torch.int32)), f"replay {rep}"
        assert torch.equal(bits16(other), bits16(ref)), f"eager {rep}"


# ------------------------------------------------------------------ quantize with given maxima
GIVEN_MODES = {
    "row": dict(rowwise=True),
    "rowcol": dict(rowwise=True, colwise=True),
    "sr": dict(rowwise=True, colwise=True, round_row=1, round_col=1, seed=77),
    "2d": dict(rowwise=True, colwise=True, block2d=True),
    "46": dict(rowwise=True, colwise=True, scale46=True),
}


def same_copy(x, y):
    assert torch.equal(x.codes, y.codes)
    assert torch.equal(x.scales, y.scales)
    assert torch.equal(x.gscale.view(torch.int32), y.gscale.view(torch.int32))


@pytest.mark.parametrize("mode", list(GIVEN_MODES))
def test_quantize_given_amax_is_bitwise_the_two_pass(nv, operands, monkeypatch, mode):
    qa, qb = operands
    M, N = qa.shape[0], qb.shape[0]
    if M % 16 or N % 16:
        pytest.skip("quantize needs multiples of 16")
    setenv(monkeypatch)
    h, tmax = nv.nvfp4_gemm_bf16(to_gpu_qtensor(nv, qa), to_gpu_qtensor(nv, qb))
    p = nv.quant_params(**GIVEN_MODES[mode])
    print(f"quantize {M}x{N} {mode} with the GEMM's tile maxima", flush=True)
    r0, c0 = nv.nvfp4_quantize(h, p)
    r1, c1 = nv.nvfp4_quantize(h, p, amax_parts=tmax)
    rowmax = h.float().abs().amax(dim=1).contiguous()
    r2, c2 = nv.nvfp4_quantize(h, p, amax_parts=rowmax)
    one = h.float().abs().amax().reshape(1)
    r3, c3 = nv.nvfp4_quantize(h, p, amax_parts=one)
    torch.cuda.synchronize()
    for r, c in ((r1, c1), (r2, c2), (r3, c3)):
        same_copy(r, r0)
        if p.colwise:
            same_copy(c, c0)


def test_quantize_given_amax_f32_input(nv):
    """An FP32 input with per-column maxima given, against the two-pass quantize."""
    from nvfp4_block_scaled_quantize_amd import synthetic
    x = synthetic.outlier_channels((512, 768), 5511).to(dev())
    p = nv.quant_params(rowwise=True, colwise=True, scale46=True)
    r0, c0 = nv.nvfp4_quantize(x, p)
    r1, c1 = nv.nvfp4_quantize(x, p, amax_parts=x.abs().amax(dim=0).contiguous())
    torch.cuda.synchronize()
    same_copy(r1, r0)
    same_copy(c1, c0)


def test_quantize_given_amax_refuses_rotations(nv):
    x = torch.zeros((64, 64), dtype=torch.bfloat16, device=dev())
    parts = torch.ones(4, dtype=torch.float32, device=dev())
    for kw in (dict(rowwise=True, rht_row=True), dict(rowwise=True, colwise=True, rht_col=True)):
        with pytest.raises(nv.Nvfp4Error):
            nv.nvfp4_quantize(x, nv.quant_params(**kw), amax_parts=parts)
