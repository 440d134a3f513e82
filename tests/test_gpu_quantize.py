"""GPU parity of nvfp4_quantize / nvfp4_dequantize against the CPU oracle.

Bar: bit-exact codes, scales and tensor scales for every copy, every option combination
(1D/2D, RNE/SR, Hadamard per copy), both input dtypes, shapes that span several 256x128
workgroup tiles with ragged tails, and the full-size activation, weight and gradient
tensors of the 3B workloads.  Inputs are seeded and synthetic; expected values come from
the oracle only.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_copy_equal, dev, to_gpu_qtensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load_library()
    return nv


def make_input(shape, seed, dtype):
    from nvfp4_block_scaled_quantize_amd import synthetic
    x = synthetic.spiky(shape, seed)
    g = torch.Generator().manual_seed(seed + 7)
    # rows of tiny values, an all-zero 16x16 tile, signed zeros
    if shape[0] >= 32:
        x[16:32] *= 1e-5
    if shape[0] >= 16 and shape[1] >= 32:
        x[:16, 16:32] = 0.0
        x[0, 16] = -0.0
    x[torch.rand(shape, generator=g) < 0.01] = -0.0
    return x.to(dtype)


MODES = {
    "row": dict(rowwise=True),
    "col": dict(rowwise=False, colwise=True),
    "rowcol": dict(rowwise=True, colwise=True),
    "2d": dict(rowwise=True, colwise=True, block2d=True),
    "2d_col": dict(rowwise=False, colwise=True, block2d=True),
    "sr": dict(rowwise=True, colwise=True, round_row=1, round_col=1),
    "wgrad_dy": dict(rowwise=False, colwise=True, round_col=1, rht_col=True),
    "wgrad_x": dict(rowwise=False, colwise=True, rht_col=True),
    "rht_row": dict(rowwise=True, rht_row=True),
    "dgrad_and_wgrad": dict(rowwise=True, colwise=True, round_row=1, round_col=1, rht_col=True),
    "all": dict(rowwise=True, colwise=True, round_row=1, round_col=1, rht_row=True, rht_col=True),
    # 4/6 adaptive block scaling (1x16 blocks)
    "46_row": dict(rowwise=True, scale46=True),
    "46_rowcol": dict(rowwise=True, colwise=True, scale46=True),
    "46_sr_rhtcol": dict(rowwise=True, colwise=True, round_row=1, round_col=1, rht_col=True,
                         scale46=True),
    "46_all": dict(rowwise=True, colwise=True, round_row=1, round_col=1, rht_row=True,
                   rht_col=True, scale46=True),
    # both copies rotated, nearest-even (the Newton-Schulz quantization of X and A), with and
    # without 4/6 scaling; the rowwise-rotated copy alone with 4/6 (its quantization of B)
    "rht_both": dict(rowwise=True, colwise=True, rht_row=True, rht_col=True),
    "46_rht_both": dict(rowwise=True, colwise=True, rht_row=True, rht_col=True, scale46=True),
    "46_rht_row": dict(rowwise=True, rht_row=True, scale46=True),
}
SHAPES = [(16, 16), (48, 80), (128, 256), (272, 400), (528, 144)]


def run_case(nv, oracle, x, mode, seed, kw=None):
    kw = MODES[mode] if kw is None else kw
    p = nv.quant_params(seed=seed, **kw)
    print(f"quantize case {tuple(x.shape)} {x.dtype} {mode} seed={seed:#x}", flush=True)
    gr, gc = nv.nvfp4_quantize(x.to(dev()), p)
    torch.cuda.synchronize()
    orow, ocol = oracle.quantize(x.float().numpy(), rowwise=kw.get("rowwise", True),
                                 colwise=kw.get("colwise", False),
                                 block2d=kw.get("block2d", False),
                                 round_row=kw.get("round_row", 0), round_col=kw.get("round_col", 0),
                                 rht_row=kw.get("rht_row", False), rht_col=kw.get("rht_col", False),
                                 seed=seed, scale46=kw.get("scale46", False))
    if orow is not None:
        assert_copy_equal(gr, orow, f"{mode} rowwise")
    if ocol is not None:
        assert_copy_equal(gc, ocol, f"{mode} colwise")
    return gr, gc, orow, ocol


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("mode", list(MODES))
def test_quantize_matches_oracle(nv, oracle, dtype, shape, mode):
    seed = 0x1234 + shape[0] * 7 + shape[1]
    x = make_input(shape, seed, dtype)
    run_case(nv, oracle, x, mode, 0x5EED0000 + seed)


# Tensor scales at the edges of the kernels' arithmetic shortcuts: s_g < 2^-92 takes the plain
# divisions for the block scales; s_g > 2^110 (or < 2^-92) keeps the rotation's factor 1/4
# out of the element reciprocal; below that the element reciprocal of small block scales
# overflows binary32 and the elements are divided by the scale instead; 2^-130 makes every
# input subnormal.  The largest input 2^125 keeps every butterfly sum below 2^128.
EXTREME_MODES = ["rowcol", "rht_row", "wgrad_x", "rht_both", "dgrad_and_wgrad", "all",
                 "46_rowcol", "46_rht_both", "46_all"]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("log2_amax", [125, -85, -100, -110, -120, -130])
@pytest.mark.parametrize("mode", EXTREME_MODES)
def test_extreme_tensor_scales(nv, oracle, dtype, log2_amax, mode):
    x = make_input((272, 400), 0x3E3 + log2_amax, torch.float32)
    x = x / x.abs().max() * 2.0 ** log2_amax
    run_case(nv, oracle, x.to(dtype), mode, 0x5EED0000 + log2_amax)


def test_rne_ties_and_neighbours(nv, oracle):
    # s_g = 1 (one block holds 6*448) and block amax 6 give s = 1, so the scaled values
    # are the inputs themselves: every E2M1 tie, its float32 neighbours and their negatives.
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 2.0, 3.0, 4.0, 6.0]
    vals = []
    for t in ties:
        a = np.float32(t)
        vals += [a, np.nextafter(a, np.float32(0)), np.nextafter(a, np.float32(9))]
    vals = np.array(vals + [-v for v in vals], dtype=np.float32)
    nblk = (len(vals) + 14) // 15
    x = np.zeros((16, 16 * (nblk + 1)), dtype=np.float32)
    for b in range(nblk):
        chunk = vals[15 * b:15 * b + 15]
        x[:, 16 * b] = 6.0
        x[:, 16 * b + 1:16 * b + 1 + len(chunk)] = chunk
    x[0, -16] = 2688.0
    xt = torch.from_numpy(x)
    for mode in ["rowcol", "sr"]:
        run_case(nv, oracle, xt, mode, 99)


def test_leading_dimension_and_determinism(nv, oracle):
    x = make_input((96, 160), 5, torch.bfloat16)
    big = torch.zeros((96, 256), dtype=torch.bfloat16)
    big[:, :160] = x
    xb = big.to(dev())[:, :160]
    p = nv.quant_params(rowwise=True, colwise=True, round_col=1, rht_col=True, seed=3)
    r1, c1 = nv.nvfp4_quantize(xb, p)
    r2, c2 = nv.nvfp4_quantize(x.to(dev()), p)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        r3, c3 = nv.nvfp4_quantize(xb, p)
    torch.cuda.synchronize()
    for a, b in [(r1, r2), (c1, c2), (r1, r3), (c1, c3)]:
        assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
        assert torch.equal(a.gscale, b.gscale)
    orow, ocol = oracle.quantize(x.float().numpy(), colwise=True, round_col=1, rht_col=True, seed=3)
    assert_copy_equal(r1, orow, "ld rowwise")
    assert_copy_equal(c1, ocol, "ld colwise")


def test_empty_and_zero_tensors(nv, oracle):
    p = nv.quant_params(rowwise=True, colwise=True)
    e = torch.zeros((0, 32), dtype=torch.bfloat16, device=dev())
    r, c = nv.nvfp4_quantize(e, p)
    torch.cuda.synchronize()
    assert r.gscale.item() == 1.0 and c.gscale.item() == 1.0
    z = torch.zeros((32, 48), dtype=torch.float32)
    run_case(nv, oracle, z, "rowcol", 1)


# (272, 400): one block per lane; widths that are multiples of 1024 take the whole-wave
# layout, also into a row-strided output view
@pytest.mark.parametrize("shape,pad", [((272, 400), 0), ((48, 2048), 0), ((32, 3072), 64)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dequantize_matches_oracle(nv, oracle, out_dtype, shape, pad):
    print(f"dequantize {shape} pad={pad} {out_dtype}", flush=True)
    x = make_input(shape, 11, torch.float32).numpy()
    orow, _ = oracle.quantize(x, round_row=1, seed=4)
    gq = to_gpu_qtensor(nv, orow)
    big = torch.full((shape[0], shape[1] + pad), 7.0, dtype=out_dtype, device=dev())
    out = nv.nvfp4_dequantize(gq, out_dtype=out_dtype, out=big[:, :shape[1]])
    torch.cuda.synchronize()
    if pad:
        assert torch.all(big[:, shape[1]:] == 7.0)   # the padding columns are left alone
    ref = torch.from_numpy(oracle.dequantize(orow))
    if out_dtype == torch.bfloat16:
        ref = ref.to(torch.bfloat16)          # torch's nearest-even rounding
    assert torch.equal(out.cpu().view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                       ref.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32))


# ------------------------------------------------------------------ beyond 2 GiB
def test_quantize_input_over_2gib(nv, oracle):
    """A bf16 input of 2 GiB + 512 KiB (rowwise and columnwise copies).  A planted 7.0 in
    row 0 fixes the tensor maximum; the oracle quantizes row group 0 together with each
    checked group (both sides of the 2^31-byte offset, the last group, random groups), so
    its tensor scale is the device's, and both copies of the checked group must match."""
    from nvfp4_block_scaled_quantize_amd import synthetic
    M, K = (1 << 16) + 16, 16384                  # input bytes: 2 M K = 2^31 + 524288
    print(f"quantize a {2 * M * K} byte bf16 input, {M}x{K}", flush=True)
    x = synthetic.uniform_bf16((M, K), 31, device=dev())
    x[0, 5] = 7.0
    p = nv.quant_params(rowwise=True, colwise=True)
    r, c = nv.nvfp4_quantize(x, p)
    torch.cuda.synchronize()
    edge = (1 << 31) // (2 * K)                   # first row that starts past 2^31 bytes
    rng = np.random.default_rng(32)
    groups = sorted(set([edge // 16 - 1, edge // 16, M // 16 - 1] +
                        [int(gi) for gi in rng.integers(1, M // 16, 3)]))
    head = x[:16].float().cpu().numpy()
    for gi in groups:
        rows = slice(16 * gi, 16 * gi + 16)
        orow, ocol = oracle.quantize(np.concatenate([head, x[rows].float().cpu().numpy()]),
                                     colwise=True)
        assert r.gscale.item() == np.float32(orow.sg) and c.gscale.item() == np.float32(ocol.sg)
        assert np.array_equal(r.codes[rows].cpu().numpy(), orow.codes[16:])
        assert np.array_equal(r.scales[rows].cpu().numpy(), orow.scales[16:])
        assert np.array_equal(c.codes[:, 8 * gi:8 * gi + 8].cpu().numpy(), ocol.codes[:, 8:16])
        assert np.array_equal(c.scales[:, gi:gi + 1].cpu().numpy(), ocol.scales[:, 1:2])


# ------------------------------------------------------------------ full-size tensors
def test_full_size_activation_rowcol(nv, oracle):
    from nvfp4_block_scaled_quantize_amd import synthetic
    x = synthetic.ffn()["X"]                    # 8192 x 3072 bf16, outlier channels
    run_case(nv, oracle, x, "rowcol", 0)


def test_full_size_activation_scale46(nv, oracle):
    from nvfp4_block_scaled_quantize_amd import synthetic
    x = synthetic.ffn()["X"]                    # 8192 x 3072 bf16, outlier channels
    gr, _, orow, _ = run_case(nv, oracle, x, "46_rowcol", 0)
    s46 = (orow.scales != oracle.quantize(x.float().numpy())[0].scales).mean()
    assert 0.05 < s46 < 0.95                    # both candidates occur at full size


def test_full_size_gradient_scale46_sr(nv, oracle):
    from nvfp4_block_scaled_quantize_amd import synthetic
    t = synthetic.wgrad()                       # dY 8192 x 9216, Student-t entries
    run_case(nv, oracle, t["dY"], "46_sr_rhtcol", synthetic.RHT_SEED_WGRAD)


def test_scale46_refused_with_2d_blocks(nv):
    x = torch.zeros((32, 32), dtype=torch.bfloat16, device=dev())
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_quantize(x, nv.quant_params(block2d=True, scale46=True))


def test_full_size_weight_2d(nv, oracle):
    from nvfp4_block_scaled_quantize_amd import synthetic
    w = synthetic.normal((9216, 3072), synthetic.DATA_SEEDS["ffn"] + 1000, 0.02).to(torch.bfloat16)
    run_case(nv, oracle, w, "2d", 0)


def test_full_size_wgrad_operands(nv, oracle):
    from nvfp4_block_scaled_quantize_amd import synthetic
    t = synthetic.wgrad()
    run_case(nv, oracle, t["dY"], "wgrad_dy", synthetic.RHT_SEED_WGRAD)
    run_case(nv, oracle, t["X"], "wgrad_x", synthetic.RHT_SEED_WGRAD)


# The five quantize calls of the benchmarked 3B FFN step, with its tensors, options and seeds
# (8192 tokens, hidden 3072, FFN 9216), compared whole.
BENCH_QUANT = {
    "X_row+colRHT": ("ffn", "X", dict(rowwise=True, colwise=True, rht_col=True), True),
    "Wup_2d": ("ffn", "W_up", dict(rowwise=True, colwise=True, block2d=True), False),
    "H_row": ("ffn", "H", dict(rowwise=True), False),
    "Wdown_2d": ("ffn", "W_down", dict(rowwise=True, block2d=True), False),
    "dY_rowSR+colRHTSR": ("wgrad", "dY", dict(rowwise=True, colwise=True, round_row=1, round_col=1,
                                              rht_col=True), True),
}


@pytest.mark.parametrize("call", list(BENCH_QUANT))
def test_full_size_step_calls(nv, oracle, call):
    from nvfp4_block_scaled_quantize_amd import synthetic
    src, name, kw, seeded = BENCH_QUANT[call]
    x = getattr(synthetic, src)()[name]
    run_case(nv, oracle, x, call, synthetic.RHT_SEED_WGRAD if seeded else 0, kw=kw)


def test_full_size_dequantize_wup(nv, oracle):
    """The step's decode: W_up's rowwise 16x16 copy (9216 x 3072) to FP32, every element."""
    from nvfp4_block_scaled_quantize_amd import synthetic
    w = synthetic.ffn()["W_up"]
    print("dequantize full-size W_up 9216x3072", flush=True)
    orow, _ = oracle.quantize(w.float().numpy(), rowwise=True, colwise=True, block2d=True)
    out = nv.nvfp4_dequantize(to_gpu_qtensor(nv, orow))
    torch.cuda.synchronize()
    ref = torch.from_numpy(oracle.dequantize(orow))
    assert torch.equal(out.cpu().view(torch.int32), ref.view(torch.int32))
