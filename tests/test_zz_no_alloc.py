"""nvfp4_quantize_noalloc, the quantize entry point without a workspace (for callers that
cannot allocate), called through the C ABI and compared with nvfp4_quantize bit for bit.

Two calls in a row on the library's per-device scratch array: first the full-size 3B
activation (8192 x 3072 bf16, row + column-rotated copies; the first pass then has its
maximum of 768 workgroups), then a smaller f32 input with every option on, so the second
call reads back only the partials it wrote itself.  A third call repeats the first on a
second stream after synchronising, with a ragged bf16 shape.
"""
import ctypes

import pytest
import torch

from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load_library()
    return nv


def noalloc_via_abi(nv, x, p):
    """Call the C entry point directly (ctypes), into copies allocated beforehand."""
    lib = nv.load_library()
    R, C = x.shape
    row = nv.QTensor.empty(R, C, x.device) if p.rowwise else None
    col = nv.QTensor.empty(C, R, x.device) if p.colwise else None
    rc_ = row.c() if row is not None else None
    cc_ = col.c() if col is not None else None
    dt = nv.NVFP4_BF16 if x.dtype == torch.bfloat16 else nv.NVFP4_F32
    stream = ctypes.c_void_p(torch.cuda.current_stream(x.device).cuda_stream)
    rc = lib.nvfp4_quantize_noalloc(ctypes.c_void_p(x.data_ptr()), dt, R, C, x.stride(0),
                                    ctypes.byref(p),
                                    ctypes.byref(rc_) if rc_ is not None else None,
                                    ctypes.byref(cc_) if cc_ is not None else None, stream)
    assert rc == 0, lib.nvfp4_status_string(rc)
    return row, col


def assert_same(a, b, what):
    assert torch.equal(a.codes, b.codes), f"{what}: codes differ"
    assert torch.equal(a.scales, b.scales), f"{what}: scales differ"
    assert torch.equal(a.gscale, b.gscale), f"{what}: tensor scales differ"


def check(nv, x, kw, seed, what):
    print(f"noalloc {what}: {tuple(x.shape)} {x.dtype} {kw} seed={seed:#x}", flush=True)
    p = nv.quant_params(seed=seed, **kw)
    gr, gc = noalloc_via_abi(nv, x, p)
    wr, wc = nv.nvfp4_quantize(x, p)
    torch.cuda.synchronize()
    if p.rowwise:
        assert_same(gr, wr, f"{what} rowwise")
    if p.colwise:
        assert_same(gc, wc, f"{what} colwise")


def test_noalloc_matches_quantize_two_calls(nv):
    from nvfp4_block_scaled_quantize_amd import synthetic
    x_big = synthetic.ffn()["X"].to(dev())                     # 8192 x 3072 bf16
    assert nv.nvfp4_quantize_workspace_bytes(8192, 3072, nv.quant_params()) == 6144
    check(nv, x_big, dict(rowwise=True, colwise=True, rht_col=True), synthetic.RHT_SEED_WGRAD,
          "first (full size)")
    x_small = synthetic.spiky((272, 400), 91).to(dev())
    check(nv, x_small, dict(rowwise=True, colwise=True, round_row=1, round_col=1, rht_row=True,
                            rht_col=True, scale46=True), 0x77, "second (smaller)")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        x_rag = synthetic.spiky((528, 144), 92).to(torch.bfloat16).to(dev())
        check(nv, x_rag, dict(rowwise=True, colwise=True, round_col=1, rht_col=True), 0x78,
              "third (other stream)")


def test_noalloc_argument_errors_match_quantize(nv):
    lib = nv.load_library()
    x = torch.zeros((32, 48), dtype=torch.float32, device=dev())
    q = nv.QTensor.empty(32, 48, dev()).c()
    p = nv.quant_params()
    xp = ctypes.c_void_p(x.data_ptr())
    assert lib.nvfp4_quantize_noalloc(xp, 0, 20, 48, 48, ctypes.byref(p), ctypes.byref(q), None,
                                      None) == -2
    assert lib.nvfp4_quantize_noalloc(xp, 0, 32, 48, 48, ctypes.byref(p), None, None, None) == -1
    bad = nv.quant_params(block2d=True, scale46=True)
    assert lib.nvfp4_quantize_noalloc(xp, 0, 32, 48, 48, ctypes.byref(bad), ctypes.byref(q), None,
                                      None) == -5
