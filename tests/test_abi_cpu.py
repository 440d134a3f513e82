"""C ABI checks that need no GPU: the library loads, exports every function declared in
include/nvfp4.h, and rejects invalid arguments before anything is enqueued (the calls
below never reach a kernel launch, so no HIP device is touched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    if not os.path.exists(nv.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build_hip()
    nv.load_library()
    return nv


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)
    return sorted(set(n for n in names if n not in ("sizeof",)))


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    for n in ["nvfp4_quantize", "nvfp4_dequantize", "nvfp4_gemm", "qadamw_v_encode",
              "qadamw_v_decode", "nvfp4_quantize_workspace_bytes", "qadamw_v_workspace_bytes",
              "nvfp4_status_string", "nvfp4_abi_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(nv):
    lib = ctypes.CDLL(nv.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} not exported"
    assert sorted(declared_functions()) == sorted(nv.EXPORTED)


def test_version_and_status_strings(nv):
    lib = nv.load_library()
    assert lib.nvfp4_abi_version() == nv.ABI_VERSION == 6
    assert lib.nvfp4_status_string(0) == b"ok"
    for code in range(-7, 0):
        s = lib.nvfp4_status_string(code)
        assert s and s != b"unknown status"
    assert lib.nvfp4_status_string(-99) == b"unknown status"


def _qt(base):
    return nv_mod().QTensorC(base, base + 0x10000, base + 0x20000)


def nv_mod():
    import nvfp4_block_scaled_quantize_amd as nv
    return nv


FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


def test_quantize_argument_errors(nv):
    lib = nv.load_library()
    p = nv.quant_params(rowwise=True)
    q = _qt(FAKE)
    ws = ctypes.c_void_p(FAKE + 0x40000)
    x = ctypes.c_void_p(FAKE + 0x80000)
    call = lambda *a: lib.nvfp4_quantize(*a)
    # shape: not a multiple of 16, negative, ld < cols
    assert call(x, 1, 20, 32, 32, ctypes.byref(p), ctypes.byref(q), None, ws, 1 << 20, None) == -2
    assert call(x, 1, 32, 24, 24, ctypes.byref(p), ctypes.byref(q), None, ws, 1 << 20, None) == -2
    assert call(x, 1, -16, 32, 32, ctypes.byref(p), ctypes.byref(q), None, ws, 1 << 20, None) == -2
    assert call(x, 1, 32, 32, 16, ctypes.byref(p), ctypes.byref(q), None, ws, 1 << 20, None) == -2
    # dtype
    assert call(x, 7, 32, 32, 32, ctypes.byref(p), ctypes.byref(q), None, ws, 1 << 20, None) == -4
    # null params / outputs / input
    assert call(x, 1, 32, 32, 32, None, ctypes.byref(q), None, ws, 1 << 20, None) == -1
    assert call(x, 1, 32, 32, 32, ctypes.byref(p), None, None, ws, 1 << 20, None) == -1
    assert call(None, 1, 32, 32, 32, ctypes.byref(p), ctypes.byref(q), None, ws, 1 << 20, None) == -1
    # alignment of the input and of its row pitch
    xm = ctypes.c_void_p(FAKE + 0x80008)
    assert call(xm, 1, 32, 32, 32, ctypes.byref(p), ctypes.byref(q), None, ws, 1 << 20, None) == -3
    assert call(x, 1, 32, 32, 36, ctypes.byref(p), ctypes.byref(q), None, ws, 1 << 20, None) == -3
    # workspace too small / missing
    need = lib.nvfp4_quantize_workspace_bytes(32, 32, ctypes.byref(p))
    assert need > 0
    assert call(x, 1, 32, 32, 32, ctypes.byref(p), ctypes.byref(q), None, ws, need - 1, None) == -6
    assert call(x, 1, 32, 32, 32, ctypes.byref(p), ctypes.byref(q), None, None, need, None) == -6
    # modes: no copy, bad enums, 2D with SR, RHT or 4/6 scaling
    for bad in [nv.quant_params(rowwise=False, colwise=False),
                nv.QuantParams(1, 0, 0, 0, 0, 0, 0, 2),
                nv.quant_params(block2d=True, scale46=True),
                nv.QuantParams(1, 0, 5, 0, 0, 0, 0, 0),
                nv.QuantParams(1, 0, 0, 3, 0, 0, 0, 0),
                nv.quant_params(block2d=True, round_row=nv.NVFP4_SR),
                nv.quant_params(block2d=True, rht_row=True),
                nv.quant_params(rowwise=False, colwise=True, block2d=True, rht_col=True)]:
        assert call(x, 1, 32, 32, 32, ctypes.byref(bad), ctypes.byref(q), ctypes.byref(q), ws,
                    1 << 20, None) == -5


def test_quantize_noalloc_argument_errors(nv):
    """The allocation-free variant validates like nvfp4_quantize before it looks up its
    scratch array, so none of these touches a device."""
    lib = nv.load_library()
    p = nv.quant_params(rowwise=True)
    q = _qt(FAKE)
    x = ctypes.c_void_p(FAKE + 0x80000)
    call = lambda *a: lib.nvfp4_quantize_noalloc(*a)
    assert call(x, 1, 20, 32, 32, ctypes.byref(p), ctypes.byref(q), None, None) == -2
    assert call(x, 7, 32, 32, 32, ctypes.byref(p), ctypes.byref(q), None, None) == -4
    assert call(x, 1, 32, 32, 32, None, ctypes.byref(q), None, None) == -1
    assert call(None, 1, 32, 32, 32, ctypes.byref(p), ctypes.byref(q), None, None) == -1
    assert call(ctypes.c_void_p(FAKE + 0x80008), 1, 32, 32, 32, ctypes.byref(p), ctypes.byref(q),
                None, None) == -3
    bad = nv.quant_params(block2d=True, scale46=True)
    assert call(x, 1, 32, 32, 32, ctypes.byref(bad), ctypes.byref(q), None, None) == -5
    # the scratch array holds the partial maxima of any shape (at most 768 per copy)
    for shape in [(16, 16), (8192, 3072), (65552, 16384), (1 << 20, 1 << 14)]:
        assert lib.nvfp4_quantize_workspace_bytes(*shape, ctypes.byref(p)) <= 6144


def test_quantize_lora_argument_errors(nv):
    """Shape and type limits of the fused LoRA quantize, checked before anything is enqueued."""
    lib = nv.load_library()
    p = nv.quant_params(rowwise=True)
    q = _qt(FAKE)
    x = ctypes.c_void_p(FAKE + 0x80000)
    la = ctypes.c_void_p(FAKE + 0x90000)
    t = ctypes.c_void_p(FAKE + 0xA0000)
    ws = ctypes.c_void_p(FAKE + 0xB0000)
    call = lambda rows, cols, ld, rank, dtype=1: lib.nvfp4_quantize_lora(
        x, dtype, rows, cols, ld, ctypes.byref(p), ctypes.byref(q), None, la, rank, ctypes.c_float(1.0),
        t, ws, 1 << 30, None)
    assert call(64, 256, 256, 64, dtype=0) == -4        # bfloat16 only
    assert call(64, 256, 256, 24) == -2                 # rank not a multiple of 16
    assert call(64, 256, 256, 80) == -2                 # rank above 64
    assert call(64, 200, 200, 64) == -2                 # cols not a multiple of 128
    assert call(64, 256, 1 << 24, 64) == -2             # row pitch past the 32-bit offsets
    assert call(16, 1 << 24, 1 << 24, 64) == -2         # factor past the 32-bit offsets
    # the workspace holds both copies' partial maxima and the K-parts' FP32 partials of T
    need = lib.nvfp4_quantize_lora_workspace_bytes(8192, 9216, 64)
    assert need >= 2 * 8192 * 64 * 4


def test_gemm_bf16_and_quantize_amax_argument_errors(nv):
    """The bf16-output GEMM and the quantize with caller-supplied maxima, refused before
    anything is enqueued."""
    lib = nv.load_library()
    a, b = _qt(FAKE), _qt(FAKE + 0x100000)
    c = ctypes.c_void_p(FAKE + 0x200000)
    tm = ctypes.c_void_p(FAKE + 0x280000)
    g = lambda M, N, K, cc=c, t=tm: lib.nvfp4_gemm_bf16(ctypes.byref(a), ctypes.byref(b), M, N, K,
                                                         cc, N, t, None)
    assert g(16, 16, 32, cc=None) == -1                             # no output
    assert g(16, 16, 32, cc=ctypes.c_void_p(FAKE + 0x200001)) == -3  # bf16 output misaligned
    assert g(16, 16, 32, t=ctypes.c_void_p(FAKE + 0x280002)) == -3   # tile maxima misaligned
    assert g(16, 16, 40) == -2                                       # K % 16
    assert g(0, 16, 32) == 0                                         # empty
    assert lib.nvfp4_gemm_tiles(8192, 9216) == 32 * 36
    assert lib.nvfp4_gemm_tiles(257, 1) == 2 and lib.nvfp4_gemm_tiles(0, 5) == 0
    q = _qt(FAKE + 0x300000)
    x = ctypes.c_void_p(FAKE + 0x400000)
    parts = ctypes.c_void_p(FAKE + 0x500000)
    qa = lambda params, pp=parts, n=4: lib.nvfp4_quantize_amax(
        x, 1, 64, 64, 64, ctypes.byref(params), ctypes.byref(q), ctypes.byref(q), pp, n, None)
    assert qa(nv.quant_params(rowwise=True, rht_row=True)) == -5             # rotated copy
    assert qa(nv.quant_params(rowwise=True, colwise=True, rht_col=True)) == -5
    assert qa(nv.quant_params(rowwise=True), n=0) == -2                      # no maxima
    assert qa(nv.quant_params(rowwise=True), pp=None) == -1
    assert qa(nv.quant_params(rowwise=True), pp=ctypes.c_void_p(FAKE + 0x500002)) == -3


def test_gemm_and_dequantize_argument_errors(nv):
    lib = nv.load_library()
    a, b = _qt(FAKE), _qt(FAKE + 0x100000)
    c = ctypes.c_void_p(FAKE + 0x200000)
    assert lib.nvfp4_gemm(None, ctypes.byref(b), 16, 16, 32, c, 16, None) == -1
    assert lib.nvfp4_gemm(ctypes.byref(a), ctypes.byref(b), 16, 16, 40, c, 16, None) == -2  # K % 16
    assert lib.nvfp4_gemm(ctypes.byref(a), ctypes.byref(b), 16, 16, 32, c, 8, None) == -2   # ldc < N
    assert lib.nvfp4_gemm(ctypes.byref(a), ctypes.byref(b), -1, 16, 32, c, 16, None) == -2
    assert lib.nvfp4_gemm(ctypes.byref(a), ctypes.byref(b), 16, 16, 32, None, 16, None) == -1
    am = nv.QTensorC(FAKE + 8, FAKE, FAKE)
    assert lib.nvfp4_gemm(ctypes.byref(am), ctypes.byref(b), 16, 16, 32, c, 16, None) == -3
    assert lib.nvfp4_gemm(ctypes.byref(a), ctypes.byref(b), 0, 16, 32, c, 16, None) == 0   # empty
    out = ctypes.c_void_p(FAKE + 0x300000)
    assert lib.nvfp4_dequantize(ctypes.byref(a), 16, 24, 0, out, 24, None) == -2
    assert lib.nvfp4_dequantize(ctypes.byref(a), 16, 32, 9, out, 32, None) == -4
    assert lib.nvfp4_dequantize(ctypes.byref(a), 16, 32, 0, out, 30, None) == -2
    assert lib.nvfp4_dequantize(ctypes.byref(a), 16, 32, 1, ctypes.c_void_p(FAKE + 0x300004), 32,
                                None) == -3
    assert lib.nvfp4_dequantize(None, 16, 32, 0, out, 32, None) == -1
    assert lib.nvfp4_dequantize(ctypes.byref(a), 0, 32, 0, out, 32, None) == 0


def test_qadamw_argument_errors(nv):
    lib = nv.load_library()
    q = _qt(FAKE)
    v = ctypes.c_void_p(FAKE + 0x400000)
    mu = ctypes.c_void_p(FAKE + 0x500000)
    ws = ctypes.c_void_p(FAKE + 0x600000)
    assert lib.qadamw_v_encode(v, 20, 32, 0, 1, mu, ctypes.byref(q), ws, 1 << 20, None) == -2
    assert lib.qadamw_v_encode(None, 32, 32, 0, 1, mu, ctypes.byref(q), ws, 1 << 20, None) == -1
    assert lib.qadamw_v_encode(v, 32, 32, 0, 1, None, ctypes.byref(q), ws, 1 << 20, None) == -1
    need = lib.qadamw_v_workspace_bytes(32, 32)
    assert lib.qadamw_v_encode(v, 32, 32, 0, 1, mu, ctypes.byref(q), ws, need - 1, None) == -6
    assert lib.qadamw_v_encode(ctypes.c_void_p(FAKE + 0x400004), 32, 32, 0, 1, mu,
                               ctypes.byref(q), ws, 1 << 20, None) == -3
    assert lib.qadamw_v_decode(mu, ctypes.byref(q), 32, 24, 0, 1, v, None) == -2
    assert lib.qadamw_v_decode(None, ctypes.byref(q), 32, 32, 0, 1, v, None) == -1
    assert lib.qadamw_v_decode(mu, ctypes.byref(q), 0, 32, 0, 1, v, None) == 0


def test_python_binding_refuses_cpu_tensors(nv):
    import torch
    x = torch.zeros((16, 16), dtype=torch.bfloat16)
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_quantize(x, nv.quant_params())
