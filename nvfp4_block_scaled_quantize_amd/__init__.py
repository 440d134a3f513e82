"""NVFP4 quantized-linear hot path for AMD Instinct MI355X (gfx950).

Thin ctypes binding of the C ABI in ``include/nvfp4.h`` (``libnvfp4.so``, built from
``csrc/*.hip``).  This module only marshals arguments: torch supplies device memory
and the current HIP stream, and every step of the method runs in the library's
kernels.  There is no CPU fallback; if the library is missing or no GPU is present the
calls raise.

Entry points (same names as the C ABI):
  nvfp4_quantize     rowwise and/or columnwise NVFP4 copies of a bf16/fp32 matrix
  nvfp4_dequantize   decode one copy to fp32 or bf16
  nvfp4_gemm         W4A4 GEMM C = A B^T over two K-major copies, fp32 output
  qadamw_v_encode    Q-AdamW second-moment encode (sqrt, bf16 tile mean, RHT, NVFP4)
  qadamw_v_decode    its inverse
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

NVFP4_F32, NVFP4_BF16 = 0, 1
NVFP4_RNE, NVFP4_SR = 0, 1
NVFP4_BLOCK_1D, NVFP4_BLOCK_2D = 0, 1

EXPORTED = ["nvfp4_quantize_workspace_bytes", "nvfp4_quantize", "nvfp4_dequantize",
            "nvfp4_gemm", "qadamw_v_workspace_bytes", "qadamw_v_encode", "qadamw_v_decode",
            "nvfp4_status_string", "nvfp4_abi_version", "qadamw_step_workspace_bytes",
            "qadamw_step", "nvfp4_gemm_lora", "nvfp4_quantize_lora_workspace_bytes",
            "nvfp4_quantize_lora", "nvfp4_requantize_cols_workspace_bytes",
            "nvfp4_requantize_cols", "nvfp4_gemm_axpby", "nvfp4_ns_step_workspace_bytes",
            "nvfp4_ns_step", "nvfp4_quantize_noalloc", "nvfp4_quantize_amax", "nvfp4_gemm_tiles",
            "nvfp4_gemm_bf16"]


class Nvfp4Error(RuntimeError):
    pass


class QuantParams(ctypes.Structure):
    _fields_ = [("rowwise", ctypes.c_int32), ("colwise", ctypes.c_int32),
                ("block", ctypes.c_int32), ("round_row", ctypes.c_int32),
                ("round_col", ctypes.c_int32), ("rht_row", ctypes.c_int32),
                ("rht_col", ctypes.c_int32), ("scale46", ctypes.c_int32),
                ("seed", ctypes.c_uint64)]


class QAdamWStepParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("grad_coef", ctypes.c_float), ("bias1", ctypes.c_float), ("bias2", ctypes.c_float),
                ("m_rht_seed", ctypes.c_uint64), ("m_sr_seed", ctypes.c_uint64),
                ("v_seed", ctypes.c_uint64), ("v_use_signs", ctypes.c_int32)]


class QTensorC(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("gscale", ctypes.c_void_p)]


_lib = None
ABI_VERSION = 6   # NVFP4_ABI_VERSION of include/nvfp4.h this binding matches


def load_library(path: Optional[str] = None):
    """Load libnvfp4.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise Nvfp4Error(f"{p} is missing: build the HIP library first (__graft_entry__.build())")
    lib = ctypes.CDLL(p)
    vp, i64, i32, u64, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64,
                             ctypes.c_size_t)
    P = ctypes.POINTER
    lib.nvfp4_quantize_workspace_bytes.restype = sz
    lib.nvfp4_quantize_workspace_bytes.argtypes = [i64, i64, P(QuantParams)]
    lib.nvfp4_quantize.restype = ctypes.c_int
    lib.nvfp4_quantize.argtypes = [vp, ctypes.c_int, i64, i64, i64, P(QuantParams),
                                   P(QTensorC), P(QTensorC), vp, sz, vp]
    lib.nvfp4_quantize_noalloc.restype = ctypes.c_int
    lib.nvfp4_quantize_noalloc.argtypes = [vp, ctypes.c_int, i64, i64, i64, P(QuantParams),
                                           P(QTensorC), P(QTensorC), vp]
    lib.nvfp4_dequantize.restype = ctypes.c_int
    lib.nvfp4_dequantize.argtypes = [P(QTensorC), i64, i64, ctypes.c_int, vp, i64, vp]
    lib.nvfp4_gemm.restype = ctypes.c_int
    lib.nvfp4_gemm.argtypes = [P(QTensorC), P(QTensorC), i64, i64, i64, vp, i64, vp]
    lib.nvfp4_gemm_tiles.restype = i64
    lib.nvfp4_gemm_tiles.argtypes = [i64, i64]
    lib.nvfp4_gemm_bf16.restype = ctypes.c_int
    lib.nvfp4_gemm_bf16.argtypes = [P(QTensorC), P(QTensorC), i64, i64, i64, vp, i64, vp, vp]
    lib.nvfp4_quantize_amax.restype = ctypes.c_int
    lib.nvfp4_quantize_amax.argtypes = [vp, ctypes.c_int, i64, i64, i64, P(QuantParams),
                                        P(QTensorC), P(QTensorC), vp, i64, vp]
    lib.nvfp4_quantize_lora_workspace_bytes.restype = sz
    lib.nvfp4_quantize_lora_workspace_bytes.argtypes = [i64, i64, i64]
    lib.nvfp4_quantize_lora.restype = ctypes.c_int
    lib.nvfp4_quantize_lora.argtypes = [vp, ctypes.c_int, i64, i64, i64, P(QuantParams), P(QTensorC),
                                        P(QTensorC), vp, i64, ctypes.c_float, vp, vp, sz, vp]
    lib.nvfp4_requantize_cols_workspace_bytes.restype = sz
    lib.nvfp4_requantize_cols_workspace_bytes.argtypes = [i64, i64]
    lib.nvfp4_requantize_cols.restype = ctypes.c_int
    lib.nvfp4_requantize_cols.argtypes = [P(QTensorC), i64, i64, P(QuantParams), P(QTensorC), vp,
                                          sz, vp]
    lib.nvfp4_gemm_axpby.restype = ctypes.c_int
    lib.nvfp4_gemm_axpby.argtypes = [P(QTensorC), P(QTensorC), i64, i64, i64, ctypes.c_float, vp, i64,
                                     ctypes.c_float, vp, i64, vp]
    lib.nvfp4_ns_step_workspace_bytes.restype = sz
    lib.nvfp4_ns_step_workspace_bytes.argtypes = [i64, i64]
    lib.nvfp4_ns_step.restype = ctypes.c_int
    lib.nvfp4_ns_step.argtypes = [vp, i64, i64, ctypes.c_float, ctypes.c_float, ctypes.c_float, u64,
                                  i32, vp, sz, vp]
    lib.nvfp4_gemm_lora.restype = ctypes.c_int
    lib.nvfp4_gemm_lora.argtypes = [P(QTensorC), P(QTensorC), i64, i64, i64, vp, i64, vp, vp, i64,
                                    vp]
    lib.qadamw_v_workspace_bytes.restype = sz
    lib.qadamw_v_workspace_bytes.argtypes = [i64, i64]
    lib.qadamw_v_encode.restype = ctypes.c_int
    lib.qadamw_v_encode.argtypes = [vp, i64, i64, u64, i32, vp, P(QTensorC), vp, sz, vp]
    lib.qadamw_v_decode.restype = ctypes.c_int
    lib.qadamw_v_decode.argtypes = [vp, P(QTensorC), i64, i64, u64, i32, vp, vp]
    lib.qadamw_step_workspace_bytes.restype = sz
    lib.qadamw_step_workspace_bytes.argtypes = [i64, i64]
    lib.qadamw_step.restype = ctypes.c_int
    lib.qadamw_step.argtypes = [vp, vp, ctypes.c_int, i64, i64, P(QTensorC), P(QTensorC), vp,
                                P(QTensorC), vp, P(QTensorC), P(QAdamWStepParams), vp, sz, vp]
    lib.nvfp4_status_string.restype = ctypes.c_char_p
    lib.nvfp4_status_string.argtypes = [ctypes.c_int]
    lib.nvfp4_abi_version.restype = ctypes.c_int
    lib.nvfp4_abi_version.argtypes = []
    if lib.nvfp4_abi_version() != ABI_VERSION:
        raise Nvfp4Error(f"{p} has ABI version {lib.nvfp4_abi_version()}, this binding expects "
                         f"{ABI_VERSION}: rebuild the HIP library (__graft_entry__.build())")
    if path is None:
        _lib = lib
    return lib


def _check(rc):
    if rc != 0:
        msg = load_library().nvfp4_status_string(rc).decode()
        raise Nvfp4Error(f"nvfp4 status {rc}: {msg}")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise Nvfp4Error("nvfp4 kernels take GPU tensors only (no CPU path)")


@dataclass
class QTensor:
    """One quantized copy on the GPU: codes [n][k/2] u8, scales [n][k/16] u8, gscale [1] f32."""
    codes: torch.Tensor
    scales: torch.Tensor
    gscale: torch.Tensor

    @property
    def shape(self):
        return self.codes.shape[0], self.codes.shape[1] * 2

    def c(self):
        return QTensorC(self.codes.data_ptr(), self.scales.data_ptr(), self.gscale.data_ptr())

    @staticmethod
    def empty(n, k, device):
        return QTensor(torch.empty((n, k // 2), dtype=torch.uint8, device=device),
                       torch.empty((n, k // 16), dtype=torch.uint8, device=device),
                       torch.empty((1,), dtype=torch.float32, device=device))


def quant_params(rowwise=True, colwise=False, block2d=False, round_row=NVFP4_RNE,
                 round_col=NVFP4_RNE, rht_row=False, rht_col=False, seed=0, scale46=False):
    return QuantParams(int(rowwise), int(colwise), NVFP4_BLOCK_2D if block2d else NVFP4_BLOCK_1D,
                       int(round_row), int(round_col), int(rht_row), int(rht_col), int(scale46),
                       int(seed) & 0xFFFFFFFFFFFFFFFF)


def nvfp4_quantize_workspace_bytes(rows, cols, params):
    return int(load_library().nvfp4_quantize_workspace_bytes(rows, cols, ctypes.byref(params)))


def nvfp4_quantize(x, params, row_out=None, col_out=None, workspace=None, amax_parts=None):
    """Quantize a 2-D bf16/fp32 CUDA tensor (row stride may exceed its width).

    Returns (row_copy, col_copy); a copy not requested is None.  Output buffers and the
    workspace are allocated with torch unless passed in.  amax_parts: a float32 CUDA tensor
    of partial maxima of |x| (e.g. nvfp4_gemm_bf16's tile maxima) that replaces the amax
    pass (copies without a Hadamard rotation only; no workspace is used)."""
    lib = load_library()
    _require_cuda(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise Nvfp4Error("x must be a 2-D tensor with unit column stride")
    if x.dtype == torch.bfloat16:
        dt = NVFP4_BF16
    elif x.dtype == torch.float32:
        dt = NVFP4_F32
    else:
        raise Nvfp4Error(f"unsupported dtype {x.dtype}")
    R, C = x.shape
    dev = x.device
    if params.rowwise and row_out is None:
        row_out = QTensor.empty(R, C, dev)
    if params.colwise and col_out is None:
        col_out = QTensor.empty(C, R, dev)
    rc_ = row_out.c() if params.rowwise else None
    cc_ = col_out.c() if params.colwise else None
    if amax_parts is not None:
        _require_cuda(amax_parts)
        if amax_parts.dtype != torch.float32 or not amax_parts.is_contiguous():
            raise Nvfp4Error("amax_parts must be a contiguous float32 tensor")
        _check(lib.nvfp4_quantize_amax(_ptr(x), dt, R, C, x.stride(0), ctypes.byref(params),
                                       ctypes.byref(rc_) if rc_ is not None else None,
                                       ctypes.byref(cc_) if cc_ is not None else None,
                                       _ptr(amax_parts), amax_parts.numel(), _stream(dev)))
        return (row_out if params.rowwise else None), (col_out if params.colwise else None)
    need = nvfp4_quantize_workspace_bytes(R, C, params)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    rc = lib.nvfp4_quantize(_ptr(x), dt, R, C, x.stride(0), ctypes.byref(params),
                            ctypes.byref(rc_) if rc_ is not None else None,
                            ctypes.byref(cc_) if cc_ is not None else None,
                            _ptr(workspace), workspace.numel(), _stream(dev))
    _check(rc)
    return (row_out if params.rowwise else None), (col_out if params.colwise else None)


def nvfp4_quantize_noalloc(x, params, row_out, col_out=None):
    """nvfp4_quantize into caller-allocated copies with no workspace: the library keeps the
    partial maxima in its per-device scratch array (calls on one device must not overlap)."""
    lib = load_library()
    _require_cuda(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise Nvfp4Error("x must be a 2-D tensor with unit column stride")
    if x.dtype == torch.bfloat16:
        dt = NVFP4_BF16
    elif x.dtype == torch.float32:
        dt = NVFP4_F32
    else:
        raise Nvfp4Error(f"unsupported dtype {x.dtype}")
    R, C = x.shape
    rc_ = row_out.c() if params.rowwise else None
    cc_ = col_out.c() if params.colwise else None
    with torch.cuda.device(x.device):
        _check(lib.nvfp4_quantize_noalloc(_ptr(x), dt, R, C, x.stride(0), ctypes.byref(params),
                                          ctypes.byref(rc_) if rc_ is not None else None,
                                          ctypes.byref(cc_) if cc_ is not None else None,
                                          _stream(x.device)))
    return row_out, col_out


def nvfp4_dequantize(q, out_dtype=torch.float32, out=None):
    lib = load_library()
    _require_cuda(q.codes)
    n, k = q.shape
    if out is None:
        out = torch.empty((n, k), dtype=out_dtype, device=q.codes.device)
    dt = NVFP4_BF16 if out.dtype == torch.bfloat16 else NVFP4_F32
    qc = q.c()
    _check(lib.nvfp4_dequantize(ctypes.byref(qc), n, k, dt, _ptr(out), out.stride(0),
                                _stream(out.device)))
    return out


def nvfp4_gemm(a, b, out=None):
    """C = A B^T (A: M x K copy, B: N x K copy), FP32."""
    lib = load_library()
    _require_cuda(a.codes, b.codes)
    M, K = a.shape
    N, K2 = b.shape
    if K != K2:
        raise Nvfp4Error(f"K mismatch {K} vs {K2}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.codes.device)
    ac, bc = a.c(), b.c()
    _check(lib.nvfp4_gemm(ctypes.byref(ac), ctypes.byref(bc), M, N, K, _ptr(out), out.stride(0),
                          _stream(out.device)))
    return out


def nvfp4_gemm_bf16(a, b, out=None, tile_amax=None):
    """C = A B^T rounded to bfloat16, with each 256 x 256 tile's maximum of |C|; returns
    (out, tile_amax).  tile_amax: float32 [nvfp4_gemm_tiles(M, N)] (allocated if None)."""
    lib = load_library()
    _require_cuda(a.codes, b.codes)
    M, K = a.shape
    N, K2 = b.shape
    if K != K2:
        raise Nvfp4Error(f"K mismatch {K} vs {K2}")
    dev = a.codes.device
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if out.dtype != torch.bfloat16 or out.dim() != 2 or out.stride(1) != 1:
        raise Nvfp4Error("out must be a 2-D bfloat16 tensor with unit column stride")
    if tile_amax is None:
        tile_amax = torch.empty((max(int(lib.nvfp4_gemm_tiles(M, N)), 1),), dtype=torch.float32,
                                device=dev)
    ac, bc = a.c(), b.c()
    _check(lib.nvfp4_gemm_bf16(ctypes.byref(ac), ctypes.byref(bc), M, N, K, _ptr(out),
                               out.stride(0), _ptr(tile_amax), _stream(dev)))
    return out, tile_amax


def nvfp4_quantize_lora(x, params, lora_a, beta, row_out=None, col_out=None, lora_t=None,
                        workspace=None):
    """nvfp4_quantize of a bfloat16 x with the LoRA-SVD down-projection
    lora_t = BF16(beta x lora_a^T) fused into its first pass; returns (row, col, lora_t)."""
    lib = load_library()
    _require_cuda(x, lora_a)
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise Nvfp4Error("x must be a 2-D bfloat16 tensor with unit column stride")
    if lora_a.dtype != torch.bfloat16 or not lora_a.is_contiguous() or lora_a.dim() != 2:
        raise Nvfp4Error("lora_a must be a contiguous 2-D bfloat16 tensor")
    R, C = x.shape
    rank = lora_a.shape[0]
    if lora_a.shape[1] != C:
        raise Nvfp4Error(f"lora_a has {lora_a.shape[1]} columns, x {C}")
    dev = x.device
    if params.rowwise and row_out is None:
        row_out = QTensor.empty(R, C, dev)
    if params.colwise and col_out is None:
        col_out = QTensor.empty(C, R, dev)
    if lora_t is None:
        lora_t = torch.empty((R, rank), dtype=torch.bfloat16, device=dev)
    need = int(lib.nvfp4_quantize_lora_workspace_bytes(R, C, rank))
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    rc_ = row_out.c() if params.rowwise else None
    cc_ = col_out.c() if params.colwise else None
    _check(lib.nvfp4_quantize_lora(_ptr(x), NVFP4_BF16, R, C, x.stride(0), ctypes.byref(params),
                                   ctypes.byref(rc_) if rc_ is not None else None,
                                   ctypes.byref(cc_) if cc_ is not None else None,
                                   _ptr(lora_a), rank, float(beta), _ptr(lora_t), _ptr(workspace),
                                   workspace.numel(), _stream(dev)))
    return (row_out if params.rowwise else None), (col_out if params.colwise else None), lora_t


def nvfp4_requantize_cols(row_q, params, col_out=None, workspace=None):
    """The columnwise copy of a rowwise copy's decoded values (Full-Stack FP4 eq. (2)'s
    Q_16x1(H^T Q_1x16(X))); params ask for the columnwise copy only."""
    lib = load_library()
    _require_cuda(row_q.codes)
    R, C = row_q.shape
    dev = row_q.codes.device
    if col_out is None:
        col_out = QTensor.empty(C, R, dev)
    need = int(lib.nvfp4_requantize_cols_workspace_bytes(R, C))
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    rq, cq = row_q.c(), col_out.c()
    _check(lib.nvfp4_requantize_cols(ctypes.byref(rq), R, C, ctypes.byref(params), ctypes.byref(cq),
                                     _ptr(workspace), workspace.numel(), _stream(dev)))
    return col_out


def nvfp4_gemm_axpby(a, b, alpha, d, beta, out=None):
    """C = alpha * A B^T + beta * d (d float32 [M][N]; out may be d)."""
    lib = load_library()
    _require_cuda(a.codes, b.codes, d)
    M, K = a.shape
    N, K2 = b.shape
    if K != K2:
        raise Nvfp4Error(f"K mismatch {K} vs {K2}")
    if d.dtype != torch.float32 or d.dim() != 2 or d.shape != (M, N) or d.stride(1) != 1:
        raise Nvfp4Error("d must be a float32 [M][N] tensor with unit column stride")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.codes.device)
    ac, bc = a.c(), b.c()
    _check(lib.nvfp4_gemm_axpby(ctypes.byref(ac), ctypes.byref(bc), M, N, K, float(alpha), _ptr(d),
                                d.stride(0), float(beta), _ptr(out), out.stride(0), _stream(out.device)))
    return out


def nvfp4_ns_step(x, a, b, c, seed, scale46=True, workspace=None):
    """One quantized Newton-Schulz iteration on x (float32 [m][n], contiguous), in place."""
    lib = load_library()
    _require_cuda(x)
    if x.dtype != torch.float32 or x.dim() != 2 or not x.is_contiguous():
        raise Nvfp4Error("x must be a contiguous 2-D float32 tensor")
    m, n = x.shape
    if workspace is None:
        workspace = torch.empty(max(int(lib.nvfp4_ns_step_workspace_bytes(m, n)), 256),
                                dtype=torch.uint8, device=x.device)
    _check(lib.nvfp4_ns_step(_ptr(x), m, n, float(a), float(b), float(c),
                             int(seed) & 0xFFFFFFFFFFFFFFFF, int(scale46), _ptr(workspace),
                             workspace.numel(), _stream(x.device)))
    return x


def nvfp4_gemm_lora(a, b, t, lb, out=None):
    """C = A B^T + t lb^T: the W4A4 GEMM with the LoRA-SVD up-projection in its epilogue
    (t [M][r], lb [N][r] contiguous bfloat16 on the GPU, r a multiple of 16)."""
    lib = load_library()
    _require_cuda(a.codes, b.codes, t, lb)
    M, K = a.shape
    N, K2 = b.shape
    if K != K2:
        raise Nvfp4Error(f"K mismatch {K} vs {K2}")
    if t.dtype != torch.bfloat16 or lb.dtype != torch.bfloat16 or not t.is_contiguous() \
            or not lb.is_contiguous() or t.dim() != 2 or lb.dim() != 2:
        raise Nvfp4Error("t and lb must be contiguous 2-D bfloat16 tensors")
    r = t.shape[1]
    if t.shape[0] != M or lb.shape != (N, r):
        raise Nvfp4Error(f"low-rank factors {tuple(t.shape)}, {tuple(lb.shape)} do not match "
                         f"M={M}, N={N}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.codes.device)
    ac, bc = a.c(), b.c()
    _check(lib.nvfp4_gemm_lora(ctypes.byref(ac), ctypes.byref(bc), M, N, K, _ptr(out), out.stride(0),
                               _ptr(t), _ptr(lb), r, _stream(out.device)))
    return out


def qadamw_step_params(lr, beta1, beta2, eps, weight_decay, grad_coef=1.0, bias1=1.0, bias2=1.0,
                       m_rht_seed=0, m_sr_seed=0, v_seed=0, v_use_signs=True):
    return QAdamWStepParams(lr, beta1, beta2, eps, weight_decay, grad_coef, bias1, bias2,
                            int(m_rht_seed) & 0xFFFFFFFFFFFFFFFF, int(m_sr_seed) & 0xFFFFFFFFFFFFFFFF,
                            int(v_seed) & 0xFFFFFFFFFFFFFFFF, int(v_use_signs))


def qadamw_step_workspace_bytes(rows, cols):
    return int(load_library().qadamw_step_workspace_bytes(rows, cols))


def qadamw_step(w, g, m, mu, v, params, m_out=None, mu_out=None, v_out=None, workspace=None):
    """One quantized-state AdamW step: updates w (f32, in place) and returns the new states
    (m_out, mu_out, v_out), allocated here unless passed (they must not alias the inputs)."""
    lib = load_library()
    _require_cuda(w, g)
    if w.dtype != torch.float32 or not w.is_contiguous() or w.dim() != 2:
        raise Nvfp4Error("w must be a contiguous 2-D float32 tensor")
    if g.shape != w.shape or not g.is_contiguous() or g.dtype not in (torch.float32, torch.bfloat16):
        raise Nvfp4Error("g must be a contiguous float32/bfloat16 tensor shaped like w")
    R, C = w.shape
    d = w.device
    m_out = m_out if m_out is not None else QTensor.empty(R, C, d)
    v_out = v_out if v_out is not None else QTensor.empty(R, C, d)
    mu_out = mu_out if mu_out is not None else torch.empty((R // 16, C // 16), dtype=torch.int16, device=d)
    if workspace is None:
        workspace = torch.empty(max(qadamw_step_workspace_bytes(R, C), 16),
                                dtype=torch.uint8, device=d)
    dt = NVFP4_BF16 if g.dtype == torch.bfloat16 else NVFP4_F32
    mi, mo, vi, vo = m.c(), m_out.c(), v.c(), v_out.c()
    _check(lib.qadamw_step(_ptr(w), _ptr(g), dt, R, C, ctypes.byref(mi), ctypes.byref(mo), _ptr(mu),
                           ctypes.byref(vi), _ptr(mu_out), ctypes.byref(vo), ctypes.byref(params),
                           _ptr(workspace), workspace.numel(), _stream(d)))
    return m_out, mu_out, v_out


def qadamw_v_workspace_bytes(rows, cols):
    return int(load_library().qadamw_v_workspace_bytes(rows, cols))


def qadamw_v_encode(v, seed=0, use_signs=True, mu=None, q=None, workspace=None):
    lib = load_library()
    _require_cuda(v)
    if v.dtype != torch.float32 or v.dim() != 2 or not v.is_contiguous():
        raise Nvfp4Error("v must be a contiguous 2-D float32 tensor")
    R, C = v.shape
    dev = v.device
    if mu is None:
        mu = torch.empty((R // 16, C // 16), dtype=torch.int16, device=dev)
    if q is None:
        q = QTensor.empty(R, C, dev)
    need = qadamw_v_workspace_bytes(R, C)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    qc = q.c()
    _check(lib.qadamw_v_encode(_ptr(v), R, C, int(seed) & 0xFFFFFFFFFFFFFFFF, int(use_signs),
                               _ptr(mu), ctypes.byref(qc), _ptr(workspace), workspace.numel(),
                               _stream(dev)))
    return mu, q


def qadamw_v_decode(mu, q, seed=0, use_signs=True, out=None):
    lib = load_library()
    _require_cuda(mu, q.codes)
    R, C = q.shape
    if out is None:
        out = torch.empty((R, C), dtype=torch.float32, device=q.codes.device)
    qc = q.c()
    _check(lib.qadamw_v_decode(_ptr(mu), ctypes.byref(qc), R, C, int(seed) & 0xFFFFFFFFFFFFFFFF,
                               int(use_signs), _ptr(out), _stream(out.device)))
    return out


def abi_version():
    return load_library().nvfp4_abi_version()
