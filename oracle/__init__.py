"""CPU oracle for the NVFP4 quantized linear path (ctypes binding of nvfp4_oracle.c).

TEST INFRASTRUCTURE ONLY.  The only code that may import this package is the
test suite, the package smoke check (``__graft_entry__.smoke``) and the CPU
baseline leg of ``bench.py``.  The GPU library never imports, links or calls
it, and it shares no code with the GPU library: only the seeded input
generators are common to both sides.

All arrays are numpy; binary32 inputs only (a bfloat16 tensor is widened to
binary32 exactly before it is passed in).  Functions raise ValueError on the
argument errors the C code reports.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-fPIC", "-shared"]


def build():
    """Compile the oracle into oracle/liboracle.so (plain gcc, no GPU code)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64, u64, u32, f32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float
    sig = {
        "or_e2m1_value": (ctypes.c_double, [ctypes.c_int]),
        "or_e2m1_rne": (ctypes.c_int, [f32]),
        "or_e2m1_sr": (ctypes.c_int, [f32, u32]),
        "or_e4m3_encode": (ctypes.c_uint8, [f32]),
        "or_e4m3_value": (ctypes.c_double, [ctypes.c_uint8]),
        "or_bf16_rne": (ctypes.c_uint16, [f32]),
        "or_bf16_value": (f32, [ctypes.c_uint16]),
        "or_philox4x32_10": (None, [P, P, P]),
        "or_sr_bits": (u32, [u64, u32, u64]),
        "or_rht_signs": (None, [u64, P]),
        "or_wht16": (None, [P]),
        "or_rht16_forward": (None, [P, P]),
        "or_rht16_inverse": (None, [P, P]),
        "or_quantize_rows": (ctypes.c_int, [P, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, u64, u32, P, P, P]),
        "or_dequantize": (ctypes.c_int, [P, P, f32, i64, i64, P]),
        "or_gemm_f64": (ctypes.c_int, [P, P, f32, P, P, f32, i64, i64, i64, P, P]),
        "or_gemm_f64_entries": (ctypes.c_int, [P, P, f32, P, P, f32, i64, i64, i64, P, P, i64,
                                               P, P]),
        "or_qadamw_v_encode": (ctypes.c_int, [P, i64, i64, u64, ctypes.c_int, P, P, P, P]),
        "or_qadamw_v_decode": (ctypes.c_int, [P, P, P, f32, i64, i64, u64, ctypes.c_int, P]),
        "or_scale46_disagreements": (ctypes.c_int, [P, i64, i64, ctypes.c_int, u64, P, P, P]),
        "or_num_threads": (ctypes.c_int, []),
        "or_set_num_threads": (None, [ctypes.c_int]),
        "or_lora_down": (ctypes.c_int, [P, i64, i64, P, i64, f32, P, P, P]),
        "or_gemm_lora_f64": (ctypes.c_int, [P, P, f32, P, P, f32, i64, i64, i64, P, P, i64, P, P]),
        "or_gemm_lora_f64_entries": (ctypes.c_int, [P, P, f32, P, P, f32, i64, i64, i64, P, P, i64,
                                                    P, P, i64, P, P]),
        "or_qadamw_step": (ctypes.c_int, [P, P, i64, i64, P, P, f32, P, P, P, f32, P, u64, u64, u64,
                                          ctypes.c_int, P, P, P, P, P, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


# ---------------------------------------------------------------- scalar formats
def e2m1_value(code):
    return _load().or_e2m1_value(int(code))


def e2m1_rne(u):
    return _load().or_e2m1_rne(float(u))


def e2m1_sr(u, r16):
    return _load().or_e2m1_sr(float(u), int(r16))


def e4m3_encode(v):
    return int(_load().or_e4m3_encode(float(v)))


def e4m3_value(code):
    return _load().or_e4m3_value(int(code))


def bf16_rne(v):
    return int(_load().or_bf16_rne(float(v)))


def bf16_value(b):
    return _load().or_bf16_value(int(b))


def num_threads():
    return _load().or_num_threads()


def set_num_threads(n):
    """Thread count of the C oracle's row loops (timing only: results do not depend on it)."""
    _load().or_set_num_threads(int(n))


# ---------------------------------------------------------------- generator, transforms
def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    _load().or_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_bits(seed, copy_id, j):
    return int(_load().or_sr_bits(int(seed), int(copy_id), int(j)))


def rht_signs(seed):
    out = np.zeros(16, dtype=np.float32)
    _load().or_rht_signs(int(seed), _ptr(out))
    return out


def wht16(v):
    a = np.array(v, dtype=np.float32).copy()
    assert a.shape == (16,)
    _load().or_wht16(_ptr(a))
    return a


def rht16_forward(v, sgn):
    a = np.array(v, dtype=np.float32).copy()
    s = np.ascontiguousarray(sgn, dtype=np.float32)
    _load().or_rht16_forward(_ptr(a), _ptr(s))
    return a


def rht16_inverse(v, sgn):
    a = np.array(v, dtype=np.float32).copy()
    s = np.ascontiguousarray(sgn, dtype=np.float32)
    _load().or_rht16_inverse(_ptr(a), _ptr(s))
    return a


# ---------------------------------------------------------------- quantize / dequantize
RNE, SR = 0, 1


class QTensor:
    """One quantized copy: codes [n][k/2] uint8, scales [n][k/16] uint8, sg float."""

    def __init__(self, codes, scales, sg):
        self.codes, self.scales, self.sg = codes, scales, float(sg)

    @property
    def shape(self):
        return self.codes.shape[0], self.codes.shape[1] * 2


def quantize_rows(x, block2d=False, rounding=RNE, rht=False, seed=0, copy_id=0, scale46=False):
    """Quantize x[n][k] along its rows (blocks of 16 consecutive row elements, or
    16x16 tiles); scale46 selects 4/6 adaptive block scaling (1x16 blocks only)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n, k = x.shape
    codes = np.zeros((n, k // 2), dtype=np.uint8)
    scales = np.zeros((n, k // 16), dtype=np.uint8)
    sg = ctypes.c_float(0.0)
    rc = _load().or_quantize_rows(_ptr(x), n, k, int(block2d), int(rounding), int(rht),
                                  int(scale46), int(seed), int(copy_id), _ptr(codes),
                                  _ptr(scales), ctypes.byref(sg))
    _check(rc, "quantize_rows")
    return QTensor(codes, scales, sg.value)


def quantize(x, rowwise=True, colwise=False, block2d=False, round_row=RNE, round_col=RNE,
             rht_row=False, rht_col=False, seed=0, scale46=False):
    """Rowwise copy = quantization of x along rows; columnwise copy = the same
    quantization applied to x transposed (blocks of 16 consecutive rows of x)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    row = col = None
    if rowwise:
        row = quantize_rows(x, block2d, round_row, rht_row, seed, copy_id=0, scale46=scale46)
    if colwise:
        col = quantize_rows(np.ascontiguousarray(x.T), block2d, round_col, rht_col, seed,
                            copy_id=1, scale46=scale46)
    return row, col


def scale46_disagreements(x, rht=False, seed=0):
    """For the rows of x (rotated when rht), the number of 1x16 blocks whose 4/6 choice
    differs between the binary32 squared errors the method compares and the same errors in
    binary64, and the number of blocks whose binary64 errors tie exactly (a measurement of
    the evaluation-order convention, not part of the method), and the largest relative gap
    |e4 - e6| / max(e4, e6) of the binary64 errors among the differing blocks."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n, k = x.shape
    differ, ties, gap = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_double(0.0)
    _check(_load().or_scale46_disagreements(_ptr(x), n, k, int(rht), int(seed),
                                            ctypes.byref(differ), ctypes.byref(ties),
                                            ctypes.byref(gap)),
           "scale46_disagreements")
    return differ.value, ties.value, gap.value


def dequantize(q):
    n, k = q.shape
    out = np.zeros((n, k), dtype=np.float32)
    rc = _load().or_dequantize(_ptr(q.codes), _ptr(q.scales), q.sg, n, k, _ptr(out))
    _check(rc, "dequantize")
    return out


def gemm_f64(qa, qb):
    """C = A * B^T over exact dequantized operands, binary64; returns (C, sum|a*b|)."""
    M, K = qa.shape
    N, K2 = qb.shape
    assert K == K2
    C = np.zeros((M, N), dtype=np.float64)
    ad = np.zeros((M, N), dtype=np.float64)
    rc = _load().or_gemm_f64(_ptr(qa.codes), _ptr(qa.scales), qa.sg, _ptr(qb.codes),
                             _ptr(qb.scales), qb.sg, M, N, K, _ptr(C), _ptr(ad))
    _check(rc, "gemm_f64")
    return C, ad


def gemm_f64_entries(qa, qb, em, en):
    M, K = qa.shape
    N, _ = qb.shape
    em = np.ascontiguousarray(em, dtype=np.int64)
    en = np.ascontiguousarray(en, dtype=np.int64)
    out = np.zeros(em.shape[0], dtype=np.float64)
    ad = np.zeros(em.shape[0], dtype=np.float64)
    rc = _load().or_gemm_f64_entries(_ptr(qa.codes), _ptr(qa.scales), qa.sg, _ptr(qb.codes),
                                     _ptr(qb.scales), qb.sg, M, N, K, _ptr(em), _ptr(en),
                                     em.shape[0], _ptr(out), _ptr(ad))
    _check(rc, "gemm_f64_entries")
    return out, ad


# ---------------------------------------------------------------- LoRA-SVD low-rank branch
def lora_down(x, a, beta):
    """Down-projection t = BF16(beta x a^T) of Full-Stack FP4 sec. 3.2 eq. (1): x [M][K]
    (binary32), a [r][K] BF16 bits.  Returns (t [M][r] BF16 bits, binary64 value before
    the rounding, |beta| sum |x a|)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    a = np.ascontiguousarray(a, dtype=np.uint16)
    M, K = x.shape
    r, K2 = a.shape
    assert K == K2
    t = np.zeros((M, r), dtype=np.uint16)
    t64 = np.zeros((M, r), dtype=np.float64)
    tabs = np.zeros((M, r), dtype=np.float64)
    _check(_load().or_lora_down(_ptr(x), M, K, _ptr(a), r, float(beta), _ptr(t), _ptr(t64),
                                _ptr(tabs)), "lora_down")
    return t, t64, tabs


def requantize_cols(q_row, round_col=RNE, rht_col=False, seed=0, scale46=False):
    """Full-Stack FP4 eq. (2): the Wgrad operand Q_16x1(H^T Q_1x16(X)) is the columnwise
    quantization of the dequantized rowwise copy Q_1x16(X) (reading: the decoded values
    fl(fl(v s) s_g) are quantized exactly as an input tensor would be)."""
    xh = dequantize(q_row)
    _, col = quantize(xh, rowwise=False, colwise=True, round_col=round_col, rht_col=rht_col,
                      seed=seed, scale46=scale46)
    return col


def ns_step(x, a, b, c, seed, scale46=True):
    """One quantized Newton-Schulz iteration of NVFP4 Root (Full-Stack FP4 sec. 3.4):
    qX = Q_1x16(X H), qX' = Q_16x1(H^T X), A = qX qX^T, qA = Q_1x16(A H),
    qA' = Q_16x1(H^T A), B = b A + c qA qA', qB = Q_1x16(B H), X' = a X + qB qX'.
    Readings: every quantization nearest-even with 4/6 scaling and one random Hadamard
    (seed) for the whole iteration; the GEMM products are binary64 over the dequantized
    copies, A and B are held in binary32 (the GEMM output precision) before being
    quantized, and B and X' are formed in binary64 and rounded once to binary32.
    Returns (X', A, B) as binary32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    qx, qxc = quantize(x, rowwise=True, colwise=True, rht_row=True, rht_col=True, seed=seed,
                       scale46=scale46)
    A64, _ = gemm_f64(qx, qx)
    A = A64.astype(np.float32)
    qa, qac = quantize(A, rowwise=True, colwise=True, rht_row=True, rht_col=True, seed=seed,
                       scale46=scale46)
    P, _ = gemm_f64(qa, qac)
    B = (np.float64(np.float32(b)) * A.astype(np.float64) + np.float64(np.float32(c)) * P) \
        .astype(np.float32)
    qb, _ = quantize(B, rowwise=True, rht_row=True, seed=seed, scale46=scale46)
    Q, _ = gemm_f64(qb, qxc)
    xn = (np.float64(np.float32(a)) * x.astype(np.float64) + Q).astype(np.float32)
    return xn, A, B


def gemm_lora_f64(qa, qb, t, b):
    """A B^T over the dequantized operands plus t b^T (t [M][r], b [N][r] BF16 bits),
    binary64; returns (C, sum of |terms|)."""
    M, K = qa.shape
    N, _ = qb.shape
    t = np.ascontiguousarray(t, dtype=np.uint16)
    b = np.ascontiguousarray(b, dtype=np.uint16)
    r = t.shape[1]
    assert t.shape == (M, r) and b.shape == (N, r)
    C = np.zeros((M, N), dtype=np.float64)
    ad = np.zeros((M, N), dtype=np.float64)
    _check(_load().or_gemm_lora_f64(_ptr(qa.codes), _ptr(qa.scales), qa.sg, _ptr(qb.codes),
                                    _ptr(qb.scales), qb.sg, M, N, K, _ptr(t), _ptr(b), r, _ptr(C),
                                    _ptr(ad)), "gemm_lora_f64")
    return C, ad


def gemm_lora_f64_entries(qa, qb, t, b, em, en):
    M, K = qa.shape
    N, _ = qb.shape
    t = np.ascontiguousarray(t, dtype=np.uint16)
    b = np.ascontiguousarray(b, dtype=np.uint16)
    r = t.shape[1]
    em = np.ascontiguousarray(em, dtype=np.int64)
    en = np.ascontiguousarray(en, dtype=np.int64)
    out = np.zeros(em.shape[0], dtype=np.float64)
    ad = np.zeros(em.shape[0], dtype=np.float64)
    _check(_load().or_gemm_lora_f64_entries(_ptr(qa.codes), _ptr(qa.scales), qa.sg,
                                            _ptr(qb.codes), _ptr(qb.scales), qb.sg, M, N, K,
                                            _ptr(t), _ptr(b), r, _ptr(em), _ptr(en), em.shape[0],
                                            _ptr(out), _ptr(ad)), "gemm_lora_f64_entries")
    return out, ad


# ---------------------------------------------------------------- Q-AdamW second moment
def qadamw_v_encode(v, seed=0, use_signs=True):
    v = np.ascontiguousarray(v, dtype=np.float32)
    R, C = v.shape
    mu = np.zeros((R // 16, C // 16), dtype=np.uint16)
    codes = np.zeros((R, C // 2), dtype=np.uint8)
    scales = np.zeros((R, C // 16), dtype=np.uint8)
    sg = ctypes.c_float(0.0)
    rc = _load().or_qadamw_v_encode(_ptr(v), R, C, int(seed), int(use_signs), _ptr(mu),
                                    _ptr(codes), _ptr(scales), ctypes.byref(sg))
    _check(rc, "qadamw_v_encode")
    return mu, QTensor(codes, scales, sg.value)


def qadamw_v_decode(mu, q, seed=0, use_signs=True):
    R, C = q.shape
    mu = np.ascontiguousarray(mu, dtype=np.uint16)
    out = np.zeros((R, C), dtype=np.float32)
    rc = _load().or_qadamw_v_decode(_ptr(mu), _ptr(q.codes), _ptr(q.scales), q.sg, R, C,
                                    int(seed), int(use_signs), _ptr(out))
    _check(rc, "qadamw_v_decode")
    return out


# ---------------------------------------------------------------- helpers for tests
def unpack_codes(codes):
    """[n][k/2] bytes -> [n][k] 4-bit codes (element 2i in the low nibble)."""
    lo = codes & 0x0F
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], codes.shape[1] * 2)


def qadamw_step(w, g, m, mu, v, hp, m_rht_seed, m_sr_seed, v_seed, v_use_signs=True):
    """One quantized-state AdamW step (see or_qadamw_step).  w, g: float32 [R][C]; m: the
    moment state (QTensor of the rotated first moment); mu, v: the second-moment state.
    hp = dict(lr, beta1, beta2, eps, weight_decay, grad_coef, bias1, bias2).
    Returns (w_new, m_state, mu_new, v_state, m_new_f32, v_new_f32)."""
    w = np.array(w, dtype=np.float32, copy=True)
    g = np.ascontiguousarray(g, dtype=np.float32)
    R, C = w.shape
    h = np.array([hp[k] for k in ("lr", "beta1", "beta2", "eps", "weight_decay", "grad_coef",
                                  "bias1", "bias2")], dtype=np.float32)
    mc = np.zeros((R, C // 2), dtype=np.uint8)
    ms = np.zeros((R, C // 16), dtype=np.uint8)
    vc = np.zeros((R, C // 2), dtype=np.uint8)
    vs = np.zeros((R, C // 16), dtype=np.uint8)
    mu_out = np.zeros((R // 16, C // 16), dtype=np.uint16)
    msg, vsg = ctypes.c_float(0.0), ctypes.c_float(0.0)
    m_new = np.zeros((R, C), dtype=np.float32)
    v_new = np.zeros((R, C), dtype=np.float32)
    rc = _load().or_qadamw_step(_ptr(w), _ptr(g), R, C,
                                _ptr(np.ascontiguousarray(m.codes)), _ptr(np.ascontiguousarray(m.scales)), m.sg,
                                _ptr(np.ascontiguousarray(mu, dtype=np.uint16)),
                                _ptr(np.ascontiguousarray(v.codes)), _ptr(np.ascontiguousarray(v.scales)), v.sg,
                                _ptr(h), int(m_rht_seed), int(m_sr_seed), int(v_seed), int(v_use_signs),
                                _ptr(mc), _ptr(ms), ctypes.byref(msg), _ptr(mu_out), _ptr(vc), _ptr(vs),
                                ctypes.byref(vsg), _ptr(m_new), _ptr(v_new))
    _check(rc, "qadamw_step")
    return w, QTensor(mc, ms, msg.value), mu_out, QTensor(vc, vs, vsg.value), m_new, v_new
