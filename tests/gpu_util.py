"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch


def dev():
    return torch.device("cuda:0")


def to_gpu_qtensor(nv, oq):
    """Upload an oracle-quantized copy so GPU kernels consume oracle data."""
    d = dev()
    return nv.QTensor(torch.from_numpy(np.ascontiguousarray(oq.codes)).to(d),
                      torch.from_numpy(np.ascontiguousarray(oq.scales)).to(d),
                      torch.tensor([oq.sg], dtype=torch.float32, device=d))


def assert_copy_equal(gq, oq, what=""):
    codes = gq.codes.cpu().numpy()
    scales = gq.scales.cpu().numpy()
    sg = gq.gscale.cpu().numpy()[0]
    assert sg == np.float32(oq.sg), f"{what}: tensor scale {sg!r} vs oracle {oq.sg!r}"
    if not np.array_equal(scales, oq.scales):
        bad = np.argwhere(scales != oq.scales)
        r, c = bad[0]
        raise AssertionError(f"{what}: {len(bad)} scale mismatches, first at {tuple(bad[0])}: "
                             f"gpu {scales[r, c]:#x} oracle {oq.scales[r, c]:#x}")
    if not np.array_equal(codes, oq.codes):
        bad = np.argwhere(codes != oq.codes)
        r, c = bad[0]
        raise AssertionError(f"{what}: {len(bad)} code-byte mismatches, first at {tuple(bad[0])}: "
                             f"gpu {codes[r, c]:#04x} oracle {oq.codes[r, c]:#04x}")


def gemm_errors(c_gpu, ref, absdot):
    """Tolerance measures for C = A B^T against the binary64 reference:
    (i) relative Frobenius error, (ii) max over entries of |err| / sum_k |a_k b_k|."""
    c = np.asarray(c_gpu, dtype=np.float64)
    err = np.abs(c - ref)
    fro = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)
    nw = (err / np.maximum(absdot, 1e-300)).max() if err.size else 0.0
    return fro, nw


# Stated GEMM tolerance: the products v*s are exact in binary16 and the MFMA products
# exact in FP32, so the only error is FP32 accumulation over K (sqrt(K/16) * 2^-24 ~ 1e-6
# typical, gamma_{K/16} ~ 3e-5 worst case at K = 9216).
GEMM_TOL = 1e-5
