"""GPU parity of nvfp4_gemm against the oracle's binary64 GEMM.

Operands are quantized by the oracle and uploaded, so every input and every expected
value comes from the oracle.  Tolerance (stated in gpu_util.GEMM_TOL): relative Frobenius
error <= 1e-5 and max_ij |C - C64| / sum_k |a_ik b_jk| <= 1e-5; the only rounding in the
kernel is FP32 accumulation because every decoded product v*s is exact in binary16.
Full-size shapes (the 3B QKV, FFN-up, FFN-down and weight-gradient GEMMs) are checked on
4096 sampled entries plus two full rows and two full columns.
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


def quantized_pair(oracle, M, N, K, seed, wstd=0.02):
    from nvfp4_block_scaled_quantize_amd import synthetic
    a = synthetic.outlier_channels((M, K), seed).to(torch.bfloat16).float().numpy()
    b = synthetic.normal((N, K), seed + 1, wstd).to(torch.bfloat16).float().numpy()
    qa, _ = oracle.quantize(a)
    qb, _ = oracle.quantize(b, block2d=(N % 16 == 0 and K % 16 == 0))
    return qa, qb


@pytest.mark.parametrize("M,N,K", [(16, 16, 32), (128, 128, 256), (48, 80, 64), (272, 400, 160),
                                   (528, 272, 416), (256, 256, 128 * 3 + 32), (64, 96, 1024),
                                   (16, 512, 32),
                                   # K % 32 == 16: rows end in a half chunk, read 8 bytes at a time
                                   (16, 16, 16), (48, 80, 48), (272, 400, 144), (304, 272, 16 * 27)])
def test_gemm_small_shapes_full_matrix(nv, oracle, M, N, K):
    print(f"gemm case {M}x{N}x{K}", flush=True)
    qa, qb = quantized_pair(oracle, M, N, K, 100 + M + N + K)
    c = nv.nvfp4_gemm(to_gpu_qtensor(nv, qa), to_gpu_qtensor(nv, qb))
    torch.cuda.synchronize()
    ref, absdot = oracle.gemm_f64(qa, qb)
    fro, nw = gemm_errors(c.cpu().numpy(), ref, absdot)
    print(f"  frobenius {fro:.3e} normwise {nw:.3e}")
    assert fro <= GEMM_TOL and nw <= GEMM_TOL


def test_gemm_tiny_workload(nv, oracle):
    # X, W fp32 128x256 N(0,1) with 1% entries x50, RNE 1x16, Y = X W^T 128x128
    from nvfp4_block_scaled_quantize_amd import synthetic
    t = synthetic.tiny()
    qa, _ = oracle.quantize(t["X"].numpy())
    qb, _ = oracle.quantize(t["W"].numpy())
    c = nv.nvfp4_gemm(to_gpu_qtensor(nv, qa), to_gpu_qtensor(nv, qb))
    torch.cuda.synchronize()
    ref, absdot = oracle.gemm_f64(qa, qb)
    fro, nw = gemm_errors(c.cpu().numpy(), ref, absdot)
    assert fro <= GEMM_TOL and nw <= GEMM_TOL


def test_gemm_ldc_and_zero_k(nv, oracle):
    qa, qb = quantized_pair(oracle, 64, 48, 64, 7)
    out = torch.full((64, 80), 123.0, device=dev())
    nv.nvfp4_gemm(to_gpu_qtensor(nv, qa), to_gpu_qtensor(nv, qb), out=out[:, :48])
    torch.cuda.synchronize()
    ref, absdot = oracle.gemm_f64(qa, qb)
    fro, nw = gemm_errors(out[:, :48].cpu().numpy(), ref, absdot)
    assert fro <= GEMM_TOL and nw <= GEMM_TOL
    assert torch.all(out[:, 48:] == 123.0)
    # K = 0: C = 0
    z = nv.QTensor(torch.zeros((16, 0), dtype=torch.uint8, device=dev()),
                   torch.zeros((16, 0), dtype=torch.uint8, device=dev()),
                   torch.ones((1,), device=dev()))
    c = nv.nvfp4_gemm(z, z)
    torch.cuda.synchronize()
    assert torch.all(c == 0)


def sampled_check(nv, oracle, qa, qb, M, N, seed):
    c = nv.nvfp4_gemm(to_gpu_qtensor(nv, qa), to_gpu_qtensor(nv, qb))
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    em = list(rng.integers(0, M, 4096)) + [0] * N + [M - 1] * N + list(range(M)) * 2
    en = list(rng.integers(0, N, 4096)) + list(range(N)) * 2 + [0] * M + [N - 1] * M
    em, en = np.array(em), np.array(en)
    ref, absdot = oracle.gemm_f64_entries(qa, qb, em, en)
    got = c.cpu().numpy()[em, en]
    fro, nw = gemm_errors(got, ref, absdot)
    print(f"  sampled frobenius {fro:.3e} normwise {nw:.3e}")
    assert fro <= GEMM_TOL and nw <= GEMM_TOL


@pytest.mark.parametrize("name,M,N,K", [("qkv", 8192, 6144, 3072), ("ffn_up", 8192, 9216, 3072),
                                        ("ffn_down", 8192, 3072, 9216),
                                        ("wgrad", 9216, 3072, 8192)])
def test_gemm_full_size_sampled(nv, oracle, name, M, N, K):
    print(f"gemm full-size {name} {M}x{N}x{K}", flush=True)
    qa, qb = quantized_pair(oracle, M, N, K, 1000 + M + N)
    sampled_check(nv, oracle, qa, qb, M, N, 5)


def test_gemm_operand_over_2gib(nv, oracle):
    """A holds 2 GiB + 64 KiB of codes, past the direct path's 32-bit buffer offsets, so the
    generic path runs.  Rows on both sides of the 2^31-byte offset, the first and last rows
    and 32 random rows are checked against the oracle's binary64 product."""
    from nvfp4_block_scaled_quantize_amd import synthetic
    M, N, K = (1 << 19) + 16, 16, 8192            # A codes: M K / 2 = 2^31 + 65536 bytes
    print(f"gemm with a {M * K // 2} byte operand, {M}x{N}x{K}", flush=True)
    ca, sa = synthetic.random_nvfp4_parts(M, K, 21, device=dev())
    cb, sb = synthetic.random_nvfp4_parts(N, K, 22, device=dev())
    c = nv.nvfp4_gemm(nv.QTensor(ca, sa, torch.ones((1,), device=dev())),
                      nv.QTensor(cb, sb, torch.ones((1,), device=dev())))
    torch.cuda.synchronize()
    edge = (1 << 31) // (K // 2)                  # first row that starts past 2^31 bytes
    rng = np.random.default_rng(23)
    rows = sorted(set([0, edge - 1, edge, edge + 1, M - 1] + [int(r) for r in rng.integers(0, M, 32)]))
    idx = torch.tensor(rows, device=dev())
    qa = oracle.QTensor(ca[idx].cpu().numpy(), sa[idx].cpu().numpy(), 1.0)
    qb = oracle.QTensor(cb.cpu().numpy(), sb.cpu().numpy(), 1.0)
    ref, absdot = oracle.gemm_f64(qa, qb)
    fro, nw = gemm_errors(c[idx].cpu().numpy(), ref, absdot)
    print(f"  rows {len(rows)} frobenius {fro:.3e} normwise {nw:.3e}")
    assert fro <= GEMM_TOL and nw <= GEMM_TOL

