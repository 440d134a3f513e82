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
