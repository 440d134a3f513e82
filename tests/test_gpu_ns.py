"""GPU parity of the Newton-Schulz building blocks and of one quantized NVFP4 Root
iteration (Full-Stack FP4 sec. 3.4) against the oracle.

nvfp4_gemm_axpby: C = alpha A B^T + beta D with oracle-quantized operands; tolerance
|C - (alpha C64 + beta D)| <= 1e-5 (|alpha| sum_k |a b| + |beta d|) per element, as the
plain GEMM's plus the one rounding of beta d.

nvfp4_ns_step: the quantize stages are bit-exact on oracle inputs (the quantize tests); the
whole iteration feeds GEMM outputs (FP32, accumulated in another order than the oracle's
binary64) into the next quantization, so an element at a rounding boundary can take the
neighbouring code.  The check: relative Frobenius distance between the GPU's and the
oracle's X' at most 2e-3 (well below the step's NVFP4 error of several percent), and both
equally close to the exact (unquantized) step.
"""
import numpy as np
import pytest
import torch

from gpu_util import dev, to_gpu_qtensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load_library()
    return nv


@pytest.mark.parametrize("M,N,K", [(32, 32, 32), (96, 160, 64), (288, 544, 256), (512, 256, 320)])
@pytest.mark.parametrize("inplace", [False, True])
def test_gemm_axpby(nv, oracle, M, N, K, inplace):
    print(f"gemm_axpby {M}x{N}x{K} inplace={inplace}", flush=True)
    rng = np.random.default_rng(M + N + K)
    qa, _ = oracle.quantize(rng.standard_normal((M, K)).astype(np.float32))
    qb, _ = oracle.quantize(rng.standard_normal((N, K)).astype(np.float32))
    d = rng.standard_normal((M, N)).astype(np.float32)
    alpha, beta = -0.75, 1.25
    dg = torch.from_numpy(d).to(dev())
    c = nv.nvfp4_gemm_axpby(to_gpu_qtensor(nv, qa), to_gpu_qtensor(nv, qb), alpha, dg, beta,
                            out=dg if inplace else None)
    torch.cuda.synchronize()
    P, ad = oracle.gemm_f64(qa, qb)
    ref = alpha * P + np.float64(np.float32(beta)) * d.astype(np.float64)
    err = np.abs(c.cpu().numpy().astype(np.float64) - ref)
    bound = 1e-5 * (abs(alpha) * ad + np.abs(beta * d.astype(np.float64))) + 1e-30
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g}"


def wide(m, n, seed, scale=0.9):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, n)) * np.exp(0.3 * rng.standard_normal((1, n)))
    return (x / np.linalg.norm(x, 2) * scale).astype(np.float32)


def exact_step(x, a, b, c):
    x = x.astype(np.float64)
    A = x @ x.T
    return a * x + b * (A @ x) + c * (A @ (A @ x))


# (256, 1024) and (512, 2048): A = qX qX^T is formed on the triangle tiles with K split into
# 2 and 4 parts, then reduced and mirrored; the other shapes take the plain GEMM
@pytest.mark.parametrize("m,n", [(32, 64), (64, 192), (96, 288), (288, 544), (256, 1024), (512, 2048)])
@pytest.mark.parametrize("abc", [(1.5, -0.5, 0.0), (2.0, -1.5, 0.5)])
def test_ns_step_matches_oracle(nv, oracle, m, n, abc):
    print(f"ns_step {m}x{n} coefficients {abc}", flush=True)
    x = wide(m, n, m + n)
    xg = torch.from_numpy(x.copy()).to(dev())
    nv.nvfp4_ns_step(xg, *abc, seed=0x5EED4)
    torch.cuda.synchronize()
    got = xg.cpu().numpy().astype(np.float64)
    want, _, _ = oracle.ns_step(x, *abc, seed=0x5EED4)
    want = want.astype(np.float64)
    d = np.linalg.norm(got - want) / np.linalg.norm(want)
    ex = exact_step(x, *abc)
    e_gpu = np.linalg.norm(got - ex) / np.linalg.norm(ex)
    e_or = np.linalg.norm(want - ex) / np.linalg.norm(ex)
    print(f"  gpu vs oracle {d:.3e}; vs exact: gpu {e_gpu:.3e} oracle {e_or:.3e}")
    assert d <= 2e-3
    assert abs(e_gpu - e_or) <= 0.1 * e_or + 1e-6


def test_ns_step_identity_and_refusals(nv):
    x = torch.from_numpy(wide(64, 128, 3)).to(dev())
    x0 = x.clone()
    nv.nvfp4_ns_step(x, 1.0, 0.0, 0.0, seed=1)
    torch.cuda.synchronize()
    assert torch.equal(x, x0)
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_ns_step(torch.zeros((48, 64), device=dev()), 1.5, -0.5, 0.0, seed=1)


def test_ns_full_size_orthogonalises(nv):
    """W_up's orientation 3072 x 9216 (the 3B FFN weight, wide): five textbook iterations
    from a normalised matrix bring X X^T to the identity within the quantization floor."""
    print("ns_step full-size 3072x9216 x5", flush=True)
    g = torch.Generator().manual_seed(11)
    x = torch.randn(3072, 9216, generator=g)
    x = (x / torch.linalg.matrix_norm(x, ord=2) * 0.9).to(dev())
    gram0 = (x @ x.T - torch.eye(3072, device=dev())).abs().max().item()
    ws = torch.empty(nv.load_library().nvfp4_ns_step_workspace_bytes(3072, 9216), dtype=torch.uint8,
                     device=dev())
    for k in range(5):
        nv.nvfp4_ns_step(x, 1.5, -0.5, 0.0, seed=200 + k, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(x).all()
    gram = (x @ x.T - torch.eye(3072, device=dev())).abs().max().item()
    print(f"  max |X X^T - I|: {gram0:.3f} -> {gram:.3f}")
    assert gram0 > 0.5 and gram < 0.25
