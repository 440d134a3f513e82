"""GPU parity of the Newton-Schulz building blocks and of one quantized NVFP4 Root
iteration (Full-Stack FP4 sec. 3.4) against the oracle.

nvfp4_gemm_axpby: C = alpha A B^T + beta D with oracle-quantized operands; tolerance
|C - (alpha C64 + beta D)| <= 1e-5 (|alpha| sum_k |a b| + |beta d|) per element, as the
plain GEMM's plus the one rounding of beta d.

nvfp4_ns_step, stage by stage: the step leaves its intermediates in the workspace (at the
offsets include/nvfp4.h documents), and each stage is checked against the oracle on the
GPU's own input to that stage -- qX, qX' bit-exact from X; A against the binary64 product
of qX at the GEMM tolerance (the triangle split-K path for m a multiple of 256); qA, qA'
bit-exact from the GPU's A; B against b A + c qA qA' (binary64) at the alpha/beta GEMM
tolerance; qB bit-exact from the GPU's B; X' against a X + qB qX' likewise.  The full-size
3072 x 9216 step is checked the same way on sampled entries plus full rows and columns.

The whole iteration, run separately on the oracle, feeds its own binary64 GEMM outputs into
the next quantization, so an element at a rounding boundary can take the neighbouring code;
end to end the two are compared through the relative Frobenius distance of X' (at most
2e-3, well below the step's NVFP4 error of several percent), both equally close to the
exact (unquantized) step.
"""
import numpy as np
import pytest
import torch

from gpu_util import GEMM_TOL, assert_copy_equal, dev, to_gpu_qtensor

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


# ------------------------------------------------------------------ stage by stage
def al256(n):
    return (n + 255) & ~255


def ns_intermediates(nv, ws, m, n):
    """The intermediates nvfp4_ns_step leaves in its workspace, in the documented order:
    qX, qX', A, qA, qA', B, qB, each piece 256-byte aligned after the previous one."""
    off = 0

    def take(nbytes):
        nonlocal off
        t = ws[off:off + nbytes]
        off += al256(nbytes)
        return t

    def copy(r, c):
        codes = take(r * c // 2).view(r, c // 2)
        scales = take(r * c // 16).view(r, c // 16)
        return nv.QTensor(codes, scales, take(4).view(torch.float32))

    qx, qxc = copy(m, n), copy(n, m)
    A = take(m * m * 4).view(torch.float32).view(m, m)
    qa, qac = copy(m, m), copy(m, m)
    B = take(m * m * 4).view(torch.float32).view(m, m)
    qb = copy(m, m)
    return qx, qxc, A, qa, qac, B, qb


def check_product(what, got, ref, absdot, extra):
    """|got - ref| <= GEMM_TOL (sum |a b| + |extra|) per entry (ref and the bound in
    binary64), and the relative Frobenius error at most GEMM_TOL."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bound = GEMM_TOL * (absdot + np.abs(extra)) + 1e-30
    fro = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)
    print(f"  {what}: max err/bound {np.max(err / bound):.3f}, frobenius {fro:.2e}")
    assert np.all(err <= bound), f"{what}: {(err > bound).sum()} entries outside the bound"
    assert fro <= GEMM_TOL


def run_stagewise(nv, oracle, x, abc, seed, sampled):
    a, b, c = abc
    m, n = x.shape
    ws = torch.empty(nv.load_library().nvfp4_ns_step_workspace_bytes(m, n), dtype=torch.uint8,
                     device=dev())
    xg = torch.from_numpy(x.copy()).to(dev())
    nv.nvfp4_ns_step(xg, a, b, c, seed=seed, workspace=ws)
    torch.cuda.synchronize()
    qx, qxc, A, qa, qac, B, qb = ns_intermediates(nv, ws, m, n)
    rng = np.random.default_rng(seed)

    def entries(rows, cols):
        if not sampled:
            return None
        em = list(rng.integers(0, rows, 4096)) + [0] * cols + [rows - 1] * cols + list(range(rows)) * 2
        en = list(rng.integers(0, cols, 4096)) + list(range(cols)) * 2 + [0] * rows + [cols - 1] * rows
        return np.array(em), np.array(en)

    def product(qa_, qb_, idx):
        if idx is None:
            return oracle.gemm_f64(qa_, qb_)
        return oracle.gemm_f64_entries(qa_, qb_, *idx)

    def pick(t, idx):
        t = t.cpu().numpy() if isinstance(t, torch.Tensor) else t
        return t if idx is None else t[idx]

    # qX, qX' from X
    oqx, oqxc = oracle.quantize(x, rowwise=True, colwise=True, rht_row=True, rht_col=True,
                                seed=seed, scale46=True)
    assert_copy_equal(qx, oqx, "qX")
    assert_copy_equal(qxc, oqxc, "qX'")
    # A = qX qX^T
    idx = entries(m, m)
    P, ad = product(oqx, oqx, idx)
    check_product("A", pick(A, idx), P, ad, 0.0)
    # qA, qA' from the GPU's A
    A_np = A.cpu().numpy()
    oqa, oqac = oracle.quantize(A_np, rowwise=True, colwise=True, rht_row=True, rht_col=True,
                                seed=seed, scale46=True)
    assert_copy_equal(qa, oqa, "qA")
    assert_copy_equal(qac, oqac, "qA'")
    # B = b A + c qA qA'
    P, ad = product(oqa, oqac, idx)
    bA = np.float64(np.float32(b)) * pick(A_np, idx).astype(np.float64)
    check_product("B", pick(B, idx), np.float64(np.float32(c)) * P + bA, abs(c) * ad, bA)
    # qB from the GPU's B
    oqb, _ = oracle.quantize(B.cpu().numpy(), rowwise=True, rht_row=True, seed=seed, scale46=True)
    assert_copy_equal(qb, oqb, "qB")
    # X' = a X + qB qX'
    idx = entries(m, n)
    P, ad = product(oqb, oqxc, idx)
    aX = np.float64(np.float32(a)) * pick(x, idx).astype(np.float64)
    check_product("X'", pick(xg, idx), P + aX, ad, aX)


# (64, 192): A by the plain GEMM; (256, 1024) and (512, 2048): A on the triangle tiles with K
# split into 2 and 4 parts, reduced and mirrored
@pytest.mark.parametrize("m,n", [(64, 192), (256, 1024), (512, 2048)])
@pytest.mark.parametrize("abc", [(1.5, -0.5, 0.0), (2.0, -1.5, 0.5)])
def test_ns_step_stagewise(nv, oracle, m, n, abc):
    print(f"ns_step stage by stage {m}x{n} coefficients {abc}", flush=True)
    run_stagewise(nv, oracle, wide(m, n, 7 * m + n), abc, 0x5EED4 + m, sampled=False)


def test_ns_step_stagewise_full_size(nv, oracle):
    """W_up's wide orientation 3072 x 9216: A by the triangle split-K path; every stage on
    4096 sampled entries plus two full rows and two full columns."""
    print("ns_step stage by stage full-size 3072x9216", flush=True)
    run_stagewise(nv, oracle, wide(3072, 9216, 12), (2.0, -1.5, 0.5), 0x5EED7, sampled=True)
