"""GPU parity of qadamw_step against the oracle's quantized-state AdamW step: bit-exact
updated weights, first-moment state (codes, scales, tensor scale), tile means and
second-moment state, for f32 and bf16 gradients, over chained steps (states fed back),
and at the full 9216x3072 state size of the 3B FFN weight.  Inputs are seeded and
synthetic; the starting states are encoded by the oracle."""
import numpy as np
import pytest
import torch

from gpu_util import dev, to_gpu_qtensor

pytestmark = pytest.mark.gpu

HP = dict(lr=1.5e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_coef=1.0,
          bias1=1 / (1 - 0.9 ** 5), bias2=1 / (1 - 0.95 ** 5))
M_RHT, V_SEED = 0x4D5254, 0x56535444


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load_library()
    return nv


def start_state(oracle, R, C, seed):
    rng = np.random.default_rng(seed + 1000)
    m = (rng.standard_normal((R, C)) * 1e-3).astype(np.float32)
    v = np.exp(-18 + 3 * rng.standard_normal((R, C))).astype(np.float32)
    # any valid state will do: the oracle's quantizer rotates with M_RHT (and rounds with the
    # same seed), which is the layout the step decodes
    qm = oracle.quantize_rows(m, rounding=oracle.SR, rht=True, seed=M_RHT, scale46=True)
    mu, qv = oracle.qadamw_v_encode(v, seed=V_SEED, use_signs=True)
    w = (rng.standard_normal((R, C)) * 0.02).astype(np.float32)
    return w, qm, mu, qv


def grad(R, C, seed, bf16):
    rng = np.random.default_rng(seed)
    g = (rng.standard_normal((R, C)) * 1e-3 * np.exp(rng.standard_normal((1, C)))).astype(np.float32)
    if bf16:
        g = torch.from_numpy(g).to(torch.bfloat16).float().numpy()
    return g


def check_step(nv, oracle, w, g, qm, mu, qv, sr_seed, bf16):
    R, C = w.shape
    print(f"qadamw_step case {R}x{C} bf16={bf16} sr={sr_seed:#x}", flush=True)
    p = nv.qadamw_step_params(m_rht_seed=M_RHT, m_sr_seed=sr_seed, v_seed=V_SEED, v_use_signs=True,
                              **HP)
    wg = torch.from_numpy(w.copy()).to(dev())
    gg = torch.from_numpy(g).to(dev())
    if bf16:
        gg = gg.to(torch.bfloat16)
    mo, muo, vo = nv.qadamw_step(wg, gg, to_gpu_qtensor(nv, qm),
                                 torch.from_numpy(mu.view(np.int16)).to(dev()), to_gpu_qtensor(nv, qv), p)
    torch.cuda.synchronize()
    ow, oqm, omu, oqv, _, _ = oracle.qadamw_step(w, g, qm, mu, qv, HP, M_RHT, sr_seed, V_SEED, True)
    assert np.array_equal(wg.cpu().numpy().view(np.uint32), ow.view(np.uint32)), \
        f"{np.count_nonzero(wg.cpu().numpy() != ow)} weights differ"
    assert mo.gscale.item() == np.float32(oqm.sg) and vo.gscale.item() == np.float32(oqv.sg)
    assert np.array_equal(mo.scales.cpu().numpy(), oqm.scales)
    assert np.array_equal(mo.codes.cpu().numpy(), oqm.codes)
    assert np.array_equal(muo.cpu().numpy().view(np.uint16), omu)
    assert np.array_equal(vo.scales.cpu().numpy(), oqv.scales)
    assert np.array_equal(vo.codes.cpu().numpy(), oqv.codes)
    return ow, oqm, omu, oqv


@pytest.mark.parametrize("shape", [(16, 16), (48, 80), (272, 400)])
@pytest.mark.parametrize("bf16", [False, True])
def test_step_matches_oracle(nv, oracle, shape, bf16):
    w, qm, mu, qv = start_state(oracle, *shape, 10 + shape[1])
    check_step(nv, oracle, w, grad(*shape, 20 + shape[0], bf16), qm, mu, qv, 0x53520001, bf16)


def test_three_chained_steps(nv, oracle):
    R, C = 64, 256
    w, qm, mu, qv = start_state(oracle, R, C, 3)
    for k in range(3):
        w, qm, mu, qv = check_step(nv, oracle, w, grad(R, C, 100 + k, False), qm, mu, qv,
                                   0x53520100 + k, False)


def test_step_from_zero_state(nv, oracle):
    R, C = 32, 64
    z = np.zeros((R, C), dtype=np.float32)
    qm = oracle.quantize_rows(z, rounding=oracle.SR, seed=1, scale46=True)
    mu, qv = oracle.qadamw_v_encode(z, seed=V_SEED)
    w = np.random.default_rng(8).standard_normal((R, C)).astype(np.float32)
    check_step(nv, oracle, w, grad(R, C, 9, False), qm, mu, qv, 0x53520200, False)


def test_step_tiny_second_moments(nv, oracle):
    """Gradients of 1e-20 from the zero state give second moments far below 2^-96 (some
    subnormal): the weight update's square roots take the rescaled path for those waves."""
    R, C = 64, 256
    z = np.zeros((R, C), dtype=np.float32)
    qm = oracle.quantize_rows(z, rounding=oracle.SR, seed=1, scale46=True)
    mu, qv = oracle.qadamw_v_encode(z, seed=V_SEED)
    w = np.random.default_rng(12).standard_normal((R, C)).astype(np.float32)
    g = grad(R, C, 13, False)
    g[:16, :64] = 1e-20
    g[20, 5] = 3e-23
    check_step(nv, oracle, w, g, qm, mu, qv, 0x53520300, False)


@pytest.mark.parametrize("gscale", [1e-36, 1e-41])
def test_step_tiny_first_moments(nv, oracle, gscale):
    """Every gradient scaled to about 1e-36 (1e-41: subnormal) from the zero state: the new
    first moment's tensor scale is so small that the reciprocals of its small block scales
    leave binary32's range (the extended-range reciprocal), and its elements are tiny."""
    R, C = 64, 256
    z = np.zeros((R, C), dtype=np.float32)
    qm = oracle.quantize_rows(z, rounding=oracle.SR, seed=1, scale46=True)
    mu, qv = oracle.qadamw_v_encode(z, seed=V_SEED)
    w = np.random.default_rng(14).standard_normal((R, C)).astype(np.float32)
    g = (grad(R, C, 15, False).astype(np.float64) * gscale).astype(np.float32)
    g[3, 16:32] *= np.float32(1e-4)                  # blocks with much smaller scales
    check_step(nv, oracle, w, g, qm, mu, qv, 0x53520500, False)


def test_step_full_size(nv, oracle):
    from nvfp4_block_scaled_quantize_amd import synthetic
    R, C = 9216, 3072                      # the FFN weight's state, log-normal v as for Q-AdamW
    w, qm, mu, qv = start_state(oracle, R, C, 5)
    check_step(nv, oracle, w, grad(R, C, 6, True), qm, mu, qv, synthetic.RHT_SEED_QADAMW, True)


def test_step_refuses_aliased_states(nv):
    R, C = 16, 16
    d = dev()
    q = nv.QTensor.empty(R, C, d)
    v = nv.QTensor.empty(R, C, d)
    mu = torch.zeros((1, 1), dtype=torch.int16, device=d)
    w = torch.zeros((R, C), device=d)
    p = nv.qadamw_step_params(**HP)
    with pytest.raises(nv.Nvfp4Error):
        nv.qadamw_step(w, w.clone(), q, mu, v, p, m_out=q)


def test_step_many_partials(nv, oracle):
    """144000 x 16: 9000 first-pass workgroups (more partial maxima than one round of the
    reduction's loads covers), the largest gradient in the last tile."""
    R, C = 144000, 16
    w, qm, mu, qv = start_state(oracle, R, C, 31)
    g = grad(R, C, 32, False)
    g[-1, 7] = np.float32(np.abs(g).max() * 8.0)
    check_step(nv, oracle, w, g, qm, mu, qv, 0x53520400, False)
