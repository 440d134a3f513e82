"""Pins of the oracle's quantized-state AdamW step.

Full-Stack FP4 sec. 2 gives the moment recurrences (m_t = beta1 m_{t-1} + g_t,
v_t = beta2 v_{t-1} + (1 - beta2) g_t^2) and sec. 3.3 the state storage (m through a
Hadamard rotation, stochastic rounding and 4/6 scaling; v through the sqrt / tile mean /
Hadamard / NVFP4 pipeline); the update is decoupled AdamW with caller-supplied bias
multipliers (reading).  The checks:
  * the fp32 moments and weights equal the real-number update of the decoded states to a
    few ulps (binary64 evaluation written here from the formula, not the oracle's code);
  * closed forms: lr = 0 leaves w bit-identical; beta1 = 0 with coefficient 1 gives m = g;
    beta2 = 1 with g = 0 keeps v;
  * the m state is the SR + 4/6 quantization of the rotated moment (same seeds through the
    separately pinned quantizer), and it is unbiased over stochastic-rounding seeds;
  * the v state is the second-moment pipeline's encoding of the new v.
"""
import numpy as np
import pytest

HP = dict(lr=2e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_coef=1.0,
          bias1=1 / (1 - 0.9 ** 3), bias2=1 / (1 - 0.95 ** 3))
M_RHT, M_SR, V_SEED = 0x4D52, 0x5352, 0x5653


def rotate(x, seed, oracle, inverse=False):
    sgn = oracle.rht_signs(seed)
    y = np.array(x, dtype=np.float32)
    f = oracle.rht16_inverse if inverse else oracle.rht16_forward
    for r in range(y.shape[0]):
        for c in range(0, y.shape[1], 16):
            y[r, c:c + 16] = f(y[r, c:c + 16], sgn)
    return y


def make_state(oracle, R, C, seed):
    rng = np.random.default_rng(seed)
    m = (rng.standard_normal((R, C)) * 1e-3).astype(np.float32)
    v = np.exp(-14 + 2 * rng.standard_normal((R, C))).astype(np.float32)
    qm = oracle.quantize_rows(rotate(m, M_RHT, oracle), rounding=oracle.SR, seed=11, scale46=True)
    mu, qv = oracle.qadamw_v_encode(v, seed=V_SEED, use_signs=True)
    w = rng.standard_normal((R, C)).astype(np.float32)
    g = (rng.standard_normal((R, C)) * 1e-3 * np.exp(rng.standard_normal((R, 1)))).astype(np.float32)
    return w, g, qm, mu, qv


def decoded(oracle, qm, mu, qv):
    m = rotate(oracle.dequantize(qm), M_RHT, oracle, inverse=True)
    v = oracle.qadamw_v_decode(mu, qv, seed=V_SEED, use_signs=True)
    return m, v


def step(oracle, w, g, qm, mu, qv, hp=HP, sr=M_SR):
    return oracle.qadamw_step(w, g, qm, mu, qv, hp, M_RHT, sr, V_SEED, True)


def test_update_is_the_formula(oracle):
    w, g, qm, mu, qv = make_state(oracle, 48, 96, 1)
    mp, vp = decoded(oracle, qm, mu, qv)
    w1, _, _, _, m1, v1 = step(oracle, w, g, qm, mu, qv)
    d = {k: np.float64(np.float32(v)) for k, v in HP.items()}
    g64, mp64, vp64, w64 = (a.astype(np.float64) for a in (g, mp, vp, w))
    t1, t2 = d["beta1"] * mp64, d["grad_coef"] * g64
    m_ex = t1 + t2
    omb2 = np.float64(np.float32(1 - np.float32(HP["beta2"])))
    u1, u2 = d["beta2"] * vp64, omb2 * g64 * g64
    v_ex = u1 + u2
    # each result is three binary32 roundings of these terms: error <= 3 * 2^-24 * (|t1| + |t2|)
    eps32 = 2.0 ** -24
    assert np.all(np.abs(m1 - m_ex) <= 3 * eps32 * (np.abs(t1) + np.abs(t2)) + 1e-45)
    assert np.all(np.abs(v1 - v_ex) <= 4 * eps32 * (u1 + u2) + 1e-45)
    # the weight update from the oracle's own moments (isolates the update formula)
    m64, v64 = m1.astype(np.float64), v1.astype(np.float64)
    q = d["bias1"] * m64 / (np.sqrt(d["bias2"] * v64) + d["eps"])
    upd = q + d["weight_decay"] * w64
    w_ex = w64 - d["lr"] * upd
    # roundings: the quotient chain (sqrt, add, multiply, divide), the add, the lr product
    # and the final subtraction
    bound = eps32 * (2 * np.abs(w64) + 8 * d["lr"] * (np.abs(q) + np.abs(d["weight_decay"] * w64)))
    assert np.all(np.abs(w1 - w_ex) <= bound)
    assert np.max(np.abs(w1 - w)) > 0


def test_closed_forms(oracle):
    w, g, qm, mu, qv = make_state(oracle, 32, 64, 2)
    mp, vp = decoded(oracle, qm, mu, qv)
    w1, *_ = step(oracle, w, g, qm, mu, qv, dict(HP, lr=0.0))
    assert np.array_equal(w1, w)
    _, _, _, _, m1, _ = step(oracle, w, g, qm, mu, qv, dict(HP, beta1=0.0, grad_coef=1.0))
    assert np.array_equal(m1, g)
    _, _, _, _, _, v1 = step(oracle, w, np.zeros_like(g), qm, mu, qv, dict(HP, beta2=1.0))
    assert np.array_equal(v1, vp)
    # only weight decay acts when m = v = 0 would divide 0 by eps: start from zero states
    zq = oracle.quantize_rows(np.zeros_like(w), rounding=oracle.SR, seed=1, scale46=True)
    zmu, zv = oracle.qadamw_v_encode(np.zeros_like(w), seed=V_SEED)
    w2, *_ = step(oracle, w, np.zeros_like(g), zq, zmu, zv)
    expect = w - np.float32(HP["lr"]) * (np.float32(HP["weight_decay"]) * w)
    assert np.array_equal(w2, expect.astype(np.float32))


def test_m_state_is_sr46_of_rotated_moment(oracle):
    w, g, qm, mu, qv = make_state(oracle, 32, 128, 3)
    _, qm1, _, _, m1, _ = step(oracle, w, g, qm, mu, qv)
    ref = oracle.quantize_rows(rotate(m1, M_RHT, oracle), rounding=oracle.SR, seed=M_SR,
                               scale46=True)
    assert np.array_equal(qm1.codes, ref.codes) and np.array_equal(qm1.scales, ref.scales)
    assert qm1.sg == ref.sg
    # unbiased over stochastic-rounding seeds (in the rotated domain)
    target = rotate(m1, M_RHT, oracle).astype(np.float64)
    acc = np.zeros_like(target)
    n = 48
    for k in range(n):
        _, q, *_ = step(oracle, w, g, qm, mu, qv, sr=1000 + k)
        acc += oracle.dequantize(q)
    err = acc / n - target
    scale = np.abs(target).max()
    assert np.abs(err.mean()) < 2e-3 * scale
    assert np.abs(err).max() < 0.35 * scale


def test_v_state_is_the_pipeline(oracle):
    w, g, qm, mu, qv = make_state(oracle, 32, 96, 4)
    _, _, mu1, qv1, _, v1 = step(oracle, w, g, qm, mu, qv)
    mu_ref, qv_ref = oracle.qadamw_v_encode(v1, seed=V_SEED, use_signs=True)
    assert np.array_equal(mu1, mu_ref)
    assert np.array_equal(qv1.codes, qv_ref.codes) and np.array_equal(qv1.scales, qv_ref.scales)
    assert qv1.sg == qv_ref.sg
