"""Pins of the oracle's quantized Newton-Schulz iteration (Full-Stack FP4 sec. 3.4; the
iteration X = a X + b X (X^T X) + c X (X^T X)^2 of sec. 2, wide orientation A = X X^T).

Independent of the oracle's arithmetic:
  * closed forms: a = 1, b = c = 0 returns X bit for bit (B = 0 quantizes to zero codes);
    c = 0 gives B = fl(b A) exactly;
  * one step approximates the exact step a X + b (X X^T) X + c (X X^T)^2 X (numpy float64)
    to within NVFP4 noise;
  * the textbook coefficients (1.5, -0.5, 0) drive X towards the orthogonal polar factor
    of scipy.linalg.polar: within four steps X X^T falls from 0.63 off the identity to the
    quantization noise floor (about 0.1), close to the polar factor.  Further steps keep
    X X^T near I while the noise moves X along the orthogonal group, so the distance to
    the polar factor is checked at step four.
"""
import numpy as np
import scipy.linalg


def wide(m, n, seed, scale=0.9):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, n)) * np.exp(0.3 * rng.standard_normal((1, n)))
    return (x / np.linalg.norm(x, 2) * scale).astype(np.float32)


def exact_step(x, a, b, c):
    x = x.astype(np.float64)
    A = x @ x.T
    return a * x + b * (A @ x) + c * (A @ (A @ x))


def rel(u, v):
    return np.linalg.norm(u - v) / np.linalg.norm(v)


def test_identity_coefficients(oracle):
    x = wide(32, 64, 1)
    xn, A, B = oracle.ns_step(x, 1.0, 0.0, 0.0, seed=3)
    assert np.array_equal(xn, x)
    assert np.all(B == 0)


def test_c_zero_gives_b_times_a(oracle):
    x = wide(32, 96, 2)
    _, A, B = oracle.ns_step(x, 1.5, -0.5, 0.0, seed=4)
    assert np.array_equal(B, (np.float32(-0.5) * A).astype(np.float32))


def test_one_step_approximates_the_exact_iteration(oracle):
    x = wide(64, 192, 5)
    for abc in ((1.5, -0.5, 0.0), (2.0, -1.5, 0.5)):
        xn, A, _ = oracle.ns_step(x, *abc, seed=6)
        e = rel(xn.astype(np.float64), exact_step(x, *abc))
        assert 0 < e < 0.1, (abc, e)
        assert rel(A.astype(np.float64), x.astype(np.float64) @ x.T.astype(np.float64)) < 0.1


def test_textbook_coefficients_orthogonalise(oracle):
    x = wide(32, 128, 7, scale=0.8)
    u = scipy.linalg.polar(x.T.astype(np.float64))[0].T      # orthonormal rows
    g0 = np.abs(x.astype(np.float64) @ x.T.astype(np.float64) - np.eye(32)).max()
    for k in range(4):
        x, _, _ = oracle.ns_step(x, 1.5, -0.5, 0.0, seed=100 + k)
    gram = x.astype(np.float64) @ x.T.astype(np.float64)
    assert g0 > 0.5 and np.abs(gram - np.eye(32)).max() < 0.2
    assert rel(x.astype(np.float64), u) < 0.15
