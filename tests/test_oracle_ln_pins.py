"""Pins for the oracle's TTT-Linear with the inner bias and, optionally,
LayerNorm and a residual inside f: f(x) = x + LN(W x + b) (diosapp "Test-Time
Training (TTT) guide" §3 for W x + b; the LN-and-residual ablation discussed in
PaperTrace "5 · TestingTime 训练与长上下文" §3.1).

  - bias only: the model equals the plain TTT-Linear oracle on inputs with an
    appended constant-1 feature (the bias as an extra column of W);
  - LN + residual: one step of the update equals minus eta times the central
    finite-difference gradient of the loss 1/2 ||k + LN(W k + b) - v||^2, with
    LN written out here;
  - the output normalisation: with unit LN weight and zero LN bias, every
    z_t - q_t has mean 0 and variance var/(var + eps);
  - zero LN weight: f(x) = x + beta has no gradient, so the state never moves.
CPU only."""
import numpy as np
import pytest

import oracle


def rand_case(rng, n, T, d, per_token=True):
    K = rng.standard_normal((n, T, d))
    Q = rng.standard_normal((n, T, d))
    V = rng.standard_normal((n, T, d))
    K /= np.linalg.norm(K, axis=-1, keepdims=True)
    eta = rng.uniform(0.05, 0.3, (n, T)) if per_token else None
    W0 = rng.standard_normal((n, d, d)) * 0.3
    b0 = rng.standard_normal((n, d)) * 0.3
    lnw = 1.0 + 0.2 * rng.standard_normal((n, d))
    lnb = 0.2 * rng.standard_normal((n, d))
    return K, Q, V, eta, W0, b0, lnw, lnb


@pytest.mark.parametrize("chunk,T", [(1, 9), (4, 13), (16, 16), (7, 30)])
def test_bias_is_an_extra_constant_feature(chunk, T):
    """f(x) = W x + b equals the plain scan over x' = [x; 1] with W' = [[W, b], [0, 0]]
    and v' = [v; 0]: the last row of W' gets no gradient and stays zero."""
    rng = np.random.default_rng(71)
    n, d = 2, 5
    K, Q, V, eta, W0, b0, _, _ = rand_case(rng, n, T, d)
    Z, WT, bT = oracle.linear_ln(K, Q, V, eta, 0.0, W0, b0, None, None, 1e-6, chunk)
    one = np.ones((n, T, 1))
    Ka = np.concatenate([K, one], -1)
    Qa = np.concatenate([Q, one], -1)
    Va = np.concatenate([V, np.zeros((n, T, 1))], -1)
    W0a = np.zeros((n, d + 1, d + 1))
    W0a[:, :d, :d] = W0
    W0a[:, :d, d] = b0
    Za, WTa = oracle.linear(Ka, Qa, Va, eta, 0.0, W0a, chunk)
    np.testing.assert_allclose(Z, Za[:, :, :d], rtol=0, atol=1e-12)
    np.testing.assert_allclose(Za[:, :, d], 0.0, atol=0)
    np.testing.assert_allclose(WT, WTa[:, :d, :d], rtol=0, atol=1e-12)
    np.testing.assert_allclose(bT, WTa[:, :d, d], rtol=0, atol=1e-12)


def _ln(u, w, b, eps):
    mu = u.mean()
    var = ((u - mu) ** 2).mean()
    return w * (u - mu) / np.sqrt(var + eps) + b


@pytest.mark.parametrize("d,eps", [(4, 1e-6), (8, 1e-5), (16, 1e-3)])
def test_ln_update_is_a_gradient_step(d, eps):
    """Chunk 1, one token: W_1 = W_0 - eta dl/dW and b_1 = b_0 - eta dl/db, with the
    gradient of l = 1/2 ||k + LN(W k + b) - v||^2 from central differences."""
    rng = np.random.default_rng(72 + d)
    K, Q, V, eta, W0, b0, lnw, lnb = rand_case(rng, 1, 1, d)
    _, W1, b1 = oracle.linear_ln(K, Q, V, eta, 0.0, W0, b0, lnw, lnb, eps, 1)
    k, v = K[0, 0], V[0, 0]

    def loss(W, b):
        r = k + _ln(W @ k + b, lnw[0], lnb[0], eps) - v
        return 0.5 * r @ r

    h = 1e-6
    gW = np.zeros((d, d))
    for i in range(d):
        for j in range(d):
            Wp, Wm = W0[0].copy(), W0[0].copy()
            Wp[i, j] += h
            Wm[i, j] -= h
            gW[i, j] = (loss(Wp, b0[0]) - loss(Wm, b0[0])) / (2 * h)
    gb = np.zeros(d)
    for i in range(d):
        bp, bm = b0[0].copy(), b0[0].copy()
        bp[i] += h
        bm[i] -= h
        gb[i] = (loss(W0[0], bp) - loss(W0[0], bm)) / (2 * h)
    et = eta[0, 0]
    np.testing.assert_allclose(W1[0], W0[0] - et * gW, rtol=0, atol=1e-8)
    np.testing.assert_allclose(b1[0], b0[0] - et * gb, rtol=0, atol=1e-8)


def test_ln_chunk_uses_the_chunk_start_state():
    """Chunk 3: the state after the chunk is W_0 minus the eta-weighted sum of the
    three tokens' finite-difference gradients, all taken at W_0, b_0."""
    rng = np.random.default_rng(75)
    d, eps = 5, 1e-5
    K, Q, V, eta, W0, b0, lnw, lnb = rand_case(rng, 1, 3, d)
    _, W1, b1 = oracle.linear_ln(K, Q, V, eta, 0.0, W0, b0, lnw, lnb, eps, 3)
    h = 1e-6
    Wn, bn = W0[0].copy(), b0[0].copy()
    for t in range(3):
        k, v = K[0, t], V[0, t]

        def loss(W, b):
            r = k + _ln(W @ k + b, lnw[0], lnb[0], eps) - v
            return 0.5 * r @ r
        for i in range(d):
            for j in range(d):
                Wp, Wm = W0[0].copy(), W0[0].copy()
                Wp[i, j] += h
                Wm[i, j] -= h
                Wn[i, j] -= eta[0, t] * (loss(Wp, b0[0]) - loss(Wm, b0[0])) / (2 * h)
            bp, bm = b0[0].copy(), b0[0].copy()
            bp[i] += h
            bm[i] -= h
            bn[i] -= eta[0, t] * (loss(W0[0], bp) - loss(W0[0], bm)) / (2 * h)
    np.testing.assert_allclose(W1[0], Wn, rtol=0, atol=1e-8)
    np.testing.assert_allclose(b1[0], bn, rtol=0, atol=1e-8)


def test_output_is_normalised():
    rng = np.random.default_rng(73)
    n, T, d, eps = 2, 20, 8, 1e-5
    K, Q, V, eta, W0, b0, _, _ = rand_case(rng, n, T, d)
    lnw, lnb = np.ones((n, d)), np.zeros((n, d))
    Z, _, _ = oracle.linear_ln(K, Q, V, eta, 0.0, W0, b0, lnw, lnb, eps, 4)
    y = Z - Q
    np.testing.assert_allclose(y.mean(-1), 0.0, atol=1e-12)
    var = y.var(-1)
    assert np.all(var < 1.0) and np.all(var > 0.9)


def test_zero_ln_weight_has_no_gradient():
    rng = np.random.default_rng(74)
    n, T, d = 2, 17, 6
    K, Q, V, eta, W0, b0, _, lnb = rand_case(rng, n, T, d)
    Z, WT, bT = oracle.linear_ln(K, Q, V, eta, 0.0, W0, b0, np.zeros((n, d)), lnb, 1e-6, 5)
    np.testing.assert_array_equal(WT, W0)
    np.testing.assert_array_equal(bT, b0)
    np.testing.assert_allclose(Z, Q + lnb[:, None, :], rtol=0, atol=1e-15)
