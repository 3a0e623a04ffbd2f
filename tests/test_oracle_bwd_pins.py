"""Pins for the oracle's vector-Jacobian product of the TTT-Linear scan.

The pages give the forward scan only (PaperTrace "5 · TestingTime 训练与长上下文"
§1.1, §2.1, §2.3); its gradient is fixed by the mathematics.  The oracle's VJP is
pinned to:
  - central finite differences of the oracle's forward scan (itself pinned by
    test_oracle_pins.py), for every element of K, Q, V, eta and W0;
  - the closed form of a single delta-rule step, derived by hand;
  - linearity in the cotangent, and the scalar-eta gradient being the sum of
    the per-token ones.
CPU only."""
import numpy as np
import pytest

import oracle


def rand_case(rng, n, T, d, per_token=True):
    K = rng.standard_normal((n, T, d))
    Q = rng.standard_normal((n, T, d))
    V = rng.standard_normal((n, T, d))
    K /= np.linalg.norm(K, axis=-1, keepdims=True)
    eta = rng.uniform(0.05, 0.4, (n, T)) if per_token else None
    W0 = rng.standard_normal((n, d, d)) * 0.4
    dZ = rng.standard_normal((n, T, d))
    dWT = rng.standard_normal((n, d, d))
    return K, Q, V, eta, W0, dZ, dWT


def loss(args, eta_scalar, chunk, dZ, dWT):
    K, Q, V, eta, W0 = args
    Z, W = oracle.linear(K, Q, V, eta, eta_scalar, W0, chunk, nthreads=1)
    L = float((Z * dZ).sum())
    if dWT is not None:
        L += float((W * dWT).sum())
    return L


def finite_difference(args, which, eta_scalar, chunk, dZ, dWT, h=1e-6):
    A = args[which]
    fd = np.zeros_like(A)
    for idx in np.ndindex(A.shape):
        up = [None if a is None else a.copy() for a in args]
        dn = [None if a is None else a.copy() for a in args]
        up[which][idx] += h
        dn[which][idx] -= h
        fd[idx] = (loss(up, eta_scalar, chunk, dZ, dWT) - loss(dn, eta_scalar, chunk, dZ, dWT)) / (2 * h)
    return fd


@pytest.mark.parametrize("d,T,chunk,with_dWT", [
    (4, 7, 3, True),     # ragged last chunk
    (3, 5, 1, True),     # delta rule, one token per chunk
    (4, 6, 8, False),    # one chunk longer than the sequence, no state cotangent
    (2, 9, 4, True),
    (5, 4, 2, False),
])
def test_vjp_matches_finite_differences(d, T, chunk, with_dWT):
    rng = np.random.default_rng(300 + d * 10 + chunk)
    K, Q, V, eta, W0, dZ, dWT = rand_case(rng, 2, T, d)
    dWT = dWT if with_dWT else None
    grads = oracle.linear_bwd(K, Q, V, eta, 0.0, W0, chunk, dZ, dWT)
    args = [K, Q, V, eta, W0]
    for which, name in enumerate(["K", "Q", "V", "eta", "W0"]):
        g = grads[which]
        fd = finite_difference(args, which, 0.0, chunk, dZ, dWT)
        scale = max(1.0, np.abs(fd).max())
        assert np.abs(g - fd).max() < 1e-7 * scale, (name, np.abs(g - fd).max())


def test_scalar_eta_gradient_is_the_sum_over_tokens():
    rng = np.random.default_rng(311)
    K, Q, V, _, W0, dZ, dWT = rand_case(rng, 2, 7, 4, per_token=False)
    c, chunk = 0.15, 3
    g_scalar = oracle.linear_bwd(K, Q, V, None, c, W0, chunk, dZ, dWT)
    g_tokens = oracle.linear_bwd(K, Q, V, np.full((2, 7), c), 0.0, W0, chunk, dZ, dWT)
    for a, b in zip(g_scalar, g_tokens):
        np.testing.assert_array_equal(a, b)
    h = 1e-6
    args = [K, Q, V, None, W0]
    for s in range(2):
        fd = (loss(args, c + h, chunk, dZ, dWT) - loss(args, c - h, chunk, dZ, dWT)) / (2 * h)
        # the two slices' losses add: the scalar's gradient is the sum over all tokens
        assert abs(g_scalar[3].sum() - fd) < 1e-7 * max(1.0, abs(fd))


def test_single_step_closed_form():
    """T = 1: W1 = W0 - eta e k^T with e = W0 k - v, z = W1 q.  With M = dz q^T + dW_T
    (the cotangent of W1): dW0 = M (I - eta k k^T), dv = eta M k, deta = -e^T M k,
    dq = W1^T dz, dk = -eta (W0^T M k + M^T e)."""
    rng = np.random.default_rng(312)
    d = 5
    K, Q, V, eta, W0, dZ, dWT = rand_case(rng, 1, 1, d)
    dK, dQ, dV, deta, dW0 = oracle.linear_bwd(K, Q, V, eta, 0.0, W0, 1, dZ, dWT)
    k, q, v, et, W, dz = K[0, 0], Q[0, 0], V[0, 0], eta[0, 0], W0[0], dZ[0, 0]
    e = W @ k - v
    W1 = W - et * np.outer(e, k)
    M = np.outer(dz, q) + dWT[0]
    np.testing.assert_allclose(dW0[0], M @ (np.eye(d) - et * np.outer(k, k)), atol=1e-13)
    np.testing.assert_allclose(dV[0, 0], et * M @ k, atol=1e-13)
    np.testing.assert_allclose(deta[0, 0], -e @ M @ k, atol=1e-13)
    np.testing.assert_allclose(dQ[0, 0], W1.T @ dz, atol=1e-13)
    np.testing.assert_allclose(dK[0, 0], -et * (W.T @ M @ k + M.T @ e), atol=1e-13)


def test_linear_in_the_cotangent():
    rng = np.random.default_rng(313)
    K, Q, V, eta, W0, dZ1, dW1 = rand_case(rng, 3, 11, 4)
    dZ2 = rng.standard_normal(dZ1.shape)
    dW2 = rng.standard_normal(dW1.shape)
    a = -1.7
    g1 = oracle.linear_bwd(K, Q, V, eta, 0.0, W0, 4, dZ1, dW1)
    g2 = oracle.linear_bwd(K, Q, V, eta, 0.0, W0, 4, dZ2, dW2)
    g = oracle.linear_bwd(K, Q, V, eta, 0.0, W0, 4, a * dZ1 + dZ2, a * dW1 + dW2)
    for x, y, z in zip(g1, g2, g):
        np.testing.assert_allclose(z, a * x + y, rtol=1e-12, atol=1e-12)


def test_slices_are_independent():
    rng = np.random.default_rng(314)
    K, Q, V, eta, W0, dZ, dWT = rand_case(rng, 4, 9, 3)
    g = oracle.linear_bwd(K, Q, V, eta, 0.0, W0, 2, dZ, dWT, nthreads=3)
    for s in (0, 3):
        gs = oracle.linear_bwd(K[s:s + 1], Q[s:s + 1], V[s:s + 1], eta[s:s + 1], 0.0,
                               W0[s:s + 1], 2, dZ[s:s + 1], dWT[s:s + 1], nthreads=1)
        for a, b in zip(g, gs):
            np.testing.assert_array_equal(a[s:s + 1], b)
