"""fp64 numpy "dual form" of the chunked TTT scan — test-only brute force.

This is a second, independently written formulation used to pin the oracle:
the oracle runs the per-token primal loop, this file rewrites each chunk's
outer products as matrix products with an inclusive causal mask (the dual form
of diosapp "Test-Time Training (TTT) guide" §3 and PaperTrace
"5 · TestingTime 训练与长上下文" §1.1).  Token-row layout: K_c, Q_c, V_c are
n x d, row t is token t; the mask keeps writer s <= reader t.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf


def linear_dual(K, Q, V, eta, eta_scalar, W0, chunk):
    """One slice: K, Q, V [T, d]; eta [T] or None; W0 [d, d] -> (Z [T, d], W_T)."""
    K, Q, V, W = (np.asarray(a, np.float64) for a in (K, Q, V, W0))
    T, d = K.shape
    et = np.full(T, float(eta_scalar)) if eta is None else np.asarray(eta, np.float64)
    Z = np.zeros((T, d))
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(T, c0 + chunk))
        Kc, Qc, Vc, ec = K[sl], Q[sl], V[sl], et[sl]
        E = Kc @ W.T - Vc                                  # row s: W k_s - v_s
        S = np.tril(Qc @ Kc.T)                             # [t, s] = q_t . k_s, s <= t
        Z[sl] = Qc @ W.T - (S * ec[None, :]) @ E
        W = W - (E * ec[:, None]).T @ Kc
    return Z, W


def _gelu(x):
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def _gelu_prime(x):
    return 0.5 * (1.0 + erf(x / np.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)


def mlp_dual(K, Q, V, eta, eta_scalar, W1, b1, W2, b2, chunk):
    """One slice of TTT-MLP in dual form.  b1/b2 None = bias-free model."""
    K, Q, V = (np.asarray(a, np.float64) for a in (K, Q, V))
    W1 = np.asarray(W1, np.float64).copy()
    W2 = np.asarray(W2, np.float64).copy()
    has_b1, has_b2 = b1 is not None, b2 is not None
    b1 = np.asarray(b1, np.float64).copy() if has_b1 else np.zeros(W1.shape[0])
    b2 = np.asarray(b2, np.float64).copy() if has_b2 else np.zeros(W2.shape[0])
    T, d = K.shape
    et = np.full(T, float(eta_scalar)) if eta is None else np.asarray(eta, np.float64)
    Z = np.zeros((T, d))
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(T, c0 + chunk))
        Kc, Qc, Vc, ec = K[sl], Q[sl], V[sl], et[sl]
        Hk = Kc @ W1.T + b1
        A = _gelu(Hk)
        E = A @ W2.T + b2 - Vc
        Dl = (E @ W2) * _gelu_prime(Hk)
        M1 = np.tril(Qc @ Kc.T + (1.0 if has_b1 else 0.0))
        Hq = Qc @ W1.T + b1 - (M1 * ec[None, :]) @ Dl
        Aq = _gelu(Hq)
        M2 = np.tril(Aq @ A.T + (1.0 if has_b2 else 0.0))
        Z[sl] = Aq @ W2.T + b2 - (M2 * ec[None, :]) @ E
        W1 = W1 - (Dl * ec[:, None]).T @ Kc
        W2 = W2 - (E * ec[:, None]).T @ A
        if has_b1:
            b1 = b1 - ec @ Dl
        if has_b2:
            b2 = b2 - ec @ E
    return Z, W1, (b1 if has_b1 else None), W2, (b2 if has_b2 else None)
