"""ctypes wrapper around libttt_oracle.so (plain C, fp64) — TEST INFRASTRUCTURE ONLY.

Forward scans of TTT-Linear and TTT-MLP, and the vector-Jacobian product of the
TTT-Linear scan."""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ttt_oracle.c")
_LIB = os.path.join(_HERE, "libttt_oracle.so")
# a prebuilt oracle library to load instead (the mutation tests point this at
# copies of the oracle with a planted mistake)
_LIB_OVERRIDE = os.environ.get("TTT_ORACLE_LIB")
_lib = None


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O3, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off",
                               "-fno-fast-math", "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp,
                               "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
        P = ctypes.POINTER(ctypes.c_double)
        lib.ttt_oracle_linear.argtypes = [P, P, P, P, ctypes.c_double, P, P, P,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int]
        lib.ttt_oracle_linear.restype = ctypes.c_int
        lib.ttt_oracle_linear_read.argtypes = [P, P, P, P, ctypes.c_double, P, P, P,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.ttt_oracle_linear_read.restype = ctypes.c_int
        lib.ttt_oracle_linear_momentum.argtypes = [P, P, P, P, ctypes.c_double, P, P,
                                                   ctypes.c_double, P, P, P,
                                                   ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                   ctypes.c_int, ctypes.c_int]
        lib.ttt_oracle_linear_momentum.restype = ctypes.c_int
        lib.ttt_oracle_linear_ln.argtypes = [P, P, P, P, ctypes.c_double, P, P, P, P,
                                             ctypes.c_double, P, P, P,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int]
        lib.ttt_oracle_linear_ln.restype = ctypes.c_int
        lib.ttt_oracle_linear_bwd.argtypes = [P, P, P, P, ctypes.c_double, P, P, P,
                                              P, P, P, P, P,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int]
        lib.ttt_oracle_linear_bwd.restype = ctypes.c_int
        lib.ttt_oracle_mlp.argtypes = [P, P, P, P, ctypes.c_double, P, P, P, P,
                                       P, P, P, P, P,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.ttt_oracle_mlp.restype = ctypes.c_int
        lib.ttt_oracle_gelu.argtypes = [ctypes.c_double]
        lib.ttt_oracle_gelu.restype = ctypes.c_double
        lib.ttt_oracle_gelu_prime.argtypes = [ctypes.c_double]
        lib.ttt_oracle_gelu_prime.restype = ctypes.c_double
        _lib = lib
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def linear(K, Q, V, eta, eta_scalar: float, W0, chunk: int,
           nthreads: int = 0, return_threads: bool = False, read_start: bool = False):
    """TTT-Linear scan.  K, Q, V: [n, T, d]; eta: [n, T] or None; W0: [n, d, d].
    read_start: every token of a chunk reads with the chunk-start state (apply,
    then update) instead of the inclusive read.
    Returns (Z [n, T, d], W_T [n, d, d]) in fp64 (and the thread count if asked)."""
    K, Q, V, W0 = _f64(K), _f64(Q), _f64(V), _f64(W0)
    eta = _f64(eta)
    n, T, d = K.shape
    assert Q.shape == K.shape == V.shape and W0.shape == (n, d, d)
    if eta is not None:
        assert eta.shape == (n, T)
    Z = np.empty((n, T, d), np.float64)
    W = np.empty((n, d, d), np.float64)
    rc = _load().ttt_oracle_linear_read(_ptr(K), _ptr(Q), _ptr(V), _ptr(eta),
                                        float(eta_scalar), _ptr(W0), _ptr(Z), _ptr(W), n, T, d,
                                        int(chunk), int(bool(read_start)), int(nthreads))
    if rc <= 0:
        raise ValueError("ttt_oracle_linear rejected its arguments")
    return (Z, W, rc) if return_threads else (Z, W)


def linear_momentum(K, Q, V, eta, eta_scalar: float, W0, M0, beta: float, chunk: int,
                    nthreads: int = 0, return_threads: bool = False):
    """TTT-Linear with a momentum state (chunk-start reads).  M0: [n, d, d] or None.
    Returns (Z, W_T, M_T) in fp64."""
    K, Q, V, W0, M0, eta = _f64(K), _f64(Q), _f64(V), _f64(W0), _f64(M0), _f64(eta)
    n, T, d = K.shape
    Z = np.empty((n, T, d), np.float64)
    W = np.empty((n, d, d), np.float64)
    M = np.empty((n, d, d), np.float64)
    rc = _load().ttt_oracle_linear_momentum(_ptr(K), _ptr(Q), _ptr(V), _ptr(eta),
                                            float(eta_scalar), _ptr(W0), _ptr(M0), float(beta),
                                            _ptr(Z), _ptr(W), _ptr(M), n, T, d, int(chunk),
                                            int(nthreads))
    if rc <= 0:
        raise ValueError("ttt_oracle_linear_momentum rejected its arguments")
    return (Z, W, M, rc) if return_threads else (Z, W, M)


def linear_ln(K, Q, V, eta, eta_scalar: float, W0, b0, ln_weight, ln_bias, eps: float,
              chunk: int, nthreads: int = 0, return_threads: bool = False):
    """TTT-Linear with the bias as state and f(x) = x + LN(W x + b) (LayerNorm and
    residual inside f), or f(x) = W x + b when ln_weight and ln_bias are None.
    b0, ln_weight, ln_bias: [n, d].  Returns (Z, W_T, b_T) in fp64."""
    K, Q, V, W0, b0 = _f64(K), _f64(Q), _f64(V), _f64(W0), _f64(b0)
    eta, lnw, lnb = _f64(eta), _f64(ln_weight), _f64(ln_bias)
    n, T, d = K.shape
    assert W0.shape == (n, d, d) and b0.shape == (n, d)
    Z = np.empty((n, T, d), np.float64)
    W = np.empty((n, d, d), np.float64)
    b = np.empty((n, d), np.float64)
    rc = _load().ttt_oracle_linear_ln(_ptr(K), _ptr(Q), _ptr(V), _ptr(eta), float(eta_scalar),
                                      _ptr(W0), _ptr(b0), _ptr(lnw), _ptr(lnb), float(eps),
                                      _ptr(Z), _ptr(W), _ptr(b), n, T, d, int(chunk),
                                      int(nthreads))
    if rc <= 0:
        raise ValueError("ttt_oracle_linear_ln rejected its arguments")
    return (Z, W, b, rc) if return_threads else (Z, W, b)


def linear_bwd(K, Q, V, eta, eta_scalar: float, W0, chunk: int, dZ, dW_T=None,
               nthreads: int = 0, return_threads: bool = False):
    """Gradient of L = <dZ, Z> + <dW_T, W_T> through the TTT-Linear scan.
    dZ: [n, T, d]; dW_T: [n, d, d] or None (zero).  Returns (dK, dQ, dV, deta [n, T],
    dW0) in fp64; deta is per token also when eta is None (eta_scalar for all)."""
    K, Q, V, W0, dZ = _f64(K), _f64(Q), _f64(V), _f64(W0), _f64(dZ)
    eta, dW_T = _f64(eta), _f64(dW_T)
    n, T, d = K.shape
    assert Q.shape == K.shape == V.shape == dZ.shape and W0.shape == (n, d, d)
    if eta is not None:
        assert eta.shape == (n, T)
    if dW_T is not None:
        assert dW_T.shape == (n, d, d)
    dK = np.empty((n, T, d), np.float64)
    dQ = np.empty((n, T, d), np.float64)
    dV = np.empty((n, T, d), np.float64)
    deta = np.empty((n, T), np.float64)
    dW0 = np.empty((n, d, d), np.float64)
    rc = _load().ttt_oracle_linear_bwd(_ptr(K), _ptr(Q), _ptr(V), _ptr(eta), float(eta_scalar),
                                       _ptr(W0), _ptr(dZ), _ptr(dW_T), _ptr(dK), _ptr(dQ),
                                       _ptr(dV), _ptr(deta), _ptr(dW0), n, T, d, int(chunk),
                                       int(nthreads))
    if rc <= 0:
        raise ValueError("ttt_oracle_linear_bwd rejected its arguments")
    res = (dK, dQ, dV, deta, dW0)
    return res + (rc,) if return_threads else res


def mlp(K, Q, V, eta, eta_scalar: float, W1, b1, W2, b2, chunk: int,
        nthreads: int = 0, return_threads: bool = False):
    """TTT-MLP scan.  W1: [n, hd, d], b1: [n, hd] or None, W2: [n, d, hd],
    b2: [n, d] or None.  Returns (Z, W1_T, b1_T, W2_T, b2_T) in fp64."""
    K, Q, V, W1, W2 = _f64(K), _f64(Q), _f64(V), _f64(W1), _f64(W2)
    eta, b1, b2 = _f64(eta), _f64(b1), _f64(b2)
    n, T, d = K.shape
    hd = W1.shape[1]
    assert W1.shape == (n, hd, d) and W2.shape == (n, d, hd)
    Z = np.empty((n, T, d), np.float64)
    W1o = np.empty_like(W1)
    W2o = np.empty_like(W2)
    b1o = np.empty((n, hd), np.float64) if b1 is not None else None
    b2o = np.empty((n, d), np.float64) if b2 is not None else None
    rc = _load().ttt_oracle_mlp(_ptr(K), _ptr(Q), _ptr(V), _ptr(eta), float(eta_scalar),
                                _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
                                _ptr(Z), _ptr(W1o), _ptr(b1o), _ptr(W2o), _ptr(b2o),
                                n, T, d, hd, int(chunk), int(nthreads))
    if rc <= 0:
        raise ValueError("ttt_oracle_mlp rejected its arguments")
    res = (Z, W1o, b1o, W2o, b2o)
    return res + (rc,) if return_threads else res


def gelu(x: float) -> float:
    return _load().ttt_oracle_gelu(float(x))


def gelu_prime(x: float) -> float:
    return _load().ttt_oracle_gelu_prime(float(x))
