"""Python binding of libttt_amd.so (the C ABI in include/ttt.h).

Argument marshalling only: torch provides device memory and the stream; every
step of the scan runs in the library's HIP kernels.  There is no fallback: if
the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libttt_amd.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_LAUNCH = 0, -1, -2, -3, -4
DTYPE_F32, DTYPE_BF16 = 0, 1
PLAN_AUTO, PLAN_GENERIC, PLAN_MFMA, PLAN_BIGCHUNK, PLAN_SPLIT = 0, 1, 2, 3, 4
READ_INCLUSIVE, READ_CHUNK_START = 0, 1

# every symbol include/ttt.h declares
EXPORTS = ("ttt_linear_workspace_bytes", "ttt_linear_workspace_bytes_ex",
           "ttt_linear_select_plan", "ttt_linear_fwd",
           "ttt_linear_step", "ttt_linear_bwd_workspace_bytes", "ttt_linear_bwd",
           "ttt_linear_fwd_ex", "ttt_linear_select_plan_ex",
           "ttt_linear_fwd_varlen", "ttt_linear_select_plan_varlen", "ttt_linear_ln_fwd",
           "ttt_linear_fwd_momentum", "ttt_linear_fwd_noalloc",
           "ttt_linear_noalloc_scratch_bytes",
           "ttt_mlp_workspace_bytes", "ttt_mlp_workspace_bytes_ex", "ttt_mlp_select_plan",
           "ttt_mlp_fwd", "ttt_mlp_fwd_ex",
           "ttt_status_string", "ttt_plan_name")


class TTTError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s: %s (status %d)" % (what, status_string(status), status))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libttt_amd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libttt_amd.so is not built (run __graft_entry__.build()); "
                               "the TTT scan has no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.ttt_linear_workspace_bytes.argtypes = [i] * 5
        L.ttt_linear_workspace_bytes.restype = sz
        L.ttt_linear_workspace_bytes_ex.argtypes = [i] * 7
        L.ttt_linear_workspace_bytes_ex.restype = sz
        L.ttt_linear_select_plan.argtypes = [i] * 7
        L.ttt_linear_select_plan.restype = i
        L.ttt_linear_fwd.argtypes = [vp, vp, vp, vp, f, vp, vp, vp, i, i, i, i, i, i, vp, sz, vp]
        L.ttt_linear_fwd.restype = i
        L.ttt_linear_fwd_ex.argtypes = [vp, vp, vp, vp, f, vp, vp, vp, i, i, i, i, i, i, vp, sz,
                                        vp, i, i]
        L.ttt_linear_fwd_ex.restype = i
        L.ttt_linear_fwd_noalloc.argtypes = [vp, vp, vp, vp, f, vp, vp, vp, i, i, i, i, i, i, vp]
        L.ttt_linear_fwd_noalloc.restype = i
        L.ttt_linear_noalloc_scratch_bytes.argtypes = []
        L.ttt_linear_noalloc_scratch_bytes.restype = sz
        L.ttt_linear_fwd_momentum.argtypes = [vp, vp, vp, vp, f, vp, vp, f, vp, vp, vp,
                                              i, i, i, i, i, i, vp, sz, vp, i]
        L.ttt_linear_fwd_momentum.restype = i
        L.ttt_linear_ln_fwd.argtypes = [vp, vp, vp, vp, f, vp, vp, vp, vp, f, vp, vp, vp,
                                        i, i, i, i, i, i, vp]
        L.ttt_linear_ln_fwd.restype = i
        L.ttt_linear_fwd_varlen.argtypes = [vp, vp, vp, vp, f, vp, vp, vp, vp, i, i, i, i, i, i,
                                            vp, i]
        L.ttt_linear_fwd_varlen.restype = i
        L.ttt_linear_select_plan_varlen.argtypes = [i] * 7
        L.ttt_linear_select_plan_varlen.restype = i
        L.ttt_linear_select_plan_ex.argtypes = [i] * 8
        L.ttt_linear_select_plan_ex.restype = i
        L.ttt_linear_bwd_workspace_bytes.argtypes = [i] * 6
        L.ttt_linear_bwd_workspace_bytes.restype = sz
        L.ttt_linear_bwd.argtypes = [vp, vp, vp, vp, f, vp, vp, vp, vp, vp, vp, vp, vp,
                                     i, i, i, i, i, i, vp, sz, vp]
        L.ttt_linear_bwd.restype = i
        L.ttt_linear_step.argtypes = [vp, vp, vp, vp, f, vp, vp, i, vp, i, i, i, i, i, i, vp]
        L.ttt_linear_step.restype = i
        L.ttt_mlp_workspace_bytes.argtypes = [i] * 5
        L.ttt_mlp_workspace_bytes.restype = sz
        L.ttt_mlp_workspace_bytes_ex.argtypes = [i] * 7
        L.ttt_mlp_workspace_bytes_ex.restype = sz
        L.ttt_mlp_select_plan.argtypes = [i] * 7
        L.ttt_mlp_select_plan.restype = i
        L.ttt_mlp_fwd.argtypes = [vp, vp, vp, vp, f, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                  i, i, i, i, i, i, vp, sz, vp]
        L.ttt_mlp_fwd.restype = i
        L.ttt_mlp_fwd_ex.argtypes = [vp, vp, vp, vp, f, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     i, i, i, i, i, i, vp, sz, vp, i]
        L.ttt_mlp_fwd_ex.restype = i
        L.ttt_status_string.argtypes = [i]
        L.ttt_status_string.restype = ctypes.c_char_p
        L.ttt_plan_name.argtypes = [i]
        L.ttt_plan_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ttt_status_string(int(status)).decode()


def plan_name(plan: int) -> str:
    return lib().ttt_plan_name(int(plan)).decode()


def _io_dtype(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError("K/Q/V must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device, stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _check(t, name, shape, dtype=None):
    import torch
    if t is None:
        raise ValueError("%s is required" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s" % (name, dtype))


def linear_workspace_bytes(B, H, T, d, chunk, io_dtype=None, plan=PLAN_AUTO) -> int:
    """Workspace bytes for the shape; with io_dtype, for that dtype and plan exactly."""
    if io_dtype is None:
        return int(lib().ttt_linear_workspace_bytes(B, H, T, d, chunk))
    return int(lib().ttt_linear_workspace_bytes_ex(B, H, T, d, chunk, io_dtype, plan))


def linear_select_plan(B, H, T, d, chunk, io_dtype, plan=PLAN_AUTO,
                       read_mode: int = READ_INCLUSIVE) -> int:
    if read_mode == READ_INCLUSIVE:
        return int(lib().ttt_linear_select_plan(B, H, T, d, chunk, io_dtype, plan))
    return int(lib().ttt_linear_select_plan_ex(B, H, T, d, chunk, io_dtype, plan, read_mode))


def mlp_workspace_bytes(B, H, T, d, chunk, io_dtype=None, plan=PLAN_AUTO) -> int:
    """Workspace bytes for the shape; with io_dtype, for that dtype and plan exactly."""
    if io_dtype is None:
        return int(lib().ttt_mlp_workspace_bytes(B, H, T, d, chunk))
    return int(lib().ttt_mlp_workspace_bytes_ex(B, H, T, d, chunk, io_dtype, plan))


def mlp_select_plan(B, H, T, d, chunk, io_dtype, plan=PLAN_AUTO) -> int:
    return int(lib().ttt_mlp_select_plan(B, H, T, d, chunk, io_dtype, plan))


def _workspace(nbytes, device, workspace):
    import torch
    if nbytes == 0:
        return None
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace


def linear_fwd(K, Q, V, eta, W0, chunk: int, eta_scalar: float = 0.0, *, Z=None, W_out=None,
               workspace=None, plan: int = PLAN_AUTO, stream=None,
               read_mode: int = READ_INCLUSIVE) -> Tuple:
    """TTT-Linear forward scan.  K, Q, V: [B, H, T, d] fp32 or bf16; eta: [B, H, T]
    fp32 or None (then eta_scalar); W0: [B, H, d, d] fp32; read_mode: READ_INCLUSIVE
    or READ_CHUNK_START.  Returns (Z, W_out)."""
    import torch
    B, H, T, d = K.shape
    _check(K, "K", (B, H, T, d))
    _check(Q, "Q", (B, H, T, d), K.dtype)
    _check(V, "V", (B, H, T, d), K.dtype)
    _check(W0, "W0", (B, H, d, d), torch.float32)
    if eta is not None:
        _check(eta, "eta", (B, H, T), torch.float32)
    if Z is None:
        Z = torch.empty_like(K)
    if W_out is None:
        W_out = torch.empty_like(W0)
    _check(Z, "Z", (B, H, T, d), K.dtype)
    _check(W_out, "W_out", (B, H, d, d), torch.float32)
    io = _io_dtype(K)
    p = linear_select_plan(B, H, T, d, chunk, io, plan, read_mode)
    nbytes = linear_workspace_bytes(B, H, T, d, chunk, io, p) if p > 0 else 0
    ws = _workspace(nbytes, K.device, workspace)
    rc = lib().ttt_linear_fwd_ex(K.data_ptr(), Q.data_ptr(), V.data_ptr(), _ptr(eta),
                                 float(eta_scalar), W0.data_ptr(), Z.data_ptr(),
                                 W_out.data_ptr(), B, H, T, d, int(chunk), io, _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream(K.device, stream),
                                 int(plan), int(read_mode))
    if rc != OK:
        raise TTTError(rc, "ttt_linear_fwd")
    return Z, W_out


def linear_fwd_noalloc(K, Q, V, eta, W0, chunk: int, eta_scalar: float = 0.0, *, Z, W_out,
                       stream=None) -> Tuple:
    """ttt_linear_fwd_noalloc: the AUTO-plan scan with any workspace taken from the
    library's static per-GPU scratch.  Z and W_out are caller-given (this call
    allocates nothing).  Returns (Z, W_out)."""
    import torch
    B, H, T, d = K.shape
    _check(K, "K", (B, H, T, d))
    _check(Q, "Q", (B, H, T, d), K.dtype)
    _check(V, "V", (B, H, T, d), K.dtype)
    _check(W0, "W0", (B, H, d, d), torch.float32)
    if eta is not None:
        _check(eta, "eta", (B, H, T), torch.float32)
    _check(Z, "Z", (B, H, T, d), K.dtype)
    _check(W_out, "W_out", (B, H, d, d), torch.float32)
    rc = lib().ttt_linear_fwd_noalloc(K.data_ptr(), Q.data_ptr(), V.data_ptr(), _ptr(eta),
                                      float(eta_scalar), W0.data_ptr(), Z.data_ptr(),
                                      W_out.data_ptr(), B, H, T, d, int(chunk), _io_dtype(K),
                                      _stream(K.device, stream))
    if rc != OK:
        raise TTTError(rc, "ttt_linear_fwd_noalloc")
    return Z, W_out


def linear_noalloc_scratch_bytes() -> int:
    return int(lib().ttt_linear_noalloc_scratch_bytes())


def linear_bwd_workspace_bytes(B, H, T, d, chunk, io_dtype) -> int:
    return int(lib().ttt_linear_bwd_workspace_bytes(B, H, T, d, chunk, io_dtype))


def linear_bwd(K, Q, V, eta, W0, dZ, chunk: int, eta_scalar: float = 0.0, dW_T=None, *,
               dK=None, dQ=None, dV=None, deta=None, dW0=None, want_deta: bool = True,
               workspace=None, stream=None) -> Tuple:
    """Gradients of <dZ, Z> + <dW_T, W_T> through linear_fwd(K, Q, V, eta, W0, chunk).
    dZ: like K; dW_T: [B, H, d, d] fp32 or None.  Returns (dK, dQ, dV, deta, dW0);
    deta [B, H, T] fp32 is per token (None when want_deta is False)."""
    import torch
    B, H, T, d = K.shape
    _check(K, "K", (B, H, T, d))
    _check(Q, "Q", (B, H, T, d), K.dtype)
    _check(V, "V", (B, H, T, d), K.dtype)
    _check(dZ, "dZ", (B, H, T, d), K.dtype)
    _check(W0, "W0", (B, H, d, d), torch.float32)
    if eta is not None:
        _check(eta, "eta", (B, H, T), torch.float32)
    if dW_T is not None:
        _check(dW_T, "dW_T", (B, H, d, d), torch.float32)
    dK = torch.empty_like(K) if dK is None else dK
    dQ = torch.empty_like(K) if dQ is None else dQ
    dV = torch.empty_like(K) if dV is None else dV
    dW0 = torch.empty_like(W0) if dW0 is None else dW0
    if want_deta and deta is None:
        deta = torch.empty((B, H, T), dtype=torch.float32, device=K.device)
    for t, name in ((dK, "dK"), (dQ, "dQ"), (dV, "dV")):
        _check(t, name, (B, H, T, d), K.dtype)
    _check(dW0, "dW0", (B, H, d, d), torch.float32)
    if deta is not None:
        _check(deta, "deta", (B, H, T), torch.float32)
    io = _io_dtype(K)
    nbytes = linear_bwd_workspace_bytes(B, H, T, d, chunk, io)
    if nbytes == 0:
        raise TTTError(ERR_UNSUPPORTED, "ttt_linear_bwd")
    ws = _workspace(nbytes, K.device, workspace)
    rc = lib().ttt_linear_bwd(K.data_ptr(), Q.data_ptr(), V.data_ptr(), _ptr(eta),
                              float(eta_scalar), W0.data_ptr(), dZ.data_ptr(), _ptr(dW_T),
                              dK.data_ptr(), dQ.data_ptr(), dV.data_ptr(), _ptr(deta),
                              dW0.data_ptr(), B, H, T, d, int(chunk), io, _ptr(ws),
                              ws.numel(), _stream(K.device, stream))
    if rc != OK:
        raise TTTError(rc, "ttt_linear_bwd")
    return dK, dQ, dV, deta, dW0


def linear_step(K, Q, V, eta, W_chunk, G, pos: int, chunk: int, eta_scalar: float = 0.0, *,
                Z=None, stream=None):
    """Continue TTT-Linear scans by n tokens from a carried state, in place.
    K, Q, V: [B, H, n, d] fp32 or bf16; eta: [B, H, n] fp32 or None; W_chunk (the
    chunk-start state) and G (the chunk's update so far): [B, H, d, d] fp32, both
    updated in place; pos: tokens of the current chunk already read.  Returns
    (Z, new pos); the state after the last token is W_chunk - G."""
    import torch
    B, H, n, d = K.shape
    _check(K, "K", (B, H, n, d))
    _check(Q, "Q", (B, H, n, d), K.dtype)
    _check(V, "V", (B, H, n, d), K.dtype)
    _check(W_chunk, "W_chunk", (B, H, d, d), torch.float32)
    _check(G, "G", (B, H, d, d), torch.float32)
    if eta is not None:
        _check(eta, "eta", (B, H, n), torch.float32)
    if Z is None:
        Z = torch.empty_like(K)
    _check(Z, "Z", (B, H, n, d), K.dtype)
    rc = lib().ttt_linear_step(K.data_ptr(), Q.data_ptr(), V.data_ptr(), _ptr(eta),
                               float(eta_scalar), W_chunk.data_ptr(), G.data_ptr(), int(pos),
                               Z.data_ptr(), B, H, n, d, int(chunk), _io_dtype(K),
                               _stream(K.device, stream))
    if rc != OK:
        raise TTTError(rc, "ttt_linear_step")
    return Z, (int(pos) + n) % int(chunk)


def linear_fwd_momentum(K, Q, V, eta, W0, Mom0, beta: float, chunk: int,
                        eta_scalar: float = 0.0, *, Z=None, W_out=None, Mom_out=None,
                        workspace=None, plan: int = PLAN_AUTO, stream=None) -> Tuple:
    """TTT-Linear with a momentum state and chunk-start reads.  Mom0: [B, H, d, d]
    fp32 or None (zero).  Returns (Z, W_out, Mom_out)."""
    import torch
    B, H, T, d = K.shape
    _check(K, "K", (B, H, T, d))
    _check(Q, "Q", (B, H, T, d), K.dtype)
    _check(V, "V", (B, H, T, d), K.dtype)
    _check(W0, "W0", (B, H, d, d), torch.float32)
    if Mom0 is not None:
        _check(Mom0, "Mom0", (B, H, d, d), torch.float32)
    if eta is not None:
        _check(eta, "eta", (B, H, T), torch.float32)
    Z = torch.empty_like(K) if Z is None else Z
    W_out = torch.empty_like(W0) if W_out is None else W_out
    Mom_out = torch.empty_like(W0) if Mom_out is None else Mom_out
    io = _io_dtype(K)
    p = linear_select_plan(B, H, T, d, chunk, io, plan, READ_CHUNK_START)
    nbytes = linear_workspace_bytes(B, H, T, d, chunk, io, p) if p > 0 else 0
    ws = _workspace(nbytes, K.device, workspace)
    rc = lib().ttt_linear_fwd_momentum(K.data_ptr(), Q.data_ptr(), V.data_ptr(), _ptr(eta),
                                       float(eta_scalar), W0.data_ptr(), _ptr(Mom0), float(beta),
                                       Z.data_ptr(), W_out.data_ptr(), Mom_out.data_ptr(),
                                       B, H, T, d, int(chunk), io, _ptr(ws),
                                       0 if ws is None else ws.numel(),
                                       _stream(K.device, stream), int(plan))
    if rc != OK:
        raise TTTError(rc, "ttt_linear_fwd_momentum")
    return Z, W_out, Mom_out


def linear_ln_fwd(K, Q, V, eta, W0, b0, ln_weight, ln_bias, chunk: int, eps: float = 1e-6,
                  eta_scalar: float = 0.0, *, Z=None, W_out=None, b_out=None,
                  stream=None) -> Tuple:
    """TTT-Linear with f(x) = x + LN(W x + b) (ln_weight, ln_bias: [H, d]) or
    f(x) = W x + b (both None).  b0: [B, H, d].  Returns (Z, W_out, b_out)."""
    import torch
    B, H, T, d = K.shape
    _check(K, "K", (B, H, T, d))
    _check(Q, "Q", (B, H, T, d), K.dtype)
    _check(V, "V", (B, H, T, d), K.dtype)
    _check(W0, "W0", (B, H, d, d), torch.float32)
    _check(b0, "b0", (B, H, d), torch.float32)
    if (ln_weight is None) != (ln_bias is None):
        raise ValueError("ln_weight and ln_bias go together")
    if ln_weight is not None:
        _check(ln_weight, "ln_weight", (H, d), torch.float32)
        _check(ln_bias, "ln_bias", (H, d), torch.float32)
    if eta is not None:
        _check(eta, "eta", (B, H, T), torch.float32)
    Z = torch.empty_like(K) if Z is None else Z
    W_out = torch.empty_like(W0) if W_out is None else W_out
    b_out = torch.empty_like(b0) if b_out is None else b_out
    rc = lib().ttt_linear_ln_fwd(K.data_ptr(), Q.data_ptr(), V.data_ptr(), _ptr(eta),
                                 float(eta_scalar), W0.data_ptr(), b0.data_ptr(), _ptr(ln_weight),
                                 _ptr(ln_bias), float(eps), Z.data_ptr(), W_out.data_ptr(),
                                 b_out.data_ptr(), B, H, T, d, int(chunk), _io_dtype(K),
                                 _stream(K.device, stream))
    if rc != OK:
        raise TTTError(rc, "ttt_linear_ln_fwd")
    return Z, W_out, b_out


def linear_select_plan_varlen(n_docs, H, total_T, d, chunk, io_dtype, plan=PLAN_AUTO) -> int:
    return int(lib().ttt_linear_select_plan_varlen(n_docs, H, total_T, d, chunk, io_dtype, plan))


def linear_fwd_varlen(K, Q, V, eta, W0, cu_seqlens, chunk: int, eta_scalar: float = 0.0, *,
                      Z=None, W_out=None, plan: int = PLAN_AUTO, stream=None) -> Tuple:
    """TTT-Linear over packed documents, each reset to its own initial state.
    K, Q, V: [H, total_T, d]; eta: [H, total_T] or None; W0: [n_docs, H, d, d];
    cu_seqlens: int32 device tensor [n_docs + 1].  Returns (Z, W_out)."""
    import torch
    H, total_T, d = K.shape
    n_docs = cu_seqlens.numel() - 1
    _check(K, "K", (H, total_T, d))
    _check(Q, "Q", (H, total_T, d), K.dtype)
    _check(V, "V", (H, total_T, d), K.dtype)
    _check(W0, "W0", (n_docs, H, d, d), torch.float32)
    _check(cu_seqlens, "cu_seqlens", (n_docs + 1,), torch.int32)
    if eta is not None:
        _check(eta, "eta", (H, total_T), torch.float32)
    if Z is None:
        Z = torch.zeros_like(K)
    if W_out is None:
        W_out = torch.empty_like(W0)
    _check(Z, "Z", (H, total_T, d), K.dtype)
    _check(W_out, "W_out", (n_docs, H, d, d), torch.float32)
    rc = lib().ttt_linear_fwd_varlen(K.data_ptr(), Q.data_ptr(), V.data_ptr(), _ptr(eta),
                                     float(eta_scalar), W0.data_ptr(), Z.data_ptr(),
                                     W_out.data_ptr(), cu_seqlens.data_ptr(), n_docs, H, total_T,
                                     d, int(chunk), _io_dtype(K), _stream(K.device, stream),
                                     int(plan))
    if rc != OK:
        raise TTTError(rc, "ttt_linear_fwd_varlen")
    return Z, W_out


def mlp_fwd(K, Q, V, eta, W1, b1, W2, b2, chunk: int, eta_scalar: float = 0.0, *, Z=None,
            W1_out=None, b1_out=None, W2_out=None, b2_out=None, workspace=None,
            plan: int = PLAN_AUTO, stream=None) -> Tuple:
    """TTT-MLP forward scan (hidden 4d).  W1: [B, H, 4d, d], b1: [B, H, 4d] or None,
    W2: [B, H, d, 4d], b2: [B, H, d] or None.  Returns (Z, W1, b1, W2, b2) final."""
    import torch
    B, H, T, d = K.shape
    hd = 4 * d
    _check(K, "K", (B, H, T, d))
    _check(Q, "Q", (B, H, T, d), K.dtype)
    _check(V, "V", (B, H, T, d), K.dtype)
    _check(W1, "W1", (B, H, hd, d), torch.float32)
    _check(W2, "W2", (B, H, d, hd), torch.float32)
    if b1 is not None:
        _check(b1, "b1", (B, H, hd), torch.float32)
    if b2 is not None:
        _check(b2, "b2", (B, H, d), torch.float32)
    if eta is not None:
        _check(eta, "eta", (B, H, T), torch.float32)
    Z = torch.empty_like(K) if Z is None else Z
    W1_out = torch.empty_like(W1) if W1_out is None else W1_out
    W2_out = torch.empty_like(W2) if W2_out is None else W2_out
    if b1 is not None and b1_out is None:
        b1_out = torch.empty_like(b1)
    if b2 is not None and b2_out is None:
        b2_out = torch.empty_like(b2)
    io = _io_dtype(K)
    nbytes = mlp_workspace_bytes(B, H, T, d, chunk, io, plan)
    ws = _workspace(nbytes, K.device, workspace)
    rc = lib().ttt_mlp_fwd_ex(K.data_ptr(), Q.data_ptr(), V.data_ptr(), _ptr(eta),
                              float(eta_scalar), W1.data_ptr(), _ptr(b1), W2.data_ptr(), _ptr(b2),
                              Z.data_ptr(), W1_out.data_ptr(), _ptr(b1_out), W2_out.data_ptr(),
                              _ptr(b2_out), B, H, T, d, int(chunk), io, _ptr(ws),
                              0 if ws is None else ws.numel(), _stream(K.device, stream),
                              int(plan))
    if rc != OK:
        raise TTTError(rc, "ttt_mlp_fwd")
    return Z, W1_out, b1_out, W2_out, b2_out
