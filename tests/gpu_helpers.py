"""Helpers for the GPU parity tests: move seeded inputs to the device, run the HIP
path through the binding, and measure the error against the oracle."""
from __future__ import annotations

import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}   # max relative error per (batch, head) slice


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(gpu, ref, floor=1e-6):
    """max over slices of max|gpu - ref| / max|ref| (slices on axis 0)."""
    g = np.asarray(gpu, np.float64).reshape(ref.shape[0], -1)
    r = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    den = np.maximum(np.abs(r).max(axis=1), floor)
    return float((np.abs(g - r).max(axis=1) / den).max())


def device_inputs(wl, x, dev, eta_offset=0):
    """Device copies of the inputs.  eta_offset > 0 places eta that many floats into
    its allocation, so its pointer is 4-byte but not 16-byte aligned."""
    import torch
    io = torch.bfloat16 if wl.io == "bf16" else torch.float32
    B, H, T, d = wl.B, wl.H, wl.T, wl.d

    def t(a, shape, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).reshape(shape).to(dt).contiguous()

    out = {k: t(x[k], (B, H, T, d), io) for k in ("K", "Q", "V")}
    if x["eta"] is None:
        out["eta"] = None
    elif eta_offset:
        buf = torch.zeros(B * H * T + eta_offset, dtype=torch.float32, device=dev)
        buf[eta_offset:] = torch.from_numpy(np.ascontiguousarray(x["eta"]).reshape(-1)).to(dev)
        out["eta"] = buf[eta_offset:].view(B, H, T)
    else:
        out["eta"] = t(x["eta"], (B, H, T))
    if wl.model == "linear":
        out["W0"] = t(x["W0"], (B, H, d, d))
    else:
        hd = wl.hidden
        out["W1"] = t(x["W1"], (B, H, hd, d))
        out["W2"] = t(x["W2"], (B, H, d, hd))
        out["b1"] = None if x["b1"] is None else t(x["b1"], (B, H, hd))
        out["b2"] = None if x["b2"] is None else t(x["b2"], (B, H, d))
    return out


def host(t, n):
    return t.float().cpu().numpy().reshape(n, *t.shape[2:])


def run_linear(wl, x, dev, plan=0, eta_offset=0, **kw):
    import torch
    from test_sequence_layers_ttt_amd import ttt
    a = device_inputs(wl, x, dev, eta_offset)
    Z, W = ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], wl.chunk,
                          eta_scalar=x["eta_scalar"], plan=plan, **kw)
    torch.cuda.synchronize()
    return host(Z, wl.BH), host(W, wl.BH)


def run_mlp(wl, x, dev, plan=0, eta_offset=0, **kw):
    import torch
    from test_sequence_layers_ttt_amd import ttt
    a = device_inputs(wl, x, dev, eta_offset)
    res = ttt.mlp_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W1"], a["b1"], a["W2"], a["b2"],
                      wl.chunk, eta_scalar=x["eta_scalar"], plan=plan, **kw)
    torch.cuda.synchronize()
    return tuple(None if r is None else host(r, wl.BH) for r in res)


def take(x, idx):
    """Restrict stacked inputs to the slices `idx` (for the oracle)."""
    out = {}
    for k, v in x.items():
        if isinstance(v, np.ndarray):
            out[k] = v[idx]
        else:
            out[k] = v
    return out
