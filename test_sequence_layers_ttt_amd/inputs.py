"""Seeded synthetic inputs for the TTT scan.

This module is the only code shared by the HIP path's callers (tests, bench,
smoke) and the CPU oracle's callers.  It draws random numbers and rounds them to
the I/O dtype; it holds none of the scan's arithmetic.

The pages describe LM activations from trained projections at 2K-128K contexts
(PaperTrace "5 · TestingTime 训练与长上下文" §1.1, §3.1); no weights or text are
available, so Gaussian keys/queries/values of the same shapes stand in for them:

  linear_d16_t256   : 1x1 heads, d=16, T=256, b=16, fp32; k,q,v ~ N(0, 1/d), keys
                      L2-normalised, eta = 0.1 scalar, W0 = 0
  linear_b16_8x12   : 8x12 heads, d=64, T=2048, b=16, bf16; k,q,v ~ N(0,1), keys and
                      queries L2-normalised, eta_t = 0.1*sigmoid(N(0,1)) per token,
                      W0 ~ N(0, 0.02^2)
  linear_b16_1x32   : as above at 1x32 heads, T=32768
  mlp_b16_4x16      : TTT-MLP 64->256->64, 4x16 heads, T=8192, b=16, bf16; only keys
                      L2-normalised, eta = 0.05 scalar, W1, W2 ~ N(0, 0.02^2), zero biases
  linear_b2048_1x16 : 1x16 heads, d=128, T=131072, b=2048, bf16; keys and queries
                      L2-normalised, eta = 1/2048 scalar, W0 ~ N(0, 0.02^2)

Every (batch, head) slice has its own generator, seeded with (seed, b, h), so a
test can rebuild any single slice without drawing the whole tensor.  Draw order
inside a slice: K, Q, V (each T x d, standard normal, fp32), eta noise (T), then
W0 (d x d) or W1 (4d x d), W2 (d x 4d).  Normalisation is done in fp32 over the
head dimension, before rounding to bf16 (round-to-nearest-even).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Iterable, Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    model: str            # "linear" | "mlp"
    B: int
    H: int
    T: int
    d: int
    chunk: int
    io: str               # "f32" | "bf16"
    eta_mode: str         # "scalar" | "token"
    eta_value: float      # scalar eta, or the scale of the per-token sigmoid
    kqv_std: float        # std of the raw Gaussian draws (before normalisation)
    normalize: Tuple[str, ...]  # subset of ("k", "q")
    state_std: float      # std of W0 / W1 / W2 (0 -> zero state)
    hidden_mult: int = 4  # MLP hidden width = hidden_mult * d
    mlp_bias: bool = True

    @property
    def BH(self) -> int:
        return self.B * self.H

    @property
    def hidden(self) -> int:
        return self.hidden_mult * self.d

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "linear_d16_t256": Workload("linear_d16_t256", "linear", 1, 1, 256, 16, 16, "f32",
                                "scalar", 0.1, 1.0 / 4.0, ("k",), 0.0),
    "linear_b16_8x12": Workload("linear_b16_8x12", "linear", 8, 12, 2048, 64, 16, "bf16",
                                "token", 0.1, 1.0, ("k", "q"), 0.02),
    "linear_b16_1x32": Workload("linear_b16_1x32", "linear", 1, 32, 32768, 64, 16, "bf16",
                                "token", 0.1, 1.0, ("k", "q"), 0.02),
    "mlp_b16_4x16": Workload("mlp_b16_4x16", "mlp", 4, 16, 8192, 64, 16, "bf16",
                             "scalar", 0.05, 1.0, ("k",), 0.02),
    "linear_b2048_1x16": Workload("linear_b2048_1x16", "linear", 1, 16, 131072, 128, 2048,
                                  "bf16", "scalar", 1.0 / 2048.0, 1.0, ("k", "q"), 0.02),
}

# seed of each named workload (index in the list of five above)
WORKLOAD_SEEDS = {name: i for i, name in enumerate(WORKLOADS)}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value (ties to even), returned as fp32 holding it exactly."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _l2_normalize(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32), dtype=np.float32)
    return (x / n).astype(np.float32)


def make_slice(wl: Workload, seed: int, b: int, h: int) -> Dict[str, np.ndarray]:
    """One (batch, head) slice.  Arrays are fp32 holding values exact in `wl.io`
    (K, Q, V) and fp32 (eta, state)."""
    rng = np.random.default_rng([int(seed), int(b), int(h)])
    T, d = wl.T, wl.d
    raw = {}
    for name in ("K", "Q", "V"):
        raw[name] = rng.standard_normal((T, d), dtype=np.float32) * np.float32(wl.kqv_std)
    noise = rng.standard_normal(T, dtype=np.float32)
    if "k" in wl.normalize:
        raw["K"] = _l2_normalize(raw["K"])
    if "q" in wl.normalize:
        raw["Q"] = _l2_normalize(raw["Q"])
    out = {}
    for name in ("K", "Q", "V"):
        out[name] = round_to_bf16(raw[name]) if wl.io == "bf16" else raw[name].astype(np.float32)
    if wl.eta_mode == "token":
        sig = 1.0 / (1.0 + np.exp(-noise.astype(np.float64)))
        out["eta"] = (wl.eta_value * sig).astype(np.float32)
    else:
        out["eta"] = None
    if wl.model == "linear":
        W0 = rng.standard_normal((d, d), dtype=np.float32) * np.float32(wl.state_std)
        out["W0"] = W0.astype(np.float32)
    else:
        hd = wl.hidden
        out["W1"] = (rng.standard_normal((hd, d), dtype=np.float32)
                     * np.float32(wl.state_std)).astype(np.float32)
        out["W2"] = (rng.standard_normal((d, hd), dtype=np.float32)
                     * np.float32(wl.state_std)).astype(np.float32)
        out["b1"] = np.zeros(hd, np.float32) if wl.mlp_bias else None
        out["b2"] = np.zeros(d, np.float32) if wl.mlp_bias else None
    return out


def make_inputs(wl: Workload, seed: int,
                slices: Optional[Iterable[Tuple[int, int]]] = None) -> Dict[str, np.ndarray]:
    """Stack slices into [n, T, d] / [n, T] / [n, ...] arrays.

    `slices` is a list of (b, h); None means every slice in (b, h) order, which is
    the [B, H, ...] layout flattened to [B*H, ...]."""
    if slices is None:
        slices = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    slices = list(slices)
    parts = [make_slice(wl, seed, b, h) for (b, h) in slices]
    out: Dict[str, np.ndarray] = {}
    for key in parts[0]:
        if parts[0][key] is None:
            out[key] = None
        else:
            out[key] = np.stack([p[key] for p in parts])
    out["eta_scalar"] = float(np.float32(wl.eta_value)) if wl.eta_mode == "scalar" else 0.0
    out["slices"] = slices
    return out


def workload(name: str, **overrides) -> Workload:
    wl = WORKLOADS[name]
    return wl.with_(**overrides) if overrides else wl
