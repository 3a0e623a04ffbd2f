"""GPU parity of ttt_linear_ln_fwd (TTT-Linear with the inner bias as state and
LayerNorm + residual inside f, or the bias alone) against the fp64 oracle.

Tolerance: max relative error per (batch, head) slice for Z, W and b, 1e-4 with
fp32 I/O and 2e-2 with bf16 I/O."""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, device_inputs, host, rel_err, say, take
from test_sequence_layers_ttt_amd import inputs, ttt

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ttt.lib()
    return torch.device("cuda:0")


def case(d, chunk, io, per_token, T, B=2, H=3):
    base = inputs.workload("linear_b16_8x12")
    return base.with_(B=B, H=H, T=T, d=d, chunk=chunk, io=io,
                      eta_mode="token" if per_token else "scalar",
                      eta_value=0.1 if per_token else 0.05, state_std=0.1)


def ln_params(wl, seed, with_ln):
    rng = np.random.default_rng([seed, 55])
    b0 = (0.1 * rng.standard_normal((wl.BH, wl.d))).astype(np.float32)
    if not with_ln:
        return b0, None, None
    lnw = (1.0 + 0.1 * rng.standard_normal((wl.H, wl.d))).astype(np.float32)
    lnb = (0.1 * rng.standard_normal((wl.H, wl.d))).astype(np.float32)
    return b0, lnw, lnb


def check(wl, seed, dev, with_ln=True, eps=1e-5, slices=None):
    import torch
    x = inputs.make_inputs(wl, seed)
    b0, lnw, lnb = ln_params(wl, seed, with_ln)
    say("case", wl, "seed", seed, "ln", with_ln)
    a = device_inputs(wl, x, dev)
    t = lambda arr: None if arr is None else torch.from_numpy(arr).to(dev)
    B, H, d = wl.B, wl.H, wl.d
    Z, W, b = ttt.linear_ln_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"],
                                t(b0).reshape(B, H, d), t(lnw), t(lnb), wl.chunk, eps=eps,
                                eta_scalar=x["eta_scalar"])
    torch.cuda.synchronize()
    idx = np.arange(wl.BH) if slices is None else np.asarray(slices)
    xo = take(x, idx)
    heads = idx % H
    Zo, Wo, bo = oracle.linear_ln(xo["K"], xo["Q"], xo["V"], xo["eta"], xo["eta_scalar"],
                                  xo["W0"], b0[idx], None if lnw is None else lnw[heads],
                                  None if lnb is None else lnb[heads], eps, wl.chunk)
    ez = rel_err(host(Z, wl.BH)[idx], Zo)
    ew = rel_err(host(W, wl.BH)[idx], Wo)
    eb = rel_err(b.cpu().numpy().reshape(wl.BH, d)[idx], bo)
    say("  max rel err Z %.3e  W %.3e  b %.3e" % (ez, ew, eb))
    tol = TOL[wl.io]
    assert ez < tol and ew < tol and eb < tol, (ez, ew, eb)


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("chunk", [1, 5, 16, 40])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_ln_residual(dev, d, chunk, io):
    check(case(d, chunk, io, per_token=(chunk != 5), T=77), 701, dev)


@pytest.mark.parametrize("d,chunk,io", [(16, 16, "f32"), (64, 3, "f32"), (128, 16, "bf16"),
                                        (32, 40, "bf16")])
def test_bias_only(dev, d, chunk, io):
    check(case(d, chunk, io, per_token=True, T=61), 702, dev, with_ln=False)


@pytest.mark.parametrize("T", [1, 16, 17])
def test_short_sequences(dev, T):
    check(case(64, 16, "bf16", per_token=True, T=T), 703, dev)


def test_full_size_sampled(dev):
    """8 x 12 heads, d = 64, T = 2048, chunk 16, bf16: every slice on the GPU,
    three checked against the oracle."""
    wl = inputs.WORKLOADS["linear_b16_8x12"].with_(state_std=0.1)
    check(wl, inputs.WORKLOAD_SEEDS["linear_b16_8x12"], dev, slices=[0, 50, 95])
