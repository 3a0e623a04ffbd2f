"""GPU parity of ttt_linear_fwd_momentum (TTT-Linear with a momentum state,
chunk-start reads) against the fp64 oracle.

Tolerance: max relative error per (batch, head) slice for Z, the final state and
the final momentum, 1e-4 with fp32 I/O and 2e-2 with bf16 I/O."""
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


def case(d, chunk, io, per_token, T, B=2, H=3, eta=None):
    base = inputs.workload("linear_b16_8x12")
    return base.with_(B=B, H=H, T=T, d=d, chunk=chunk, io=io,
                      eta_mode="token" if per_token else "scalar",
                      eta_value=eta if eta is not None else (0.1 if per_token else 0.07))


def check(wl, seed, dev, beta, with_m0=True, plan=ttt.PLAN_AUTO, expect_plan=None, slices=None):
    import torch
    io_code = ttt.DTYPE_BF16 if wl.io == "bf16" else ttt.DTYPE_F32
    p = ttt.linear_select_plan(wl.B, wl.H, wl.T, wl.d, wl.chunk, io_code, plan,
                               ttt.READ_CHUNK_START)
    if expect_plan is not None:
        assert p == expect_plan
    x = inputs.make_inputs(wl, seed)
    rng = np.random.default_rng([seed, 66])
    M0 = (0.01 * rng.standard_normal((wl.BH, wl.d, wl.d))).astype(np.float32) if with_m0 else None
    say("case", wl, "seed", seed, "beta", beta, "plan", ttt.plan_name(p))
    a = device_inputs(wl, x, dev)
    M0d = None if M0 is None else torch.from_numpy(M0).to(dev).reshape(wl.B, wl.H, wl.d, wl.d)
    Z, W, Mo = ttt.linear_fwd_momentum(a["K"], a["Q"], a["V"], a["eta"], a["W0"], M0d, beta,
                                       wl.chunk, eta_scalar=x["eta_scalar"], plan=plan)
    torch.cuda.synchronize()
    idx = np.arange(wl.BH) if slices is None else np.asarray(slices)
    xo = take(x, idx)
    Zo, Wo, Mref = oracle.linear_momentum(xo["K"], xo["Q"], xo["V"], xo["eta"], xo["eta_scalar"],
                                          xo["W0"], None if M0 is None else M0[idx], beta,
                                          wl.chunk)
    ez = rel_err(host(Z, wl.BH)[idx], Zo)
    ew = rel_err(host(W, wl.BH)[idx], Wo)
    em = rel_err(host(Mo, wl.BH)[idx], Mref)
    say("  max rel err Z %.3e  W %.3e  M %.3e" % (ez, ew, em))
    tol = TOL[wl.io]
    assert ez < tol and ew < tol and em < tol, (ez, ew, em)


@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("chunk", [1, 16, 40])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_generic(dev, d, chunk, io):
    check(case(d, chunk, io, per_token=(chunk != 1), T=77), 801, dev, beta=0.9,
          expect_plan=ttt.PLAN_GENERIC)


@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_generic_betas(dev, beta):
    check(case(32, 8, "f32", per_token=True, T=50), 802, dev, beta=beta, with_m0=(beta > 0))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T,chunk,per_token", [(512, 256, False), (300, 128, True),
                                               (1000, 160, True)])
def test_large_chunks(dev, d, T, chunk, per_token):
    wl = case(d, chunk, "bf16", per_token=per_token, T=T, eta=1.0 / chunk if not per_token else 0.02)
    check(wl, 803, dev, beta=0.8, expect_plan=ttt.PLAN_BIGCHUNK)


def test_full_size_large_chunk_sampled(dev):
    wl = inputs.WORKLOADS["linear_b2048_1x16"]
    check(wl, inputs.WORKLOAD_SEEDS[wl.name], dev, beta=0.9, slices=[3],
          expect_plan=ttt.PLAN_BIGCHUNK)
