"""GPU parity of the chunk-start read order (ttt_linear_fwd_ex with
TTT_READ_CHUNK_START: every token of a chunk reads with the chunk-start state,
then the state moves as usual) against the fp64 oracle.

Tolerance: max relative error per (batch, head) slice, 1e-4 for fp32 I/O and
2e-2 for bf16 I/O.  The final state must equal, bit for bit, the same plan's
inclusive-read result: the read order does not touch the state update."""
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


def check(wl, seed, dev, plan, slices=None, expect_plan=None):
    import torch
    io_code = ttt.DTYPE_BF16 if wl.io == "bf16" else ttt.DTYPE_F32
    p = ttt.linear_select_plan(wl.B, wl.H, wl.T, wl.d, wl.chunk, io_code, plan,
                               ttt.READ_CHUNK_START)
    assert p > 0, p
    if expect_plan is not None:
        assert p == expect_plan
    x = inputs.make_inputs(wl, seed)
    say("case", wl, "seed", seed, "plan", ttt.plan_name(p))
    a = device_inputs(wl, x, dev)
    Zs, Ws = ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], wl.chunk,
                            eta_scalar=x["eta_scalar"], plan=p, read_mode=ttt.READ_CHUNK_START)
    _, Wi = ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], wl.chunk,
                           eta_scalar=x["eta_scalar"], plan=p)
    torch.cuda.synchronize()
    assert torch.equal(Ws, Wi)
    idx = np.arange(wl.BH) if slices is None else np.asarray(slices)
    xo = take(x, idx)
    Zo, Wo = oracle.linear(xo["K"], xo["Q"], xo["V"], xo["eta"], xo["eta_scalar"], xo["W0"],
                           wl.chunk, read_start=True)
    ez = rel_err(host(Zs, wl.BH)[idx], Zo)
    ew = rel_err(host(Ws, wl.BH)[idx], Wo)
    say("  max rel err Z %.3e  W %.3e" % (ez, ew))
    tol = TOL[wl.io]
    assert ez < tol and ew < tol, (ez, ew)


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("chunk", [1, 5, 16, 40])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_generic(dev, d, chunk, io):
    wl = case(d, chunk, io, per_token=(chunk % 2 == 0), T=77)
    check(wl, 501, dev, ttt.PLAN_AUTO, expect_plan=ttt.PLAN_GENERIC)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T,chunk,per_token", [(512, 256, False), (300, 128, True),
                                               (1000, 160, True), (640, 128, True)])
def test_large_chunks(dev, d, T, chunk, per_token):
    wl = case(d, chunk, "bf16", per_token=per_token, T=T, eta=1.0 / chunk if not per_token else 0.02)
    check(wl, 502, dev, ttt.PLAN_AUTO, expect_plan=ttt.PLAN_BIGCHUNK)


def test_large_chunks_on_the_generic_plan(dev):
    wl = case(64, 256, "bf16", per_token=True, T=600, eta=0.02)
    check(wl, 503, dev, ttt.PLAN_GENERIC)


def test_full_size_large_chunk_sampled(dev):
    """1 x 16 heads, d = 128, T = 131072, chunk 2048: every slice on the GPU, one
    checked against the oracle."""
    wl = inputs.WORKLOADS["linear_b2048_1x16"]
    check(wl, inputs.WORKLOAD_SEEDS[wl.name], dev, ttt.PLAN_AUTO, slices=[9],
          expect_plan=ttt.PLAN_BIGCHUNK)
