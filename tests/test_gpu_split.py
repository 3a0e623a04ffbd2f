"""GPU parity of the segmented plan (chunk-16 TTT-Linear at d = 64 with few
(batch, head) slices: each sequence cut into S ~ 256 / slices + 1 segments;
segment 0 scans while segments 1 .. S-2 form their affine maps, a combine gives
every segment its start state, and the segments after the first scan again from
it) against the fp64 oracle, element by element: max relative error per slice
below 2e-2 (bf16)."""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, rel_err, run_linear, say, take
from test_sequence_layers_ttt_amd import inputs, ttt

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ttt.lib()
    return torch.device("cuda:0")


def case(T, B=1, H=3, per_token=True, seed=151):
    base = inputs.workload("linear_b16_8x12")
    return base.with_(B=B, H=H, T=T, d=64, chunk=16, io="bf16",
                      eta_mode="token" if per_token else "scalar",
                      eta_value=0.1 if per_token else 0.07), seed


def check(wl, seed, dev, plan=ttt.PLAN_SPLIT, slices=None, eta_offset=0):
    assert ttt.linear_select_plan(wl.B, wl.H, wl.T, wl.d, wl.chunk, 1, plan) == ttt.PLAN_SPLIT
    x = inputs.make_inputs(wl, seed)
    say("case", wl, "seed", seed)
    Z, W = run_linear(wl, x, dev, plan=plan, eta_offset=eta_offset)
    idx = np.arange(wl.BH) if slices is None else np.asarray(slices)
    xo = take(x, idx)
    Zo, Wo = oracle.linear(xo["K"], xo["Q"], xo["V"], xo["eta"], xo["eta_scalar"], xo["W0"],
                           wl.chunk)
    ez, ew = rel_err(Z[idx], Zo), rel_err(W[idx], Wo)
    say("  max rel err Z %.3e  W %.3e" % (ez, ew))
    assert ez < TOL["bf16"] and ew < TOL["bf16"], (ez, ew)


# lengths: the shortest taken, segment lengths that are and are not multiples of
# the LDS ring (16 chunks), and lengths that are not multiples of 16 (the last
# segment's ragged form; 2052 and 3004 with 16-byte eta loads)
@pytest.mark.parametrize("T", [2048, 2064, 3008, 4096, 5120, 2049, 2052, 3001, 3004, 5117])
@pytest.mark.parametrize("per_token", [True, False])
def test_lengths(dev, T, per_token):
    wl, seed = case(T, per_token=per_token)
    check(wl, seed, dev)


# slice counts up to the 64 the plan takes (64 down to 5 segments each)
@pytest.mark.parametrize("B,H", [(1, 1), (1, 7), (2, 9), (4, 8), (1, 33), (5, 10), (2, 32)])
def test_slice_counts(dev, B, H):
    wl, seed = case(2080, B=B, H=H)
    check(wl, seed, dev)


# 33 to 64 slices, long and ragged, where AUTO takes the plan (T >= 4096); sampled
@pytest.mark.parametrize("B,H,T", [(1, 40, 4096), (2, 32, 8195), (1, 48, 6000)])
def test_many_slices_auto(dev, B, H, T):
    wl, seed = case(T, B=B, H=H, seed=159)
    assert ttt.linear_select_plan(wl.B, wl.H, wl.T, wl.d, wl.chunk, 1) == ttt.PLAN_SPLIT
    check(wl, seed, dev, plan=ttt.PLAN_AUTO, slices=[0, 17, wl.BH - 1])



# long chains of segment maps: one slice in 32 segments (30 combine steps), two in
# 16, sixteen in 8
@pytest.mark.parametrize("B,H,T", [(1, 1, 16384), (1, 2, 8192), (2, 8, 4096)])
def test_many_segments(dev, B, H, T):
    wl, seed = case(T, B=B, H=H, seed=157)
    check(wl, seed, dev, slices=[0, wl.BH - 1])


def test_unaligned_eta(dev):
    wl, seed = case(2048, B=2, H=2)
    check(wl, seed, dev, eta_offset=1)


def test_unaligned_eta_ragged(dev):
    wl, seed = case(2060, B=2, H=2, seed=158)
    check(wl, seed, dev, eta_offset=1)


def test_linear_b16_1x32_ragged(dev):
    """The headline shape one token short of a whole chunk: 1x32 heads at
    T = 32767 on the segmented plan, sampled slices against the oracle."""
    wl = inputs.WORKLOADS["linear_b16_1x32"].with_(T=32767)
    check(wl, inputs.WORKLOAD_SEEDS["linear_b16_1x32"], dev, plan=ttt.PLAN_AUTO,
          slices=[0, 13, 31])


def test_auto_picks_split_at_1x32_heads(dev):
    wl = inputs.WORKLOADS["linear_b16_1x32"]
    assert ttt.linear_select_plan(wl.B, wl.H, wl.T, wl.d, wl.chunk, 1) == ttt.PLAN_SPLIT
    assert ttt.linear_select_plan(wl.B, wl.H, wl.T - 1, wl.d, wl.chunk, 1) == ttt.PLAN_SPLIT
    wl2 = inputs.WORKLOADS["linear_b16_8x12"]
    assert ttt.linear_select_plan(wl2.B, wl2.H, wl2.T, wl2.d, wl2.chunk, 1) == ttt.PLAN_MFMA


def test_linear_b16_1x32_full_mfma_plan(dev):
    """The single-segment chunk kernel stays available under the MFMA plan."""
    wl = inputs.WORKLOADS["linear_b16_1x32"]
    x = inputs.make_inputs(wl, inputs.WORKLOAD_SEEDS[wl.name])
    Z, W = run_linear(wl, x, dev, plan=ttt.PLAN_MFMA)
    idx = np.array([0, 17, 31])
    xo = take(x, idx)
    Zo, Wo = oracle.linear(xo["K"], xo["Q"], xo["V"], xo["eta"], xo["eta_scalar"], xo["W0"],
                           wl.chunk)
    assert rel_err(Z[idx], Zo) < TOL["bf16"] and rel_err(W[idx], Wo) < TOL["bf16"]


def test_state_may_alias_initial_state(dev):
    import torch
    from gpu_helpers import device_inputs
    wl, seed = case(2304, B=2, H=3)
    x = inputs.make_inputs(wl, seed)
    a = device_inputs(wl, x, dev)
    Z1, W1 = ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], 16, plan=ttt.PLAN_SPLIT)
    W = a["W0"].clone()
    Z2, W2 = ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], W, 16, W_out=W,
                            plan=ttt.PLAN_SPLIT)
    torch.cuda.synchronize()
    assert torch.equal(W1, W2) and torch.equal(Z1, Z2)


def test_bitwise_deterministic(dev):
    import torch
    from gpu_helpers import device_inputs
    wl, seed = case(2048, B=3, H=4)
    x = inputs.make_inputs(wl, seed)
    a = device_inputs(wl, x, dev)
    r1 = ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], 16, plan=ttt.PLAN_SPLIT)
    r2 = ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], 16, plan=ttt.PLAN_SPLIT)
    torch.cuda.synchronize()
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])


def test_nan_stays_in_its_slice(dev):
    import torch
    from gpu_helpers import device_inputs
    wl, seed = case(2048, B=2, H=3)
    x = inputs.make_inputs(wl, seed)
    a = device_inputs(wl, x, dev)
    a["V"][1, 2, 1900, 5] = float("nan")    # in the last segment
    a["K"][0, 1, 100, 7] = float("nan")     # in the first segment
    Z, W = ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], 16, plan=ttt.PLAN_SPLIT)
    torch.cuda.synchronize()
    bad = torch.isnan(Z.float()).flatten(2).any(-1) | torch.isnan(W).flatten(2).any(-1)
    assert bad[1, 2] and bad[0, 1] and int(bad.sum()) == 2
