"""GPU parity of ttt_linear_fwd against the fp64 oracle (element by element).

Tolerance: max relative error per (batch, head) slice, max|gpu - oracle| /
max|oracle|, 1e-4 for fp32 I/O and 2e-2 for bf16 I/O with fp32 state."""
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


def small(d, chunk, io, per_token, T=77, B=2, H=3, seed=101):
    base = inputs.workload("linear_b16_8x12")
    return base.with_(B=B, H=H, T=T, d=d, chunk=chunk, io=io,
                      eta_mode="token" if per_token else "scalar",
                      eta_value=0.1 if per_token else 0.07), seed


def check_linear(wl, seed, dev, plan, slices=None, eta_offset=0):
    x = inputs.make_inputs(wl, seed)
    p = ttt.linear_select_plan(wl.B, wl.H, wl.T, wl.d, wl.chunk, 1 if wl.io == "bf16" else 0, plan)
    if p < 0:
        pytest.skip("plan %d does not run this shape" % plan)
    say("case", wl, "seed", seed, "plan", ttt.plan_name(p))
    Z, W = run_linear(wl, x, dev, plan=plan, eta_offset=eta_offset)
    idx = np.arange(wl.BH) if slices is None else np.asarray(slices)
    xo = take(x, idx)
    Zo, Wo = oracle.linear(xo["K"], xo["Q"], xo["V"], xo["eta"], xo["eta_scalar"], xo["W0"],
                           wl.chunk)
    ez, ew = rel_err(Z[idx], Zo), rel_err(W[idx], Wo)
    say("  max rel err Z %.3e  W %.3e" % (ez, ew))
    tol = TOL[wl.io]
    assert ez < tol and ew < tol, (ez, ew)
    return ez, ew


@pytest.mark.parametrize("plan", [ttt.PLAN_GENERIC, ttt.PLAN_AUTO])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("chunk", [1, 3, 16, 40])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_small_shapes(dev, plan, d, chunk, io):
    wl, seed = small(d, chunk, io, per_token=(chunk % 2 == 0))
    check_linear(wl, seed, dev, plan)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T,chunk", [(1, 16), (5, 16), (16, 16), (17, 16), (300, 64), (130, 128)])
def test_edge_lengths(dev, T, chunk, d):
    wl, seed = small(d, chunk, "bf16", per_token=True, T=T)
    check_linear(wl, seed, dev, ttt.PLAN_AUTO)


# fp32 I/O on the fp32 matrix cores: lengths and chunks that leave ragged
# sub-tiles, chunks of one token, chunks longer than T, many slices
@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("T,chunk,per_token", [(1, 16, True), (5, 16, False), (16, 16, True),
                                               (17, 16, True), (33, 1, True), (70, 24, False),
                                               (300, 64, True), (40, 100, True)])
def test_f32_matrix_core_lengths(dev, T, chunk, per_token, d):
    wl, seed = small(d, chunk, "f32", per_token=per_token, T=T)
    assert ttt.linear_select_plan(wl.B, wl.H, wl.T, d, chunk, 0) == ttt.PLAN_MFMA
    check_linear(wl, seed, dev, ttt.PLAN_MFMA)


def test_f32_matrix_core_many_slices(dev):
    wl, seed = small(32, 16, "f32", per_token=True, T=50, B=9, H=15, seed=109)
    check_linear(wl, seed, dev, ttt.PLAN_MFMA)


# Many (batch, head) slices: shapes past the 256-unit threshold (units = B*H*d/16)
# where chunk-16 heads share their K/Q tiles per workgroup, and the two-block
# single-wave kernel for the shapes that cannot.  Up to 128 heads the shared-tile
# kernel splits a head over two workgroups (two waves each at d = 64, four at
# d = 128; the grid rounded up to whole rounds of the 8 XCDs), and keeps one
# workgroup of d/16 waves per head past that.
@pytest.mark.parametrize("d,B,H,T,chunk,per_token", [
    (64, 9, 8, 100, 16, True),     # shared-tile kernel, ragged last chunk, two workgroups
    (64, 5, 16, 64, 16, False),    # shared-tile kernel, scalar eta, two workgroups
    (64, 7, 11, 80, 16, True),     # 77 heads: two workgroups, grid rounded up
    (64, 9, 16, 64, 16, True),     # 144 heads: one workgroup, 16-byte eta loads
    (128, 3, 11, 48, 16, True),    # d = 128, 33 heads: two workgroups per head
    (128, 5, 14, 48, 16, True),    # d = 128, 70 heads: two workgroups per head
    (128, 9, 15, 33, 16, False),   # d = 128, 135 heads: one, ragged, scalar eta
    (32, 9, 15, 40, 16, True),     # two 16-row blocks per wave at d = 32
    (64, 2, 40, 56, 8, True),      # two blocks per wave, chunk 8
    (64, 5, 13, 48, 16, True),     # 65 heads: the smallest head count past 256 units
    (64, 8, 16, 64, 16, False),    # 128 heads: the largest with two workgroups per head
    (64, 3, 43, 61, 16, True),     # 129 heads: one workgroup per head, ragged T
])
def test_many_slices(dev, d, B, H, T, chunk, per_token):
    wl, seed = small(d, chunk, "bf16", per_token=per_token, T=T, B=B, H=H, seed=107)
    check_linear(wl, seed, dev, ttt.PLAN_AUTO)


# Per-token eta whose pointer is 4-byte but not 16-byte aligned: every kernel
# family must take its per-element eta loads (T a multiple of 16 otherwise picks
# the 16-byte loads).
@pytest.mark.parametrize("d,B,H,T,chunk", [
    (64, 9, 8, 64, 16),       # shared-tile kernel
    (64, 2, 3, 64, 16),       # single-wave chunk kernel
    (32, 9, 15, 32, 16),      # two blocks per wave
    (64, 1, 3, 256, 128),     # large-chunk plan
    (64, 2, 2, 96, 32),       # multi-sub-tile chunks
])
def test_unaligned_eta(dev, d, B, H, T, chunk):
    wl, seed = small(d, chunk, "bf16", per_token=True, T=T, B=B, H=H, seed=113)
    check_linear(wl, seed, dev, ttt.PLAN_AUTO, eta_offset=1)


def test_linear_d16_t256_fp32(dev):
    wl = inputs.WORKLOADS["linear_d16_t256"]
    check_linear(wl, inputs.WORKLOAD_SEEDS[wl.name], dev, ttt.PLAN_AUTO)


def test_linear_b16_8x12_full(dev):
    wl = inputs.WORKLOADS["linear_b16_8x12"]
    check_linear(wl, inputs.WORKLOAD_SEEDS[wl.name], dev, ttt.PLAN_AUTO)


def test_linear_b16_1x32_full(dev):
    wl = inputs.WORKLOADS["linear_b16_1x32"]
    check_linear(wl, inputs.WORKLOAD_SEEDS[wl.name], dev, ttt.PLAN_AUTO)   # all 32 slices


def test_linear_b2048_1x16_full(dev):
    wl = inputs.WORKLOADS["linear_b2048_1x16"]
    check_linear(wl, inputs.WORKLOAD_SEEDS[wl.name], dev, ttt.PLAN_AUTO)   # all 16 slices


def test_scope_table_entry_point(dev):
    """ttt_linear_fwd called through ctypes with exactly the boundary's argument
    list (no plan, no read order), against the oracle."""
    import ctypes
    import torch
    from gpu_helpers import device_inputs, host
    wl, seed = small(64, 16, "bf16", per_token=True, T=200, B=2, H=5)
    x = inputs.make_inputs(wl, seed)
    a = device_inputs(wl, x, dev)
    Z = torch.empty_like(a["K"])
    W = torch.empty_like(a["W0"])
    n = ttt.lib().ttt_linear_workspace_bytes(wl.B, wl.H, wl.T, wl.d, wl.chunk)
    assert n == 0
    rc = ttt.lib().ttt_linear_fwd(
        a["K"].data_ptr(), a["Q"].data_ptr(), a["V"].data_ptr(), a["eta"].data_ptr(),
        ctypes.c_float(0.0), a["W0"].data_ptr(), Z.data_ptr(), W.data_ptr(), wl.B, wl.H, wl.T,
        wl.d, wl.chunk, ttt.DTYPE_BF16, None, 0, torch.cuda.current_stream(dev).cuda_stream)
    assert rc == ttt.OK
    torch.cuda.synchronize()
    Zo, Wo = oracle.linear(x["K"], x["Q"], x["V"], x["eta"], x["eta_scalar"], x["W0"], wl.chunk)
    ez, ew = rel_err(host(Z, wl.BH), Zo), rel_err(host(W, wl.BH), Wo)
    say("  scope-table call: max rel err Z %.3e  W %.3e" % (ez, ew))
    assert ez < TOL["bf16"] and ew < TOL["bf16"]


def test_state_may_alias_initial_state(dev):
    import torch
    from gpu_helpers import device_inputs
    wl, seed = small(64, 16, "bf16", per_token=True)
    x = inputs.make_inputs(wl, seed)
    a = device_inputs(wl, x, dev)
    Z1, W1 = ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], wl.chunk)
    W = a["W0"].clone()
    Z2, W2 = ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], W, wl.chunk, W_out=W)
    torch.cuda.synchronize()
    assert W2.data_ptr() == W.data_ptr()
    assert torch.equal(W1, W2) and torch.equal(Z1, Z2)


def test_bitwise_deterministic_and_stream(dev):
    import torch
    from gpu_helpers import device_inputs
    wl, seed = small(64, 16, "bf16", per_token=True, T=500)
    x = inputs.make_inputs(wl, seed)
    a = device_inputs(wl, x, dev)
    Z1, W1 = ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], wl.chunk)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        Z2, W2 = ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], wl.chunk)
    s.synchronize()
    assert torch.equal(Z1, Z2) and torch.equal(W1, W2)


def test_nan_stays_in_its_slice(dev):
    import torch
    from gpu_helpers import device_inputs
    wl, seed = small(64, 16, "bf16", per_token=True, T=64)
    x = inputs.make_inputs(wl, seed)
    a = device_inputs(wl, x, dev)
    a["V"][1, 2, 10, 5] = float("nan")
    Z, W = ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], wl.chunk)
    torch.cuda.synchronize()
    bad = torch.isnan(Z.float()).flatten(2).any(-1) | torch.isnan(W).flatten(2).any(-1)
    assert bad[1, 2] and int(bad.sum()) == 1


def test_eta_zero_reads_initial_state(dev):
    import torch
    from gpu_helpers import device_inputs
    wl, seed = small(32, 16, "f32", per_token=False, T=40)
    x = inputs.make_inputs(wl, seed)
    a = device_inputs(wl, x, dev)
    Z, W = ttt.linear_fwd(a["K"], a["Q"], a["V"], None, a["W0"], wl.chunk, eta_scalar=0.0)
    torch.cuda.synchronize()
    assert torch.equal(W, a["W0"])
    ref = a["Q"].double().cpu() @ a["W0"].double().cpu().transpose(-1, -2)
    assert float((Z.double().cpu() - ref).abs().max()) < 1e-5


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T,chunk", [(256, 128), (300, 128), (1000, 256), (4096, 2048), (96, 160)])
@pytest.mark.parametrize("per_token", [True, False])
def test_large_chunk_plan(dev, d, T, chunk, per_token):
    """Three-stage large-chunk path (per-chunk Gram products, state chain, per-chunk
    sub-tile pass), including a ragged last chunk and a sequence shorter than a chunk."""
    wl, seed = small(d, chunk, "bf16", per_token=per_token, T=T, B=1, H=3)
    wl = wl.with_(eta_value=(0.1 if per_token else 1.0 / chunk))
    check_linear(wl, seed, dev, ttt.PLAN_BIGCHUNK)
