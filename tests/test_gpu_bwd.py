"""GPU parity of ttt_linear_bwd, the backward pass of the TTT-Linear scan, against
the oracle's fp64 vector-Jacobian product (element by element).

The cotangents dZ (in the I/O type) and dW_T (fp32) are seeded Gaussians.
Tolerance: max relative error per (batch, head) slice, max|gpu - oracle| /
max|oracle|, for each of dK, dQ, dV, deta and dW0: 1e-4 with fp32 I/O, 2e-2 with
bf16 I/O (dK, dQ, dV are then rounded to bf16)."""
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
                      eta_value=0.1 if per_token else 0.07)


def cotangents(wl, seed, with_dWT=True):
    rng = np.random.default_rng([seed, 77])
    dZ = rng.standard_normal((wl.BH, wl.T, wl.d), dtype=np.float32)
    if wl.io == "bf16":
        dZ = inputs.round_to_bf16(dZ)
    dWT = rng.standard_normal((wl.BH, wl.d, wl.d), dtype=np.float32) if with_dWT else None
    return dZ, dWT


def check_bwd(wl, seed, dev, with_dWT=True, slices=None, want_deta=True):
    import torch
    x = inputs.make_inputs(wl, seed)
    dZ, dWT = cotangents(wl, seed, with_dWT)
    say("case", wl, "seed", seed, "dW_T", with_dWT)
    a = device_inputs(wl, x, dev)
    io = torch.bfloat16 if wl.io == "bf16" else torch.float32
    B, H, T, d = wl.B, wl.H, wl.T, wl.d
    dZ_d = torch.from_numpy(dZ).to(dev).reshape(B, H, T, d).to(io).contiguous()
    dWT_d = None if dWT is None else torch.from_numpy(dWT).to(dev).reshape(B, H, d, d)
    dK, dQ, dV, deta, dW0 = ttt.linear_bwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], dZ_d,
                                           wl.chunk, eta_scalar=x["eta_scalar"], dW_T=dWT_d,
                                           want_deta=want_deta)
    torch.cuda.synchronize()
    idx = np.arange(wl.BH) if slices is None else np.asarray(slices)
    xo = take(x, idx)
    ref = oracle.linear_bwd(xo["K"], xo["Q"], xo["V"], xo["eta"], xo["eta_scalar"], xo["W0"],
                            wl.chunk, dZ[idx], None if dWT is None else dWT[idx])
    got = [host(dK, wl.BH), host(dQ, wl.BH), host(dV, wl.BH),
           None if deta is None else deta.cpu().numpy().reshape(wl.BH, T),
           host(dW0, wl.BH)]
    errs = {}
    for name, g, r in zip(("dK", "dQ", "dV", "deta", "dW0"), got, ref):
        if g is None:
            continue
        errs[name] = rel_err(g[idx], r)
    say("  max rel err " + "  ".join("%s %.3e" % kv for kv in errs.items()))
    tol = TOL[wl.io]
    assert all(e < tol for e in errs.values()), errs
    return errs


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("chunk", [1, 5, 16, 40])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_small_shapes(dev, d, chunk, io):
    wl = case(d, chunk, io, per_token=(chunk % 2 == 0), T=77)
    check_bwd(wl, 401, dev)


@pytest.mark.parametrize("T,chunk", [(1, 16), (16, 16), (17, 16), (33, 64), (100, 32)])
def test_edge_lengths(dev, T, chunk):
    wl = case(64, chunk, "bf16", per_token=True, T=T)
    check_bwd(wl, 402, dev)


def test_without_state_cotangent_or_deta(dev):
    wl = case(32, 16, "f32", per_token=True, T=50)
    check_bwd(wl, 403, dev, with_dWT=False, want_deta=False)


def test_many_slices(dev):
    wl = case(64, 16, "bf16", per_token=True, T=64, B=8, H=12)
    check_bwd(wl, 404, dev)


@pytest.mark.parametrize("name,slices", [("linear_b16_8x12", [0, 47, 95]),
                                         ("linear_b16_1x32", [5])])
def test_full_size_sampled(dev, name, slices):
    """The full-size workloads, all slices computed on the GPU, sampled slices
    checked against the oracle."""
    wl = inputs.WORKLOADS[name]
    check_bwd(wl, inputs.WORKLOAD_SEEDS[name], dev, slices=slices)


# Segments along T: with chunks of at most 16 tokens and fewer (sequence, row
# block) units than compute units, each sequence is cut into up to 8 segments (at
# least 64 sub-tiles each, at most four waves of units per compute unit) whose units
# recompute the forward up to their end and carry the state's cotangent back from
# the sequence end; these shapes take 2 to 8 segments.
@pytest.mark.parametrize("d,io,chunk,H,T", [
    (64, "bf16", 16, 20, 3072),    # 80 units: 3 segments (192 sub-tiles)
    (64, "bf16", 16, 20, 3001),    # ragged last sub-tile: 2 segments
    (128, "bf16", 16, 8, 4096),    # 64 units: 4 segments
    (32, "f32", 16, 10, 2048),     # 20 units: 2 segments
    (64, "bf16", 8, 12, 2048),     # chunks of 8 tokens: 256 sub-tiles, 4 segments
    (64, "bf16", 16, 4, 8192),     # 16 units: 8 segments
    (16, "f32", 16, 40, 2048),     # 40 one-wave units: 2 segments
    (128, "f32", 16, 6, 4096),     # 48 two-wave units: 4 segments
    (16, "bf16", 16, 24, 3000),    # 24 one-wave units: 2 segments, ragged
    (32, "bf16", 16, 30, 4096),    # 60 two-wave units: 4 segments
])
def test_segments(dev, d, io, chunk, H, T):
    wl = case(d, chunk, io, per_token=True, T=T, B=1, H=H)
    check_bwd(wl, 421, dev, slices=[0, H - 1])


@pytest.mark.parametrize("io,T", [("bf16", 4096), ("bf16", 5000), ("f32", 4096)])
def test_segments_bitwise(dev, io, T):
    """The segment count does not change a bit of the result: the first 20 heads of
    a 40-head call (160 row-block units: three segments with bf16 I/O, one with
    fp32 I/O) against a 20-head call of the same inputs (80 units: four segments
    with bf16 I/O, three with fp32 I/O).  (Five split points of one shape, and one
    segment against two and four, gave the same bits on the GPU too.)"""
    import torch
    wl = case(64, 16, io, True, T, B=1, H=40)
    x = inputs.make_inputs(wl, 422)
    dZ, dWT = cotangents(wl, 422)
    a = device_inputs(wl, x, dev)
    t = torch.bfloat16 if io == "bf16" else torch.float32
    dZ_d = torch.from_numpy(dZ).to(dev).reshape(1, 40, T, 64).to(t).contiguous()
    dWT_d = torch.from_numpy(dWT).to(dev).reshape(1, 40, 64, 64)
    full = ttt.linear_bwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], dZ_d, wl.chunk,
                          eta_scalar=x["eta_scalar"], dW_T=dWT_d)
    h = lambda u: u[:, :20].contiguous()   # noqa: E731
    part = ttt.linear_bwd(h(a["K"]), h(a["Q"]), h(a["V"]), h(a["eta"]), h(a["W0"]), h(dZ_d),
                          wl.chunk, eta_scalar=x["eta_scalar"], dW_T=h(dWT_d))
    torch.cuda.synchronize()
    for name, u, v in zip(("dK", "dQ", "dV", "deta", "dW0"), full, part):
        assert torch.equal(h(u), v), name


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_bitwise_deterministic(dev, io):
    """dK, dQ and deta are sums over the state's row blocks: they come out the same
    bits on every call (planes added in a fixed order, no atomics)."""
    import torch
    wl = case(64, 16, io, True, 300, B=2, H=5)
    x = inputs.make_inputs(wl, 419)
    dZ, dWT = cotangents(wl, 419)
    a = device_inputs(wl, x, dev)
    t = torch.bfloat16 if io == "bf16" else torch.float32
    dZ_d = torch.from_numpy(dZ).to(dev).reshape(wl.B, wl.H, wl.T, wl.d).to(t).contiguous()
    dWT_d = torch.from_numpy(dWT).to(dev).reshape(wl.B, wl.H, wl.d, wl.d)
    runs = [ttt.linear_bwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], dZ_d, wl.chunk,
                           eta_scalar=x["eta_scalar"], dW_T=dWT_d) for _ in range(3)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        assert all(torch.equal(u, v) for u, v in zip(runs[0], r))
