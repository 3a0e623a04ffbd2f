"""GPU parity of ttt_mlp_fwd against the fp64 oracle (element by element).

Tolerance as for TTT-Linear: max relative error per (batch, head) slice, 1e-4 for
fp32 I/O and 2e-2 for bf16 I/O; each of Z, W1, b1, W2, b2 is checked (biases that
start at zero use a floor of 1e-6 for the denominator)."""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, rel_err, run_mlp, say, take
from test_sequence_layers_ttt_amd import inputs, ttt

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ttt.lib()
    return torch.device("cuda:0")


def check_mlp(wl, seed, dev, plan, slices=None, bias_init=None, eta_offset=0):
    x = inputs.make_inputs(wl, seed)
    if bias_init is not None and wl.mlp_bias:
        rng = np.random.default_rng(seed + 999)
        x["b1"] = (rng.standard_normal(x["b1"].shape) * bias_init).astype(np.float32)
        x["b2"] = (rng.standard_normal(x["b2"].shape) * bias_init).astype(np.float32)
    p = ttt.mlp_select_plan(wl.B, wl.H, wl.T, wl.d, wl.chunk, 1 if wl.io == "bf16" else 0, plan)
    if p < 0:
        pytest.skip("plan %d does not run this shape" % plan)
    say("case", wl, "seed", seed, "plan", ttt.plan_name(p))
    got = run_mlp(wl, x, dev, plan=plan, eta_offset=eta_offset)
    idx = np.arange(wl.BH) if slices is None else np.asarray(slices)
    xo = take(x, idx)
    ref = oracle.mlp(xo["K"], xo["Q"], xo["V"], xo["eta"], xo["eta_scalar"], xo["W1"], xo["b1"],
                     xo["W2"], xo["b2"], wl.chunk)
    errs = {}
    for name, g, r in zip(("Z", "W1", "b1", "W2", "b2"), got, ref):
        if r is None:
            assert g is None
            continue
        errs[name] = rel_err(g[idx], r)
    say("  max rel err", " ".join("%s %.3e" % kv for kv in errs.items()))
    tol = TOL[wl.io]
    assert all(e < tol for e in errs.values()), errs
    return errs


def small(d, chunk, io, per_token, bias=True, T=45, B=1, H=3):
    base = inputs.workload("mlp_b16_4x16")
    return base.with_(B=B, H=H, T=T, d=d, chunk=chunk, io=io, mlp_bias=bias,
                      eta_mode="token" if per_token else "scalar",
                      eta_value=0.1 if per_token else 0.05)


@pytest.mark.parametrize("plan", [ttt.PLAN_GENERIC, ttt.PLAN_AUTO])
@pytest.mark.parametrize("d", [16, 64])
@pytest.mark.parametrize("chunk", [1, 16, 20])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("bias", [True, False])
def test_small_shapes(dev, plan, d, chunk, io, bias):
    wl = small(d, chunk, io, per_token=(chunk != 16), bias=bias)
    check_mlp(wl, 200 + d + chunk, dev, plan, bias_init=0.1)


@pytest.mark.parametrize("T", [1, 7, 33])
def test_edge_lengths(dev, T):
    check_mlp(small(64, 16, "bf16", per_token=True, T=T), 300 + T, dev, ttt.PLAN_AUTO)


def test_unaligned_eta(dev):
    # per-token eta at a 4-byte (not 16-byte) aligned address
    check_mlp(small(64, 16, "bf16", per_token=True, T=48), 317, dev, ttt.PLAN_AUTO, eta_offset=1)


def test_mlp_b16_4x16_full(dev):
    wl = inputs.WORKLOADS["mlp_b16_4x16"]
    check_mlp(wl, inputs.WORKLOAD_SEEDS[wl.name], dev, ttt.PLAN_AUTO)   # all 64 slices


# Operand range of the matrix-core plan (fp16 operands).  Values are scaled after
# generation (exact in bf16 for powers of two), so the oracle sees the same inputs.
# Scaling V alone makes the inner gradient descent itself diverge (the W1 step
# grows with the square of W2's scale), so the large-magnitude cases scale V and
# W2 together and shrink eta by the square of that factor: the descent stays
# stable and the fp64 oracle's outputs stay bounded, which each case checks first.
def scaled_case(dev, seed, plan, v=1.0, w1=1.0, w2=1.0, eta=0.1):
    wl = small(64, 16, "bf16", per_token=True, T=96, B=1, H=3).with_(eta_value=eta)
    x = inputs.make_inputs(wl, seed)
    x["V"] = (x["V"] * v).astype(np.float32)
    x["W1"] = (x["W1"] * w1).astype(np.float32)
    x["W2"] = (x["W2"] * w2).astype(np.float32)
    say("scaled case: V x%g, W1 x%g, W2 x%g, eta %g, plan %s"
        % (v, w1, w2, eta, ttt.plan_name(plan)))
    ref = oracle.mlp(x["K"], x["Q"], x["V"], x["eta"], x["eta_scalar"], x["W1"], x["b1"],
                     x["W2"], x["b2"], wl.chunk)
    bound = 1e3 * max(1.0, v, w1, w2)
    assert all(np.isfinite(r).all() and np.abs(r).max() < bound for r in ref if r is not None)
    got = run_mlp(wl, x, dev, plan=plan)
    errs = {n: rel_err(g, r) for n, g, r in zip(("Z", "W1", "b1", "W2", "b2"), got, ref)
            if r is not None}
    say("  max rel err", " ".join("%s %.3e" % kv for kv in errs.items()))
    return errs


@pytest.mark.parametrize("case", [
    dict(v=1024.0, w2=1024.0, eta=0.1 / 1024 ** 2),   # |V| ~ 4e3, |W2| ~ 1e2, eta ~ 1e-7
    dict(v=256.0, w2=256.0, eta=0.1 / 256 ** 2),
    dict(w1=8.0),                                      # |W1| ~ 0.7
    dict(eta=1.0 / 1024),                              # small gradient steps
])
def test_matrix_core_plan_inside_fp16_range(dev, case):
    errs = scaled_case(dev, 341, ttt.PLAN_MFMA, **case)
    assert all(e < TOL["bf16"] for e in errs.values()), errs


@pytest.mark.parametrize("case", [
    dict(v=2.0 ** 20, w2=2.0 ** 20, eta=0.1 / 2.0 ** 40),   # |W2| ~ 1e5 > 65504
    dict(v=2.0 ** -20, w1=2.0 ** -10, w2=2.0 ** -10),       # V ~ 1e-6, W ~ 1e-4
])
def test_generic_plan_outside_fp16_range(dev, case):
    """Magnitudes past fp16's range: the fp32 plan that callers choose for such data
    stays within the bf16 tolerance."""
    errs = scaled_case(dev, 342, ttt.PLAN_GENERIC, **case)
    assert all(e < TOL["bf16"] for e in errs.values()), errs


def test_matrix_core_overflow_is_not_silent(dev):
    """With W2 past 65504 the fp16 operands overflow: the outputs turn non-finite
    (the failure shows) rather than finite and wrong."""
    errs = scaled_case(dev, 343, ttt.PLAN_MFMA, v=2.0 ** 20, w2=2.0 ** 20, eta=0.1 / 2.0 ** 40)
    assert any(not np.isfinite(e) for e in errs.values()), errs
