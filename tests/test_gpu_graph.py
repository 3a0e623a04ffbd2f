"""HIP-graph capture of the library's entry points.

A call only enqueues kernels on the given stream (no allocation inside the
library, no memset, no host synchronisation), so a captured call must replay.
Each test captures one call with its outputs and workspace allocated beforehand,
replays the graph several times -- filling the outputs with NaN and running
unrelated eager work between replays -- and checks every replay bit for bit
against the eager call (every kernel is deterministic), and against the oracle
(same tolerances as the parity tests).
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, device_inputs, host, rel_err, say
from test_sequence_layers_ttt_amd import inputs, ttt

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ttt.lib()
    return torch.device("cuda:0")


def capture(fn):
    """Warm fn up on a side stream, then capture one call of it."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def eager_noise(dev):
    """Unrelated eager work between replays."""
    import torch
    a = torch.randn(256, 256, device=dev)
    (a @ a).sum().item()


def nan_fill(*ts):
    for t in ts:
        if t is not None:
            t.fill_(float("nan"))


def wl_small(d, chunk, io, T, B=2, H=3):
    base = inputs.workload("linear_b16_8x12")
    return base.with_(B=B, H=H, T=T, d=d, chunk=chunk, io=io, eta_mode="token", eta_value=0.1)


@pytest.mark.parametrize("d,chunk,io,T", [(64, 16, "bf16", 100),    # chunk-16 matrix-core kernel
                                          (16, 16, "f32", 77),      # fp32 matrix-core kernel
                                          (64, 128, "bf16", 300),   # three-stage plan + workspace
                                          (64, 16, "bf16", 2048)])  # segments along T + workspace
def test_linear_fwd_replays(dev, d, chunk, io, T):
    import torch
    wl = wl_small(d, chunk, io, T)
    x = inputs.make_inputs(wl, 901)
    a = device_inputs(wl, x, dev)
    io_code = 1 if io == "bf16" else 0
    plan = ttt.linear_select_plan(wl.B, wl.H, T, d, chunk, io_code)
    say("case", wl, "plan", ttt.plan_name(plan))
    nbytes = ttt.linear_workspace_bytes(wl.B, wl.H, T, d, chunk, io_code, plan)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev) if nbytes else None
    Z_ref, W_ref = ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], chunk,
                                  workspace=ws)
    torch.cuda.synchronize()
    Z, W = torch.empty_like(Z_ref), torch.empty_like(W_ref)
    g = capture(lambda: ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], chunk,
                                       Z=Z, W_out=W, workspace=ws))
    for r in range(REPLAYS):
        nan_fill(Z, W)
        eager_noise(dev)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Z, Z_ref) and torch.equal(W, W_ref), "replay %d differs" % r
    Zo, Wo = oracle.linear(x["K"], x["Q"], x["V"], x["eta"], x["eta_scalar"], x["W0"], chunk)
    assert rel_err(host(Z, wl.BH), Zo) < TOL[io] and rel_err(host(W, wl.BH), Wo) < TOL[io]


def test_linear_bwd_replays(dev):
    import torch
    wl = wl_small(64, 16, "bf16", 77)
    x = inputs.make_inputs(wl, 902)
    a = device_inputs(wl, x, dev)
    rng = np.random.default_rng([902, 77])
    dZ = inputs.round_to_bf16(rng.standard_normal((wl.BH, wl.T, wl.d), dtype=np.float32))
    dWT = rng.standard_normal((wl.BH, wl.d, wl.d), dtype=np.float32)
    B, H, T, d = wl.B, wl.H, wl.T, wl.d
    dZ_d = torch.from_numpy(dZ).to(dev).reshape(B, H, T, d).to(torch.bfloat16).contiguous()
    dWT_d = torch.from_numpy(dWT).to(dev).reshape(B, H, d, d)
    ws = torch.empty(ttt.linear_bwd_workspace_bytes(B, H, T, d, 16, 1), dtype=torch.uint8,
                     device=dev)
    outs = dict(dK=torch.empty_like(a["K"]), dQ=torch.empty_like(a["K"]),
                dV=torch.empty_like(a["K"]), deta=torch.empty((B, H, T), device=dev),
                dW0=torch.empty_like(a["W0"]))
    call = lambda: ttt.linear_bwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], dZ_d, 16,  # noqa: E731
                                  dW_T=dWT_d, workspace=ws, **outs)
    call()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    g = capture(call)
    ref = oracle.linear_bwd(x["K"], x["Q"], x["V"], x["eta"], x["eta_scalar"], x["W0"], 16,
                            dZ, dWT)
    for r in range(REPLAYS):
        nan_fill(*outs.values())
        eager_noise(dev)
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(outs[k], eager[k]) for k in outs), "replay %d differs" % r
        got = [host(outs["dK"], wl.BH), host(outs["dQ"], wl.BH), host(outs["dV"], wl.BH),
               outs["deta"].cpu().numpy().reshape(wl.BH, T), host(outs["dW0"], wl.BH)]
        errs = [rel_err(gv, rv) for gv, rv in zip(got, ref)]
        say("  replay %d max rel err %s" % (r, " ".join("%.2e" % e for e in errs)))
        assert all(e < TOL["bf16"] for e in errs), (r, errs)


def test_linear_ln_fwd_replays(dev):
    import torch
    wl = wl_small(64, 16, "bf16", 50)
    x = inputs.make_inputs(wl, 903)
    a = device_inputs(wl, x, dev)
    B, H, T, d = wl.B, wl.H, wl.T, wl.d
    rng = np.random.default_rng([903, 5])
    b0 = torch.from_numpy((0.1 * rng.standard_normal((B, H, d))).astype(np.float32)).to(dev)
    lnw = torch.from_numpy((1 + 0.1 * rng.standard_normal((H, d))).astype(np.float32)).to(dev)
    lnb = torch.from_numpy((0.1 * rng.standard_normal((H, d))).astype(np.float32)).to(dev)
    Z_ref, W_ref, b_ref = ttt.linear_ln_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], b0, lnw,
                                            lnb, 16, eps=1e-5)
    torch.cuda.synchronize()
    Z, W, b = torch.empty_like(Z_ref), torch.empty_like(W_ref), torch.empty_like(b_ref)
    g = capture(lambda: ttt.linear_ln_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], b0, lnw,
                                          lnb, 16, eps=1e-5, Z=Z, W_out=W, b_out=b))
    for r in range(REPLAYS):
        nan_fill(Z, W, b)
        eager_noise(dev)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Z, Z_ref) and torch.equal(W, W_ref) and torch.equal(b, b_ref), r


def test_linear_step_replays_continue_the_state(dev):
    """The decode step updates its state in place: each replay continues it, and
    the states after every replay equal those of the same eager calls."""
    import torch
    wl = wl_small(64, 16, "bf16", 64)
    x = inputs.make_inputs(wl, 904)
    a = device_inputs(wl, x, dev)
    n = 3   # tokens per call
    K, Q, V, eta = (a[k][:, :, :n].contiguous() for k in ("K", "Q", "V", "eta"))
    Wg, Gg = a["W0"].clone(), torch.zeros_like(a["W0"])
    We, Ge = a["W0"].clone(), torch.zeros_like(a["W0"])
    Zg, Ze = torch.empty_like(K), torch.empty_like(K)
    pos = 0
    # the graph's call runs at the position of its first replay; chunk 3 = n makes
    # every call start a chunk, so each replay is the same call on the next state
    g = capture(lambda: ttt.linear_step(K, Q, V, eta, Wg, Gg, pos, n, Z=Zg))
    # capture() ran the call once eagerly (its warm-up) and only recorded it
    # afterwards: restart both states from W0
    Wg.copy_(a["W0"])
    Gg.zero_()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        ttt.linear_step(K, Q, V, eta, We, Ge, pos, n, Z=Ze)
        eager_noise(dev)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Zg, Ze) and torch.equal(Wg, We) and torch.equal(Gg, Ge), r


def replay_equal(dev, call, outs):
    """Eager call, then capture and three replays that must equal it bit for bit."""
    import torch
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = capture(call)
    for r in range(REPLAYS):
        nan_fill(*outs)
        eager_noise(dev)
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o, e), "replay %d differs" % r
    return ref


def test_mlp_fwd_replays(dev):
    import torch
    wl = inputs.workload("mlp_b16_4x16").with_(B=2, H=2, T=40)
    x = inputs.make_inputs(wl, 905)
    a = device_inputs(wl, x, dev)
    Z = torch.empty_like(a["K"])
    W1, W2 = torch.empty_like(a["W1"]), torch.empty_like(a["W2"])
    b1, b2 = torch.empty_like(a["b1"]), torch.empty_like(a["b2"])
    say("case", wl, "plan", ttt.plan_name(ttt.mlp_select_plan(wl.B, wl.H, wl.T, wl.d, wl.chunk, 1)))
    replay_equal(dev, lambda: ttt.mlp_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W1"], a["b1"],
                                          a["W2"], a["b2"], wl.chunk,
                                          eta_scalar=x["eta_scalar"], Z=Z, W1_out=W1,
                                          b1_out=b1, W2_out=W2, b2_out=b2),
                 [Z, W1, b1, W2, b2])


def test_linear_fwd_varlen_replays(dev):
    import torch
    H, d, chunk = 3, 64, 16
    lengths = [37, 5, 64, 20]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    total_T = int(cu[-1])
    g = torch.Generator().manual_seed(906)
    K, Q, V = (torch.randn(H, total_T, d, generator=g).to(torch.bfloat16).to(dev)
               for _ in range(3))
    eta = (0.05 * torch.rand(H, total_T, generator=g)).to(dev)
    W0 = (0.02 * torch.randn(len(lengths), H, d, d, generator=g)).to(dev)
    cu_d = torch.from_numpy(cu).to(dev)
    Z, W = torch.zeros_like(K), torch.empty_like(W0)
    replay_equal(dev, lambda: ttt.linear_fwd_varlen(K, Q, V, eta, W0, cu_d, chunk, Z=Z,
                                                    W_out=W), [Z, W])


def test_linear_fwd_momentum_replays(dev):
    import torch
    wl = wl_small(64, 128, "bf16", 300)
    x = inputs.make_inputs(wl, 907)
    a = device_inputs(wl, x, dev)
    Mom0 = torch.zeros_like(a["W0"])
    plan = ttt.linear_select_plan(wl.B, wl.H, wl.T, wl.d, wl.chunk, 1,
                                  read_mode=ttt.READ_CHUNK_START)
    nbytes = ttt.linear_workspace_bytes(wl.B, wl.H, wl.T, wl.d, wl.chunk, 1, plan)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    say("case", wl, "plan", ttt.plan_name(plan))
    Z, W, M = torch.empty_like(a["K"]), torch.empty_like(a["W0"]), torch.empty_like(a["W0"])
    replay_equal(dev, lambda: ttt.linear_fwd_momentum(a["K"], a["Q"], a["V"], a["eta"], a["W0"],
                                                      Mom0, 0.9, wl.chunk, Z=Z, W_out=W,
                                                      Mom_out=M, workspace=ws), [Z, W, M])
