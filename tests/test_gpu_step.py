"""GPU parity of ttt_linear_step, the streaming continuation of the TTT-Linear
scan, against the fp64 oracle's scan of the whole sequence.

A sequence cut into segments and fed through ttt_linear_step one segment after
the other, from (W_chunk, G, pos) = (W0, 0, 0), must give the oracle's outputs
for the uncut sequence with the same chunk size, and W_chunk - G must be the
oracle's state after the last token.  The cuts fall inside chunks, on chunk
boundaries and token by token.  Tolerance as for the scan: max relative error
per (batch, head) slice, 1e-4 with fp32 I/O and 2e-2 with bf16 I/O."""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, device_inputs, host, rel_err, say
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


def run_segments(wl, x, dev, cuts, prefill=0):
    """Feed tokens [0, T) through ttt_linear_step in segments ending at `cuts`;
    with prefill > 0 the first `prefill` tokens (a multiple of the chunk) go
    through ttt_linear_fwd instead.  Returns (Z, W_chunk - G) on the host."""
    import torch
    a = device_inputs(wl, x, dev)
    Wc = a["W0"].clone()
    G = torch.zeros_like(Wc)
    Zs = []
    t0, pos = 0, 0
    if prefill:
        assert prefill % wl.chunk == 0
        sl = slice(0, prefill)
        Zp, Wc = ttt.linear_fwd(a["K"][:, :, sl].contiguous(), a["Q"][:, :, sl].contiguous(),
                                a["V"][:, :, sl].contiguous(),
                                None if a["eta"] is None else a["eta"][:, :, sl].contiguous(),
                                a["W0"], wl.chunk, eta_scalar=x["eta_scalar"])
        Zs.append(Zp)
        t0 = prefill
    for t1 in [c for c in cuts if c < wl.T] + [wl.T]:
        if t1 <= t0:
            continue
        sl = slice(t0, t1)
        Z, pos = ttt.linear_step(a["K"][:, :, sl].contiguous(), a["Q"][:, :, sl].contiguous(),
                                 a["V"][:, :, sl].contiguous(),
                                 None if a["eta"] is None else a["eta"][:, :, sl].contiguous(),
                                 Wc, G, pos, wl.chunk, eta_scalar=x["eta_scalar"])
        assert pos == t1 % wl.chunk
        Zs.append(Z)
        t0 = t1
    torch.cuda.synchronize()
    Z = torch.cat(Zs, dim=2)
    return host(Z, wl.BH), host(Wc - G, wl.BH), host(G, wl.BH)


def check(wl, seed, dev, cuts, prefill=0):
    x = inputs.make_inputs(wl, seed)
    say("case", wl, "seed", seed, "cuts", list(cuts)[:12], "prefill", prefill)
    Z, W, G = run_segments(wl, x, dev, cuts, prefill)
    Zo, Wo = oracle.linear(x["K"], x["Q"], x["V"], x["eta"], x["eta_scalar"], x["W0"], wl.chunk)
    ez, ew = rel_err(Z, Zo), rel_err(W, Wo)
    say("  max rel err Z %.3e  W %.3e" % (ez, ew))
    tol = TOL[wl.io]
    assert ez < tol and ew < tol, (ez, ew)
    if wl.T % wl.chunk == 0:
        # a completed chunk folds its update into the chunk-start state
        assert np.all(G == 0)


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("chunk", [1, 5, 16])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_segments(dev, d, chunk, io):
    """Cuts inside chunks and on their boundaries."""
    wl = case(d, chunk, io, per_token=(chunk != 5), T=83)
    check(wl, 211, dev, cuts=[1, 7, 16, 19, 32, 50, 64, 65])


@pytest.mark.parametrize("d,io", [(64, "bf16"), (128, "f32"), (16, "f32")])
def test_token_by_token(dev, d, io):
    """Decode: one token per call."""
    wl = case(d, 16, io, per_token=True, T=40, B=1, H=2)
    check(wl, 212, dev, cuts=range(1, 40))


@pytest.mark.parametrize("chunk,T,prefill", [(16, 70, 48), (64, 200, 128), (16, 36, 32)])
def test_after_forward_scan(dev, chunk, T, prefill):
    """ttt_linear_fwd over a whole number of chunks hands over to the step."""
    wl = case(64, chunk, "bf16", per_token=True, T=T)
    check(wl, 213, dev, cuts=[prefill + 1, prefill + 9], prefill=prefill)


def test_one_call_whole_sequence(dev):
    """One call over the whole sequence is the scan itself (ragged last chunk)."""
    wl = case(128, 16, "bf16", per_token=False, T=100, B=3, H=2)
    check(wl, 214, dev, cuts=[])


def test_many_slices_decode(dev):
    """Many (batch, head) slices, a few decode steps after a long segment."""
    wl = case(64, 16, "bf16", per_token=True, T=37, B=8, H=12)
    check(wl, 215, dev, cuts=[33, 34, 35, 36])
