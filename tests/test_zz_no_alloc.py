"""ttt_linear_fwd_noalloc (the entry point that allocates nothing: its workspace
is the library's static per-GPU scratch) against ttt_linear_fwd with a caller
workspace, through the C ABI, on consecutive calls of decreasing size; and
against the fp64 oracle on sampled slices (max relative error per slice below
the bf16 tolerance 2e-2)."""
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


def shape_case(B, H, T, d, chunk, per_token, seed):
    base = inputs.workload("linear_b16_8x12")
    return base.with_(B=B, H=H, T=T, d=d, chunk=chunk, io="bf16",
                      eta_mode="token" if per_token else "scalar",
                      eta_value=0.1 if per_token else 1.0 / chunk), seed


# Calls in a row on one stream, each smaller than the one before: the large-chunk
# plan in the scratch, the segmented chunk-16 plan over a smaller part of it, the
# large-chunk plan again, and a shape that needs no workspace at all.
CALLS = [(1, 4, 8192, 128, 2048, False, 301),      # 10.0 MiB of scratch
         (1, 4, 4096, 64, 16, True, 304),           # 1.5 MiB, eight segments
         (2, 3, 1000, 64, 256, True, 302),          # 0.7 MiB, ragged last chunk
         (1, 2, 300, 64, 16, True, 303)]            # chunk-16 plan, no workspace


def test_noalloc_matches_workspace_entry(dev):
    import torch
    for (B, H, T, d, chunk, per_token, seed) in CALLS:
        wl, seed = shape_case(B, H, T, d, chunk, per_token, seed)
        plan = ttt.linear_select_plan(B, H, T, d, chunk, ttt.DTYPE_BF16)
        need = ttt.linear_workspace_bytes(B, H, T, d, chunk, ttt.DTYPE_BF16, plan)
        say("case", wl, "plan", ttt.plan_name(plan), "workspace", need)
        assert need <= ttt.linear_noalloc_scratch_bytes()
        x = inputs.make_inputs(wl, seed)
        a = device_inputs(wl, x, dev)
        Z1, W1 = ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], chunk,
                                eta_scalar=x["eta_scalar"])
        Z2 = torch.full_like(Z1, float("nan"))
        W2 = torch.full_like(W1, float("nan"))
        torch.cuda.synchronize()
        ttt.linear_fwd_noalloc(a["K"], a["Q"], a["V"], a["eta"], a["W0"], chunk,
                               eta_scalar=x["eta_scalar"], Z=Z2, W_out=W2)
        torch.cuda.synchronize()
        assert torch.equal(Z1, Z2) and torch.equal(W1, W2)
        idx = np.arange(min(wl.BH, 3))
        xo = take(x, idx)
        Zo, Wo = oracle.linear(xo["K"], xo["Q"], xo["V"], xo["eta"], xo["eta_scalar"],
                               xo["W0"], chunk)
        ez = rel_err(host(Z2, wl.BH)[idx], Zo)
        ew = rel_err(host(W2, wl.BH)[idx], Wo)
        say("  max rel err Z %.3e  W %.3e" % (ez, ew))
        assert ez < TOL["bf16"] and ew < TOL["bf16"]


def test_noalloc_rejects_oversized_workspace(dev):
    import torch
    # 7 heads x 131072 tokens at d = 128, chunk 2048 need 70 MiB (> 64 MiB):
    # rejected on the host before any launch; tiny tensors stand in for the inputs
    t = torch.zeros(16, device=dev)
    rc = ttt.lib().ttt_linear_fwd_noalloc(t.data_ptr(), t.data_ptr(), t.data_ptr(), None,
                                          1.0 / 2048, t.data_ptr(), t.data_ptr(), t.data_ptr(),
                                          1, 7, 131072, 128, 2048, ttt.DTYPE_BF16, None)
    assert rc == ttt.ERR_WORKSPACE

