"""GPU parity of ttt_linear_fwd_varlen (packed documents, each reset to its own
initial state) against the fp64 oracle run on every document alone.

Documents are packed head-major, [H, total_T, d]; document n of every head is
rows cu[n] .. cu[n+1]-1 and starts from W0[n].  Each document's outputs and
final state must match the oracle's scan of that document alone (max relative
error per (document, head), 1e-4 for fp32 I/O, 2e-2 for bf16 I/O); rows that no
document covers must keep what Z held before the call."""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, rel_err, say
from test_sequence_layers_ttt_amd import inputs, ttt

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ttt.lib()
    return torch.device("cuda:0")


def packed_case(lengths, H, d, chunk, io, per_token, seed, gap=0):
    """Seeded documents (one generator call per document) packed head-major."""
    base = inputs.workload("linear_b16_8x12")
    docs = []
    for n, L in enumerate(lengths):
        wl = base.with_(B=1, H=H, T=max(L, 1), d=d, chunk=chunk, io=io,
                        eta_mode="token" if per_token else "scalar",
                        eta_value=0.1 if per_token else 0.07)
        x = inputs.make_inputs(wl, seed * 1000 + n)
        docs.append((L, x))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    total_T = int(cu[-1]) + gap
    Kp = np.zeros((H, total_T, d), np.float32)
    Qp, Vp = Kp.copy(), Kp.copy()
    etap = np.zeros((H, total_T), np.float32) if per_token else None
    W0 = np.stack([x["W0"] for _, x in docs])              # [n_docs, H, d, d]
    for n, (L, x) in enumerate(docs):
        sl = slice(cu[n], cu[n] + L)
        Kp[:, sl], Qp[:, sl], Vp[:, sl] = x["K"][:, :L], x["Q"][:, :L], x["V"][:, :L]
        if per_token:
            etap[:, sl] = x["eta"][:, :L]
    return docs, cu, Kp, Qp, Vp, etap, W0, docs[0][1]["eta_scalar"]


def check(lengths, H, d, chunk, io, per_token, seed, dev, plan=ttt.PLAN_AUTO, gap=0,
          expect_plan=None):
    import torch
    docs, cu, Kp, Qp, Vp, etap, W0, eta_scalar = packed_case(lengths, H, d, chunk, io, per_token,
                                                             seed, gap)
    io_t = torch.bfloat16 if io == "bf16" else torch.float32
    io_code = ttt.DTYPE_BF16 if io == "bf16" else ttt.DTYPE_F32
    p = ttt.linear_select_plan_varlen(len(lengths), H, Kp.shape[1], d, chunk, io_code, plan)
    assert p > 0
    if expect_plan is not None:
        assert p == expect_plan
    say("case lengths", lengths[:12], "H", H, "d", d, "chunk", chunk, io, "plan", ttt.plan_name(p))
    t = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    K, Q, V = t(Kp, io_t), t(Qp, io_t), t(Vp, io_t)
    eta = None if etap is None else t(etap)
    Z = torch.full_like(K, SENTINEL)
    Z, Wo = ttt.linear_fwd_varlen(K, Q, V, eta, t(W0), t(cu, torch.int32), chunk,
                                  eta_scalar=eta_scalar, Z=Z, plan=plan)
    torch.cuda.synchronize()
    Zh, Wh = Z.float().cpu().numpy(), Wo.cpu().numpy()
    tol = TOL[io]
    worst = 0.0
    for n, (L, x) in enumerate(docs):
        if L == 0:
            np.testing.assert_array_equal(Wh[n], W0[n])
            continue
        Zo, Wref = oracle.linear(x["K"][:, :L], x["Q"][:, :L], x["V"][:, :L],
                                 None if x["eta"] is None else x["eta"][:, :L], x["eta_scalar"],
                                 x["W0"], chunk)
        ez = rel_err(np.transpose(Zh[:, cu[n]:cu[n] + L], (0, 1, 2)), Zo)
        ew = rel_err(Wh[n], Wref)
        worst = max(worst, ez, ew)
        assert ez < tol and ew < tol, (n, L, ez, ew)
    if gap:
        assert np.all(Zh[:, cu[-1]:] == SENTINEL)
    say("  max rel err %.3e over %d documents" % (worst, len(lengths)))


@pytest.mark.parametrize("d,chunk,io", [(64, 16, "bf16"), (128, 16, "bf16"), (32, 5, "bf16"),
                                        (64, 1, "bf16"), (16, 16, "f32"), (128, 3, "f32"),
                                        (64, 40, "bf16"), (32, 16, "f32")])
def test_documents(dev, d, chunk, io):
    check([1, 15, 16, 17, 0, 100, 33, 64], 3, d, chunk, io, per_token=(chunk != 1), seed=601,
          dev=dev, gap=5)


def test_generic_plan_matches(dev):
    check([7, 0, 40, 16], 2, 64, 16, "bf16", True, 602, dev, plan=ttt.PLAN_GENERIC,
          expect_plan=ttt.PLAN_GENERIC)


def test_many_documents(dev):
    """48 documents x 12 heads: past 256 (document, head, 16-row block) units the
    (document, head) slices go to the many-head kernel (four-wave workgroups)."""
    rng = np.random.default_rng(603)
    lengths = [int(v) for v in rng.integers(0, 90, size=48)]
    check(lengths, 12, 64, 16, "bf16", True, 603, dev, expect_plan=ttt.PLAN_MFMA)


@pytest.mark.parametrize("d,H,n_docs,per_token", [
    (64, 12, 24, True),     # 288 slices: one four-wave workgroup per slice
    (64, 12, 8, False),     # 96 slices: two two-wave workgroups per slice
    (128, 8, 8, True),      # 64 slices: two four-wave workgroups per slice
    (128, 12, 12, False),   # 144 slices: one eight-wave workgroup per slice
])
def test_many_head_kernel_documents(dev, d, H, n_docs, per_token):
    """Packed documents on every workgroup shape of the many-head kernel: empty,
    one-token, ragged and whole-chunk documents, rows past the last document
    untouched."""
    rng = np.random.default_rng(604 + d + n_docs)
    edge = [0, 1, 15, 16, 17, 64, 0, 33]
    lengths = edge + [int(v) for v in rng.integers(0, 70, size=n_docs - len(edge))]
    check(lengths, H, d, 16, "bf16", per_token, 604 + n_docs, dev, gap=3,
          expect_plan=ttt.PLAN_MFMA)


def test_malformed_offsets_stay_in_bounds(dev):
    """Offsets past total_T or decreasing are clamped: no fault, empty documents."""
    import torch
    H, d, T = 2, 32, 40
    K = torch.randn(H, T, d, device=dev).to(torch.bfloat16)
    W0 = torch.randn(3, H, d, d, device=dev) * 0.02
    cu = torch.tensor([0, 25, 10, 1 << 30], dtype=torch.int32, device=dev)
    Z, Wo = ttt.linear_fwd_varlen(K, K, K, None, W0, cu, 16, eta_scalar=0.05)
    torch.cuda.synchronize()
    assert torch.equal(Wo[1], W0[1])            # [25, 10) clamps to empty
    assert torch.isfinite(Z).all() and torch.isfinite(Wo).all()


def test_malformed_offsets_many_head_kernel(dev):
    """The same clamping with enough (document, head) slices for the many-head
    kernel: decreasing offsets give empty documents, offsets past total_T end at
    total_T."""
    import torch
    H, d, T = 12, 64, 100
    g = torch.Generator(device="cpu").manual_seed(605)
    K = (torch.randn(H, T, d, generator=g) * 0.2).to(torch.bfloat16).to(dev)
    cu_h = [0, 30, 12, 12, 50, 99, 1 << 30, 40, 60]
    n_docs = len(cu_h) - 1
    W0 = (torch.randn(n_docs, H, d, d, generator=g) * 0.02).to(dev)
    cu = torch.tensor(cu_h, dtype=torch.int32, device=dev)
    Z, Wo = ttt.linear_fwd_varlen(K, K, K, None, W0, cu, 16, eta_scalar=0.05)
    torch.cuda.synchronize()
    for n in (1, 2, 6):                         # [30, 12), [12, 12), [T, 40) clamp to empty
        assert torch.equal(Wo[n], W0[n]), n
    assert torch.isfinite(Z).all() and torch.isfinite(Wo).all()
