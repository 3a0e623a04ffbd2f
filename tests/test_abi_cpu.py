"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before any HIP call (no GPU needed; every call
here carries at least one argument the host validation refuses, so nothing is
ever launched)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

from test_sequence_layers_ttt_amd import ttt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt.h")

FAKE = 0x10000000          # aligned, never dereferenced: validation fails first
MISALIGNED = FAKE + 2


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_what_the_binding_lists():
    assert declared_functions() == sorted(ttt.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ttt.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ttt.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name


def test_status_and_plan_strings():
    assert ttt.status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert ttt.status_string(s) not in ("ok", "unknown status")
    assert ttt.status_string(17) == "unknown status"
    assert [ttt.plan_name(p) for p in range(5)] == ["auto", "generic", "mfma", "bigchunk",
                                                    "split"]
    assert ttt.plan_name(5) == "unknown plan"


def _linear(**kw):
    a = dict(K=FAKE, Q=FAKE, V=FAKE, eta=FAKE, eta_scalar=0.1, W0=FAKE, Z=FAKE, W=FAKE,
             B=1, H=1, T=16, d=16, chunk=16, io=0, ws=None, wsb=0, stream=None, plan=0)
    a.update(kw)
    return ttt.lib().ttt_linear_fwd_ex(a["K"], a["Q"], a["V"], a["eta"], a["eta_scalar"],
                                       a["W0"], a["Z"], a["W"], a["B"], a["H"], a["T"], a["d"],
                                       a["chunk"], a["io"], a["ws"], a["wsb"], a["stream"],
                                       a["plan"], ttt.READ_INCLUSIVE)


def _mlp(**kw):
    a = dict(K=FAKE, Q=FAKE, V=FAKE, eta=None, eta_scalar=0.05, W1=FAKE, b1=FAKE, W2=FAKE,
             b2=FAKE, Z=FAKE, W1o=FAKE, b1o=FAKE, W2o=FAKE, b2o=FAKE, B=1, H=1, T=16, d=64,
             chunk=16, io=1, ws=None, wsb=0, stream=None, plan=0)
    a.update(kw)
    return ttt.lib().ttt_mlp_fwd_ex(a["K"], a["Q"], a["V"], a["eta"], a["eta_scalar"], a["W1"],
                                    a["b1"], a["W2"], a["b2"], a["Z"], a["W1o"], a["b1o"],
                                    a["W2o"], a["b2o"], a["B"], a["H"], a["T"], a["d"],
                                    a["chunk"], a["io"], a["ws"], a["wsb"], a["stream"],
                                    a["plan"])


def _c_prototypes(src):
    """name -> list of parameter declarations, from a C header."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(?:int|size_t|const char\*)\s+(ttt_[a-z0-9_]+)\s*\(([^)]*)\)\s*;",
                         src):
        out[m.group(1)] = [p.strip() for p in m.group(2).split(",") if p.strip()]
    return out


# The boundary's signatures as the hot-path scope table fixes them: the calls a C
# caller written to that interface makes.  Extensions (plan choice, read order)
# live in the _ex entry points, so these keep exactly this argument list.
SCOPE_SIGNATURES = {
    "ttt_linear_workspace_bytes": ["int", "int", "int", "int", "int"],
    "ttt_linear_fwd": ["void*", "void*", "void*", "float*", "float", "float*", "void*",
                       "float*", "int", "int", "int", "int", "int", "int", "void*", "size_t",
                       "void*"],
    "ttt_mlp_workspace_bytes": ["int", "int", "int", "int", "int"],
    "ttt_mlp_fwd": ["void*", "void*", "void*", "float*", "float", "float*", "float*",
                    "float*", "float*", "void*", "float*", "float*", "float*", "float*",
                    "int", "int", "int", "int", "int", "int", "void*", "size_t", "void*"],
    "ttt_status_string": ["int"],
}


def _param_type(decl):
    decl = decl.replace("const ", "").strip()
    t = re.sub(r"\s*\b[A-Za-z_][A-Za-z0-9_]*$", "", decl)   # drop the parameter name
    return t.replace(" ", "")


def test_scope_table_signatures():
    protos = _c_prototypes(open(HEADER).read())
    for name, types in SCOPE_SIGNATURES.items():
        assert name in protos, name
        assert [_param_type(p) for p in protos[name]] == types, (name, protos[name])


def test_scope_table_argument_lists_reach_validation():
    """Calls with exactly the scope table's argument lists (no plan, no read
    order) go through the host validation; each carries one refused argument."""
    L = ttt.lib()
    assert L.ttt_linear_fwd(None, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, FAKE, 1, 1, 16, 16, 16, 0,
                            None, 0, None) == ttt.ERR_INVALID_ARG
    assert L.ttt_linear_fwd(FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, FAKE, 1, 1, 16, 48, 16, 0,
                            None, 0, None) == ttt.ERR_UNSUPPORTED
    # the large-chunk shape needs its workspace under AUTO
    assert L.ttt_linear_fwd(FAKE, FAKE, FAKE, None, 1.0 / 256, FAKE, FAKE, FAKE, 1, 2, 512, 64,
                            256, 1, None, 0, None) == ttt.ERR_WORKSPACE
    assert L.ttt_mlp_fwd(FAKE, FAKE, FAKE, None, 0.05, FAKE, None, FAKE, None, FAKE, FAKE,
                         None, FAKE, None, 1, 1, 16, 128, 16, 1, None, 0,
                         None) == ttt.ERR_UNSUPPORTED
    assert L.ttt_mlp_fwd(None, FAKE, FAKE, None, 0.05, FAKE, None, FAKE, None, FAKE, FAKE,
                         None, FAKE, None, 1, 1, 16, 64, 16, 1, None, 0,
                         None) == ttt.ERR_INVALID_ARG


def test_size_only_workspace_queries_cover_every_plan():
    for shape in [(1, 2, 512, 64, 256), (1, 16, 131072, 128, 2048), (8, 12, 2048, 64, 16),
                  (2, 3, 100, 32, 40)]:
        n = ttt.linear_workspace_bytes(*shape)
        for io in (ttt.DTYPE_F32, ttt.DTYPE_BF16):
            for plan in range(5):
                assert ttt.linear_workspace_bytes(*shape, io, plan) <= n
    assert ttt.linear_workspace_bytes(1, 2, 512, 64, 256) == \
        ttt.linear_workspace_bytes(1, 2, 512, 64, 256, ttt.DTYPE_BF16, ttt.PLAN_BIGCHUNK) > 0
    assert ttt.linear_workspace_bytes(8, 12, 2048, 64, 16) == 0
    for shape in [(1, 2, 64, 64, 16), (1, 2, 64, 64, 32), (3, 1, 50, 16, 5)]:
        n = ttt.mlp_workspace_bytes(*shape)
        for io in (ttt.DTYPE_F32, ttt.DTYPE_BF16):
            for plan in range(5):
                assert ttt.mlp_workspace_bytes(*shape, io, plan) <= n
    assert ttt.mlp_workspace_bytes(1, 2, 64, 64, 32) == 2 * (2 * 256 * 64 + 256 + 64) * 4


@pytest.mark.parametrize("kw,status", [
    (dict(K=None), ttt.ERR_INVALID_ARG),
    (dict(Q=None), ttt.ERR_INVALID_ARG),
    (dict(V=None), ttt.ERR_INVALID_ARG),
    (dict(W0=None), ttt.ERR_INVALID_ARG),
    (dict(Z=None), ttt.ERR_INVALID_ARG),
    (dict(W=None), ttt.ERR_INVALID_ARG),
    (dict(K=MISALIGNED), ttt.ERR_INVALID_ARG),
    (dict(Z=MISALIGNED), ttt.ERR_INVALID_ARG),
    (dict(W0=FAKE + 8), ttt.ERR_INVALID_ARG),
    (dict(eta=FAKE + 1), ttt.ERR_INVALID_ARG),
    (dict(eta=None, eta_scalar=math.nan), ttt.ERR_INVALID_ARG),
    (dict(eta=None, eta_scalar=math.inf), ttt.ERR_INVALID_ARG),
    (dict(B=0), ttt.ERR_INVALID_ARG),
    (dict(H=-1), ttt.ERR_INVALID_ARG),
    (dict(T=0), ttt.ERR_INVALID_ARG),
    (dict(chunk=0), ttt.ERR_INVALID_ARG),
    (dict(d=0), ttt.ERR_INVALID_ARG),
    (dict(io=2), ttt.ERR_INVALID_ARG),
    (dict(plan=7), ttt.ERR_INVALID_ARG),
    (dict(plan=5), ttt.ERR_INVALID_ARG),
    (dict(d=64, io=1, T=4096, plan=ttt.PLAN_SPLIT), ttt.ERR_WORKSPACE),
    (dict(d=64, io=0, T=4096, plan=ttt.PLAN_SPLIT), ttt.ERR_UNSUPPORTED),   # fp32 I/O
    (dict(d=64, io=1, T=1024, plan=ttt.PLAN_SPLIT), ttt.ERR_UNSUPPORTED),   # too short
    (dict(d=64, io=1, T=4100, plan=ttt.PLAN_SPLIT), ttt.ERR_WORKSPACE),   # ragged T: taken
    (dict(d=64, io=1, T=4096, B=4, H=9, plan=ttt.PLAN_SPLIT), ttt.ERR_WORKSPACE),  # 36 heads
    (dict(d=64, io=1, T=4096, B=5, H=13, plan=ttt.PLAN_SPLIT), ttt.ERR_UNSUPPORTED),  # 65 heads
    (dict(d=48), ttt.ERR_UNSUPPORTED),
    (dict(d=256), ttt.ERR_UNSUPPORTED),
    (dict(d=16, io=1, plan=ttt.PLAN_MFMA), ttt.ERR_UNSUPPORTED),
    (dict(io=0, d=64, plan=ttt.PLAN_BIGCHUNK), ttt.ERR_UNSUPPORTED),
    (dict(B=1 << 20, H=1 << 20, T=1 << 20), ttt.ERR_INVALID_ARG),
])
def test_linear_rejects_bad_arguments(kw, status):
    assert _linear(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(K=None), ttt.ERR_INVALID_ARG),
    (dict(W1=None), ttt.ERR_INVALID_ARG),
    (dict(W2o=None), ttt.ERR_INVALID_ARG),
    (dict(b1o=None), ttt.ERR_INVALID_ARG),          # b1 given, b1_out missing
    (dict(b2=None), ttt.ERR_INVALID_ARG),           # b2_out given, b2 missing
    (dict(b1=FAKE + 2), ttt.ERR_INVALID_ARG),
    (dict(W2=FAKE + 4), ttt.ERR_INVALID_ARG),
    (dict(eta_scalar=math.nan), ttt.ERR_INVALID_ARG),
    (dict(d=128), ttt.ERR_UNSUPPORTED),
    (dict(d=48), ttt.ERR_UNSUPPORTED),
    (dict(io=5), ttt.ERR_INVALID_ARG),
    (dict(T=-3), ttt.ERR_INVALID_ARG),
    (dict(plan=ttt.PLAN_BIGCHUNK), ttt.ERR_UNSUPPORTED),
    (dict(chunk=32, plan=ttt.PLAN_GENERIC), ttt.ERR_WORKSPACE),   # needs a workspace
    (dict(chunk=32, plan=ttt.PLAN_GENERIC, ws=FAKE, wsb=16), ttt.ERR_WORKSPACE),
])
def test_mlp_rejects_bad_arguments(kw, status):
    assert _mlp(**kw) == status


def _step(**kw):
    a = dict(K=FAKE, Q=FAKE, V=FAKE, eta=None, eta_scalar=0.1, Wc=FAKE, G=FAKE + 65536, pos=0,
             Z=FAKE, B=1, H=1, n=1, d=64, chunk=16, io=1, stream=None)
    a.update(kw)
    return ttt.lib().ttt_linear_step(a["K"], a["Q"], a["V"], a["eta"], a["eta_scalar"], a["Wc"],
                                     a["G"], a["pos"], a["Z"], a["B"], a["H"], a["n"], a["d"],
                                     a["chunk"], a["io"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(K=None), ttt.ERR_INVALID_ARG),
    (dict(Wc=None), ttt.ERR_INVALID_ARG),
    (dict(G=None), ttt.ERR_INVALID_ARG),
    (dict(Z=None), ttt.ERR_INVALID_ARG),
    (dict(G=FAKE), ttt.ERR_INVALID_ARG),            # state and update must not overlap
    (dict(G=FAKE + 4096), ttt.ERR_INVALID_ARG),     # d = 64: 16 KiB of state per slice
    (dict(Wc=FAKE + 65536, G=FAKE + 4096 * 13), ttt.ERR_INVALID_ARG),
    (dict(G=FAKE + 65540), ttt.ERR_INVALID_ARG),    # misaligned
    (dict(V=MISALIGNED), ttt.ERR_INVALID_ARG),
    (dict(eta=FAKE + 2), ttt.ERR_INVALID_ARG),
    (dict(eta_scalar=math.nan), ttt.ERR_INVALID_ARG),
    (dict(pos=-1), ttt.ERR_INVALID_ARG),
    (dict(pos=16), ttt.ERR_INVALID_ARG),
    (dict(n=0), ttt.ERR_INVALID_ARG),
    (dict(chunk=0, pos=0), ttt.ERR_INVALID_ARG),
    (dict(io=3), ttt.ERR_INVALID_ARG),
    (dict(d=48), ttt.ERR_UNSUPPORTED),
    (dict(d=256), ttt.ERR_UNSUPPORTED),
])
def test_step_rejects_bad_arguments(kw, status):
    assert _step(**kw) == status


def _bwd(**kw):
    a = dict(K=FAKE, Q=FAKE, V=FAKE, eta=None, eta_scalar=0.1, W0=FAKE, dZ=FAKE, dWT=None,
             dK=FAKE, dQ=FAKE, dV=FAKE, deta=None, dW0=FAKE, B=1, H=2, T=40, d=64, chunk=16,
             io=1, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return ttt.lib().ttt_linear_bwd(a["K"], a["Q"], a["V"], a["eta"], a["eta_scalar"], a["W0"],
                                    a["dZ"], a["dWT"], a["dK"], a["dQ"], a["dV"], a["deta"],
                                    a["dW0"], a["B"], a["H"], a["T"], a["d"], a["chunk"], a["io"],
                                    a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(K=None), ttt.ERR_INVALID_ARG),
    (dict(dZ=None), ttt.ERR_INVALID_ARG),
    (dict(dK=None), ttt.ERR_INVALID_ARG),
    (dict(dW0=None), ttt.ERR_INVALID_ARG),
    (dict(dQ=MISALIGNED), ttt.ERR_INVALID_ARG),
    (dict(dWT=FAKE + 8), ttt.ERR_INVALID_ARG),
    (dict(deta=FAKE + 2), ttt.ERR_INVALID_ARG),
    (dict(eta_scalar=math.inf), ttt.ERR_INVALID_ARG),
    (dict(T=0), ttt.ERR_INVALID_ARG),
    (dict(chunk=-1), ttt.ERR_INVALID_ARG),
    (dict(io=4), ttt.ERR_INVALID_ARG),
    (dict(d=48), ttt.ERR_UNSUPPORTED),
    (dict(ws=None), ttt.ERR_WORKSPACE),
    (dict(wsb=1024), ttt.ERR_WORKSPACE),
    (dict(ws=FAKE + 64), ttt.ERR_WORKSPACE),
])
def test_bwd_rejects_bad_arguments(kw, status):
    assert _bwd(**kw) == status


def test_bwd_workspace_size():
    # chunk-start states (ceil(T/b) + 1 per slice), then one fp32 plane of dK, of
    # dQ and of deta per 16-row block (d/16 of each); each piece rounded up to 256
    # bytes; the same for either I/O type
    B, H, T, d, b = 1, 2, 40, 64, 16
    up = lambda x: (x + 255) // 256 * 256
    states = up(B * H * (3 + 1) * d * d * 4)
    planes = 2 * up(d // 16 * B * H * T * d * 4) + up(d // 16 * B * H * T * 4)
    assert ttt.linear_bwd_workspace_bytes(B, H, T, d, b, 1) == states + planes
    assert ttt.linear_bwd_workspace_bytes(B, H, T, d, b, 0) == states + planes
    assert ttt.linear_bwd_workspace_bytes(B, H, T, 48, b, 1) == 0


def _linear_ex(read_mode, **kw):
    a = dict(K=FAKE, Q=FAKE, V=FAKE, eta=FAKE, eta_scalar=0.1, W0=FAKE, Z=FAKE, W=FAKE,
             B=1, H=1, T=16, d=16, chunk=16, io=0, ws=None, wsb=0, stream=None, plan=0)
    a.update(kw)
    return ttt.lib().ttt_linear_fwd_ex(a["K"], a["Q"], a["V"], a["eta"], a["eta_scalar"],
                                       a["W0"], a["Z"], a["W"], a["B"], a["H"], a["T"], a["d"],
                                       a["chunk"], a["io"], a["ws"], a["wsb"], a["stream"],
                                       a["plan"], read_mode)


@pytest.mark.parametrize("read_mode,kw,status", [
    (2, dict(), ttt.ERR_INVALID_ARG),
    (-1, dict(), ttt.ERR_INVALID_ARG),
    (1, dict(K=None), ttt.ERR_INVALID_ARG),
    (1, dict(d=64, io=1, plan=ttt.PLAN_MFMA), ttt.ERR_UNSUPPORTED),
    (1, dict(d=24), ttt.ERR_UNSUPPORTED),
    (1, dict(d=64, io=1, chunk=256, T=512, plan=ttt.PLAN_BIGCHUNK), ttt.ERR_WORKSPACE),
])
def test_linear_ex_rejects_bad_arguments(read_mode, kw, status):
    assert _linear_ex(read_mode, **kw) == status


def test_read_order_plan_selection():
    R = ttt.READ_CHUNK_START
    # small chunks: the matrix-core kernels read inclusively only
    assert ttt.linear_select_plan(8, 12, 2048, 64, 16, 1) == ttt.PLAN_MFMA
    assert ttt.linear_select_plan(1, 32, 32767, 64, 16, 1) == ttt.PLAN_SPLIT   # ragged T
    # 33 to 64 slices: the segmented plan from T = 4096 on, the chain kernel below
    assert ttt.linear_select_plan(2, 32, 4096, 64, 16, 1) == ttt.PLAN_SPLIT
    assert ttt.linear_select_plan(1, 40, 32768, 64, 16, 1) == ttt.PLAN_SPLIT
    assert ttt.linear_select_plan(2, 32, 4095, 64, 16, 1) == ttt.PLAN_MFMA
    assert ttt.linear_select_plan(2, 32, 2048, 64, 16, 1, ttt.PLAN_SPLIT) == ttt.PLAN_SPLIT
    assert ttt.linear_select_plan(1, 65, 8192, 64, 16, 1, ttt.PLAN_SPLIT) == ttt.ERR_UNSUPPORTED
    assert ttt.linear_select_plan(1, 65, 8192, 64, 16, 1) == ttt.PLAN_MFMA
    assert ttt.linear_select_plan(8, 12, 2048, 64, 16, 1, read_mode=R) == ttt.PLAN_GENERIC
    assert ttt.linear_select_plan(8, 12, 2048, 64, 16, 1, ttt.PLAN_MFMA, R) == ttt.ERR_UNSUPPORTED
    # large chunks: the three-stage plan in both orders
    assert ttt.linear_select_plan(1, 16, 4096, 128, 2048, 1, read_mode=R) == ttt.PLAN_BIGCHUNK
    assert ttt.linear_select_plan(1, 1, 64, 64, 16, 1, 0, 7) == ttt.ERR_INVALID_ARG


def _varlen(**kw):
    a = dict(K=FAKE, Q=FAKE, V=FAKE, eta=None, eta_scalar=0.1, W0=FAKE, Z=FAKE, W=FAKE,
             cu=FAKE, n_docs=3, H=2, total_T=40, d=64, chunk=16, io=1, stream=None, plan=0)
    a.update(kw)
    return ttt.lib().ttt_linear_fwd_varlen(a["K"], a["Q"], a["V"], a["eta"], a["eta_scalar"],
                                           a["W0"], a["Z"], a["W"], a["cu"], a["n_docs"], a["H"],
                                           a["total_T"], a["d"], a["chunk"], a["io"], a["stream"],
                                           a["plan"])


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), ttt.ERR_INVALID_ARG),
    (dict(cu=FAKE + 2), ttt.ERR_INVALID_ARG),
    (dict(K=None), ttt.ERR_INVALID_ARG),
    (dict(W0=FAKE + 4), ttt.ERR_INVALID_ARG),
    (dict(n_docs=0), ttt.ERR_INVALID_ARG),
    (dict(total_T=-1), ttt.ERR_INVALID_ARG),
    (dict(H=0), ttt.ERR_INVALID_ARG),
    (dict(chunk=0), ttt.ERR_INVALID_ARG),
    (dict(eta_scalar=math.nan), ttt.ERR_INVALID_ARG),
    (dict(d=48), ttt.ERR_UNSUPPORTED),
    (dict(plan=ttt.PLAN_BIGCHUNK), ttt.ERR_UNSUPPORTED),
    (dict(chunk=32, plan=ttt.PLAN_MFMA), ttt.ERR_UNSUPPORTED),
])
def test_varlen_rejects_bad_arguments(kw, status):
    assert _varlen(**kw) == status


def test_varlen_plan_selection():
    assert ttt.linear_select_plan_varlen(3, 2, 40, 64, 16, 1) == ttt.PLAN_MFMA
    assert ttt.linear_select_plan_varlen(3, 2, 40, 64, 32, 1) == ttt.PLAN_GENERIC
    assert ttt.linear_select_plan_varlen(3, 2, 40, 64, 16, 0) == ttt.PLAN_GENERIC
    assert ttt.linear_select_plan_varlen(3, 2, 0, 16, 16, 0) == ttt.PLAN_GENERIC


def _ln(**kw):
    a = dict(K=FAKE, Q=FAKE, V=FAKE, eta=None, eta_scalar=0.1, W0=FAKE, b0=FAKE, lnw=FAKE,
             lnb=FAKE, eps=1e-5, Z=FAKE, W=FAKE, b=FAKE, B=1, H=2, T=40, d=64, chunk=16, io=1,
             stream=None)
    a.update(kw)
    return ttt.lib().ttt_linear_ln_fwd(a["K"], a["Q"], a["V"], a["eta"], a["eta_scalar"],
                                       a["W0"], a["b0"], a["lnw"], a["lnb"], a["eps"], a["Z"],
                                       a["W"], a["b"], a["B"], a["H"], a["T"], a["d"], a["chunk"],
                                       a["io"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(b0=None), ttt.ERR_INVALID_ARG),
    (dict(b=None), ttt.ERR_INVALID_ARG),
    (dict(lnw=None), ttt.ERR_INVALID_ARG),          # weight and bias go together
    (dict(lnb=None), ttt.ERR_INVALID_ARG),
    (dict(lnw=FAKE + 2), ttt.ERR_INVALID_ARG),
    (dict(b0=FAKE + 1), ttt.ERR_INVALID_ARG),
    (dict(W0=FAKE + 4), ttt.ERR_INVALID_ARG),
    (dict(eps=0.0), ttt.ERR_INVALID_ARG),
    (dict(eps=-1.0), ttt.ERR_INVALID_ARG),
    (dict(eps=math.inf), ttt.ERR_INVALID_ARG),
    (dict(eta_scalar=math.nan), ttt.ERR_INVALID_ARG),
    (dict(T=0), ttt.ERR_INVALID_ARG),
    (dict(io=2), ttt.ERR_INVALID_ARG),
    (dict(d=48), ttt.ERR_UNSUPPORTED),
])
def test_ln_rejects_bad_arguments(kw, status):
    assert _ln(**kw) == status


def _mom(**kw):
    a = dict(K=FAKE, Q=FAKE, V=FAKE, eta=None, eta_scalar=0.1, W0=FAKE, M0=None, beta=0.9,
             Z=FAKE, W=FAKE, Mo=FAKE, B=1, H=2, T=40, d=64, chunk=16, io=1, ws=None, wsb=0,
             stream=None, plan=0)
    a.update(kw)
    return ttt.lib().ttt_linear_fwd_momentum(a["K"], a["Q"], a["V"], a["eta"], a["eta_scalar"],
                                             a["W0"], a["M0"], a["beta"], a["Z"], a["W"],
                                             a["Mo"], a["B"], a["H"], a["T"], a["d"], a["chunk"],
                                             a["io"], a["ws"], a["wsb"], a["stream"], a["plan"])


@pytest.mark.parametrize("kw,status", [
    (dict(Mo=None), ttt.ERR_INVALID_ARG),
    (dict(M0=FAKE + 8), ttt.ERR_INVALID_ARG),
    (dict(beta=1.0), ttt.ERR_INVALID_ARG),
    (dict(beta=-0.1), ttt.ERR_INVALID_ARG),
    (dict(beta=math.nan), ttt.ERR_INVALID_ARG),
    (dict(plan=ttt.PLAN_MFMA), ttt.ERR_UNSUPPORTED),
    (dict(d=40), ttt.ERR_UNSUPPORTED),
    (dict(chunk=256, T=512, d=128), ttt.ERR_WORKSPACE),   # the large-chunk plan needs one
])
def test_momentum_rejects_bad_arguments(kw, status):
    assert _mom(**kw) == status


def test_plan_selection_and_workspace_are_host_only():
    # fp32 I/O runs on the fp32 matrix cores (any chunk) unless the generic plan
    # is asked for or the read order is the chunk-start one
    assert ttt.linear_select_plan(1, 1, 256, 16, 16, ttt.DTYPE_F32) == ttt.PLAN_MFMA
    assert ttt.linear_select_plan(1, 1, 256, 16, 40, ttt.DTYPE_F32) == ttt.PLAN_MFMA
    assert ttt.linear_select_plan(1, 1, 256, 16, 16, 0, ttt.PLAN_GENERIC) == ttt.PLAN_GENERIC
    assert ttt.linear_select_plan(1, 1, 256, 16, 16, 0, ttt.PLAN_AUTO,
                                  ttt.READ_CHUNK_START) == ttt.PLAN_GENERIC
    assert ttt.linear_select_plan(1, 1, 256, 24, 16, 0) == ttt.ERR_UNSUPPORTED
    assert ttt.linear_workspace_bytes(8, 12, 2048, 64, 16, ttt.DTYPE_BF16) == 0
    assert ttt.mlp_workspace_bytes(1, 2, 64, 64, 16, 1, ttt.PLAN_GENERIC) == 0
    assert ttt.mlp_workspace_bytes(1, 2, 64, 64, 32, 1, ttt.PLAN_GENERIC) == \
        2 * (2 * 256 * 64 + 256 + 64) * 4


def _noalloc(**kw):
    a = dict(K=FAKE, Q=FAKE, V=FAKE, eta=None, eta_scalar=1.0 / 2048, W0=FAKE, Z=FAKE, W=FAKE,
             B=1, H=16, T=131072, d=128, chunk=2048, io=1, stream=None)
    a.update(kw)
    return ttt.lib().ttt_linear_fwd_noalloc(a["K"], a["Q"], a["V"], a["eta"], a["eta_scalar"],
                                            a["W0"], a["Z"], a["W"], a["B"], a["H"], a["T"],
                                            a["d"], a["chunk"], a["io"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(), ttt.ERR_WORKSPACE),            # 160 MiB of workspace > the 64 MiB scratch
    (dict(H=7), ttt.ERR_WORKSPACE),         # 70 MiB
    (dict(K=None), ttt.ERR_INVALID_ARG),
    (dict(Z=MISALIGNED), ttt.ERR_INVALID_ARG),
    (dict(eta_scalar=math.nan), ttt.ERR_INVALID_ARG),
    (dict(d=48), ttt.ERR_UNSUPPORTED),
    (dict(T=0), ttt.ERR_INVALID_ARG),
])
def test_noalloc_rejects_before_any_hip_call(kw, status):
    assert _noalloc(**kw) == status


def test_noalloc_scratch_size():
    n = ttt.linear_noalloc_scratch_bytes()
    assert n == 64 << 20
    # the largest large-chunk shapes that fit: 6 heads x 131072 tokens at d = 128
    assert ttt.linear_workspace_bytes(1, 6, 131072, 128, 2048, ttt.DTYPE_BF16) <= n
    assert ttt.linear_workspace_bytes(1, 7, 131072, 128, 2048, ttt.DTYPE_BF16) > n


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    K = torch.zeros(1, 1, 16, 16)
    with pytest.raises(ValueError):
        ttt.linear_fwd(K, K, K, None, torch.zeros(1, 1, 16, 16), 16, 0.1)


def test_profile_hash_covers_every_kernel_source():
    """bench.py invalidates stored counter profiles through a hash of the kernel
    sources; every file under csrc/ must be part of one of the hashed lists."""
    import glob
    import bench
    csrc = os.path.join(ROOT, "test_sequence_layers_ttt_amd", "csrc")
    files = {os.path.basename(p) for p in glob.glob(os.path.join(csrc, "*"))
             if p.endswith((".hip", ".h", ".cpp"))}
    hashed = set().union(*bench.KERNEL_SOURCES.values()) | bench.HOST_ONLY_SOURCES
    assert files <= hashed, sorted(files - hashed)
