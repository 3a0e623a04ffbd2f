"""Benchmark of the TTT forward scan on one MI355X.

One step = one ttt_linear_fwd (or ttt_mlp_fwd) call over the whole batch: every
(batch, head) scans its T tokens.  Inputs are resident in HBM before the timed
region; successive steps rotate over enough input/output copies (>= 1 GiB) that
the 256 MB last-level cache cannot serve them.

Default workload: TTT-Linear, 1 x 32 heads, d = 64, T = 32768, chunk b = 16, bf16
K/Q/V, per-token eta, fp32 state (the segmented plan).  Prints ONE JSON line on stdout; diagnostics go
to stderr.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--plan auto|generic|mfma|bigchunk]
                  [--no-cpu-baseline] [--copy-calibration BYTES]

With --decode N one step is instead one ttt_linear_step call that continues
every (batch, head) sequence of the workload by N tokens from its carried state
(decode).  The states rotate over >= 1 GiB of copies, so they come from HBM.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TTT scan tokens/sec (all heads) + % of HBM/MFMA roofline, b=16 d=64"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFS = 2500.0           # MI355X dense bf16 MFMA
PLANS = {"auto": 0, "generic": 1, "mfma": 2, "bigchunk": 3, "split": 4}
# sources whose change invalidates a stored counter profile, per kernel family (the
# host-side api.cpp only validates and dispatches; the plan is part of a profile's
# file name)
KERNEL_SOURCES = {"linear_b16": ["linear_mfma.hip", "linear_coop.hip", "mfma_common.h",
                                 "device_common.h", "launch.h"],
                  "linear_f32": ["linear_f32.hip", "mfma_f32.h", "mfma_common.h",
                                 "device_common.h", "launch.h"],
                  "linear_generic": ["linear_generic.hip", "device_common.h", "launch.h"],
                  "bigchunk": ["linear_bigchunk.hip", "mfma_common.h", "device_common.h",
                               "launch.h"],
                  "seg": ["linear_seg.hip", "mfma_common.h", "device_common.h", "launch.h"],
                  "mlp": ["mlp_mfma.hip", "mlp_generic.hip", "mfma_common.h", "device_common.h",
                          "launch.h"],
                  "step": ["linear_step.hip", "device_common.h", "launch.h"],
                  "ln": ["linear_ln.hip", "mfma_f32.h", "mfma_common.h", "device_common.h",
                         "launch.h"],
                  "bwd": ["linear_bwd.hip", "mfma_f32.h", "mfma_common.h", "device_common.h",
                          "launch.h"]}
HOST_ONLY_SOURCES = {"api.cpp"}


def kernel_family(wl, plan_name: str) -> str:
    """Which kernel sources a workload's plan runs."""
    if wl.model == "mlp":
        return "mlp"
    if plan_name == "bigchunk":
        return "bigchunk"
    if plan_name == "split":
        return "seg"
    if plan_name == "generic":
        return "linear_generic"
    return "linear_f32" if wl.io == "f32" else "linear_b16"


DECODE_METRIC = "TTT-Linear decode tokens/sec (all heads) + % of HBM roofline"
BWD_METRIC = "TTT-Linear backward tokens/sec (all heads) + % of MFMA roofline"
LN_METRIC = "TTT-Linear (bias, LayerNorm, residual) tokens/sec (all heads) + % of fp32 MFMA roofline"
FP32_PEAK_TFS = 157.3            # MI355X dense fp32 matrix


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(wl) -> float:
    """Bytes the scan must move once: K, Q, V read, Z written (io dtype), eta read
    (fp32, per-token mode), initial state read and final state written (fp32)."""
    esz = 2 if wl.io == "bf16" else 4
    per_tok = 4 * wl.d * esz + (4 if wl.eta_mode == "token" else 0)
    if wl.model == "linear":
        state = wl.d * wl.d * 4
    else:
        state = (2 * wl.hidden * wl.d + wl.hidden + wl.d) * 4
    return float(wl.BH) * (wl.T * per_tok + 2 * state)


def algorithmic_flops(wl, read_start: bool = False) -> float:
    """Flops of the dual form as stated for the method: per chunk of n tokens,
    TTT-Linear 3*2*d^2*n (W K, W Q, E K^T) + 2*d*n*(n+1) (causal half of the
    K^T Q and E S products; none with the chunk-start read order); TTT-MLP
    7*2*h*d*n + 2*(d+h)*n*(n+1)."""
    total = 0.0
    for c0 in range(0, wl.T, wl.chunk):
        n = min(wl.chunk, wl.T - c0)
        if wl.model == "linear":
            total += 6.0 * wl.d * wl.d * n + (0.0 if read_start else 2.0 * wl.d * n * (n + 1))
        else:
            h = wl.hidden
            total += 14.0 * h * wl.d * n + 2.0 * (wl.d + h) * n * (n + 1)
    return total * wl.BH


def kernel_hash(family: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[family]:
        p = os.path.join(ROOT, "test_sequence_layers_ttt_amd", "csrc", name)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def executed_flops_from_profiles(wl, plan_name):
    """Matrix-core flops one call executes (sum over its kernels) from the committed
    counter summary, or None when there is none or the kernel sources changed."""
    path = os.path.join(ROOT, "profiles", "mfma_%s_%s.json" % (wl.name, plan_name))
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    if rec.get("kernel_hash") != kernel_hash(kernel_family(wl, plan_name)):
        return None
    return rec.get("mfma_flops_per_call")


def traffic_from_profiles(wl, plan_name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none for this workload or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (wl.name, plan_name))
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    if rec.get("kernel_hash") != kernel_hash(kernel_family(wl, plan_name)):
        return None
    return rec.get("hbm_bytes_per_launch")


def decode_bytes(wl, n: int) -> float:
    """Bytes one decode call must move: the carried pair (W_chunk, G) read and G
    written (fp32), W_chunk written by the calls in which a chunk completes (a
    fraction min(1, n / chunk) of them), n tokens of K, Q, V read and Z written,
    eta read."""
    esz = 2 if wl.io == "bf16" else 4
    per_tok = 4 * wl.d * esz + (4 if wl.eta_mode == "token" else 0)
    state = wl.d * wl.d * 4
    return float(wl.BH) * ((3.0 + min(1.0, n / wl.chunk)) * state + n * per_tok)


def bwd_flops(wl) -> float:
    """Flops of the backward pass per (batch, head), in 16-token sub-tiles of m
    tokens: forward recompute of the chunk-start states (E = W K, W -= F K^T:
    4 d^2 m), then E, P K, dF's and dA's masked m x m products, dK (three
    products), dQ (two), dW (two): 16 d^2 m + 5 m (m + 1) d, plus 2 d^2 m for the
    running W - G when a chunk spans several sub-tiles."""
    d, total = wl.d, 0.0
    for c0 in range(0, wl.T, wl.chunk):
        n = min(wl.chunk, wl.T - c0)
        for s0 in range(0, n, 16):
            m = min(16, n - s0)
            total += 20.0 * d * d * m + 5.0 * m * (m + 1) * d
            if wl.chunk > 16:
                total += 2.0 * d * d * m
    return total * wl.BH


def bwd_main(args, wl, x, seed):
    """One step = one ttt_linear_bwd call over the whole batch (dZ, dW_T seeded)."""
    import torch
    from test_sequence_layers_ttt_amd import inputs, ttt
    dev = torch.device("cuda:0")
    B, H, T, d = wl.B, wl.H, wl.T, wl.d
    io = torch.bfloat16 if wl.io == "bf16" else torch.float32
    rng = np.random.default_rng([seed, 77])
    dZ = rng.standard_normal((wl.BH, T, d), dtype=np.float32)
    if wl.io == "bf16":
        dZ = inputs.round_to_bf16(dZ)
    dWT = rng.standard_normal((wl.BH, d, d), dtype=np.float32)

    def dev_t(a, shape, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).reshape(shape).to(dt).contiguous()

    base = {k: dev_t(x[k], (B, H, T, d), io) for k in ("K", "Q", "V")}
    base["eta"] = None if x["eta"] is None else dev_t(x["eta"], (B, H, T))
    base["W0"] = dev_t(x["W0"], (B, H, d, d))
    base["dZ"] = dev_t(dZ, (B, H, T, d), io)
    base["dWT"] = dev_t(dWT, (B, H, d, d))
    outs = {k: torch.empty_like(base["K"]) for k in ("dK", "dQ", "dV")}
    outs["deta"] = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    outs["dW0"] = torch.empty_like(base["W0"])
    io_code = ttt.DTYPE_BF16 if wl.io == "bf16" else ttt.DTYPE_F32
    nbytes = ttt.linear_bwd_workspace_bytes(B, H, T, d, wl.chunk, io_code)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    log("backward: workspace %.1f MB" % (nbytes / 1e6))
    stream = torch.cuda.current_stream(dev)

    def step():
        ttt.linear_bwd(base["K"], base["Q"], base["V"], base["eta"], base["W0"], base["dZ"],
                       wl.chunk, eta_scalar=x["eta_scalar"], dW_T=base["dWT"], dK=outs["dK"],
                       dQ=outs["dQ"], dV=outs["dV"], deta=outs["deta"], dW0=outs["dW0"],
                       workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_event = ev0.elapsed_time(ev1) / args.steps
    ms_step = wall * 1e3 / args.steps
    log("timed %d backward calls: %.4f ms/call (events), %.4f ms/call (wall)" % (
        args.steps, ms_event, ms_step))
    flops = bwd_flops(wl)
    tfs = flops / (ms_event * 1e-3) / 1e12

    cpu = parity = None
    if not args.no_cpu_baseline:
        import oracle
        per_slice = 6.0 * wl.T * wl.d * wl.d * 4   # the oracle's fp64 work, roughly
        nsl = args.cpu_sample_slices or int(max(1, min(wl.BH, 2.0e10 * 16 // per_slice)))
        idx = np.unique(np.linspace(0, wl.BH - 1, nsl).round().astype(int))
        t1 = time.perf_counter()
        ref = oracle.linear_bwd(x["K"][idx], x["Q"][idx], x["V"][idx],
                                None if x["eta"] is None else x["eta"][idx], x["eta_scalar"],
                                x["W0"][idx], wl.chunk, dZ[idx], dWT[idx], return_threads=True)
        tcpu = time.perf_counter() - t1
        nth = ref[5]
        cpu = {"value": round(len(idx) * wl.T / wl.H / tcpu, 1), "unit": "tokens/s",
               "cores": int(nth), "kind": "oracle",
               "sample": "%d of %d (batch, head) slices, full T=%d, fp64 per-token reverse "
                         "loop, %.2f s" % (len(idx), wl.BH, wl.T, tcpu)}
        got = [outs["dK"], outs["dQ"], outs["dV"], outs["deta"], outs["dW0"]]
        errs = {}
        for name, g, r in zip(("dK", "dQ", "dV", "deta", "dW0"), got, ref[:5]):
            gg = g.float().cpu().numpy().reshape(wl.BH, -1)[idx]
            rr = r.reshape(len(idx), -1)
            den = np.maximum(np.abs(rr).max(axis=1), 1e-6)
            errs[name] = float("%.3e" % (np.abs(gg - rr).max(axis=1) / den).max())
        parity = {"max_rel_err": errs, "slices_checked": int(len(idx))}
        log("oracle: %d slices in %.2f s on %d threads; parity %s" % (len(idx), tcpu, nth, parity))

    peak = BF16_PEAK_TFS if wl.io == "bf16" else FP32_PEAK_TFS
    rec = {
        "metric": BWD_METRIC,
        "value": round(B * T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # bf16 I/O: products on the bf16 matrix cores (fp32 operands split hi + lo),
        # priced against the dense bf16 peak; fp32 I/O: the fp32 matrix peak
        "dtype": "bf16x2" if wl.io == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name + "_bwd", "scan": "ttt_linear_bwd", "batch": B,
                   "heads": H, "seq_len": T, "head_dim": d, "chunk": wl.chunk, "io": wl.io,
                   "parallelism": "single_gpu"},
        "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tfs / peak, 4), "traffic": None,
                     "kernel_ms": round(ms_event, 5), "algorithmic_flops": flops},
        "cpu_baseline": cpu,
        "parity": parity,
        "head_tokens_per_s": round(B * H * T / (ms_step * 1e-3), 1),
    }
    print(json.dumps(rec), flush=True)


def ln_main(args, wl, x, seed):
    """TTT-Linear with the inner bias and LayerNorm + residual inside f: one step
    is one ttt_linear_ln_fwd call over the batch (seeded LN weight ~ 1 + 0.1 N,
    LN bias and b0 ~ 0.1 N, W0 std 0.1, eps 1e-5)."""
    import torch
    from test_sequence_layers_ttt_amd import ttt
    dev = torch.device("cuda:0")
    B, H, T, d = wl.B, wl.H, wl.T, wl.d
    rng = np.random.default_rng([seed, 55])
    b0 = (0.1 * rng.standard_normal((B, H, d))).astype(np.float32)
    lnw = (1.0 + 0.1 * rng.standard_normal((H, d))).astype(np.float32)
    lnb = (0.1 * rng.standard_normal((H, d))).astype(np.float32)
    W0 = (0.1 * rng.standard_normal((B, H, d, d))).astype(np.float32)
    eps = 1e-5
    io = torch.bfloat16 if wl.io == "bf16" else torch.float32
    t = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    K, Q, V = (t(x[k].reshape(B, H, T, d), io) for k in ("K", "Q", "V"))
    eta = None if x["eta"] is None else t(x["eta"].reshape(B, H, T))
    W0d, b0d, lnwd, lnbd = t(W0), t(b0), t(lnw), t(lnb)
    Z = torch.empty_like(K)
    Wo, bo = torch.empty_like(W0d), torch.empty_like(b0d)
    stream = torch.cuda.current_stream(dev)

    def step():
        ttt.linear_ln_fwd(K, Q, V, eta, W0d, b0d, lnwd, lnbd, wl.chunk, eps=eps,
                          eta_scalar=x["eta_scalar"], Z=Z, W_out=Wo, b_out=bo, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_event = ev0.elapsed_time(ev1) / args.steps
    ms_step = wall * 1e3 / args.steps
    log("timed %d LN calls: %.4f ms/call (events), %.4f ms/call (wall)" % (
        args.steps, ms_event, ms_step))
    # the dual form's products (as the plain scan) plus the bias terms; LN is O(d) per token
    flops = algorithmic_flops(wl) + 4.0 * wl.BH * T * d
    tfs = flops / (ms_event * 1e-3) / 1e12
    cpu = parity = None
    if not args.no_cpu_baseline:
        import oracle
        nsl = args.cpu_sample_slices or int(max(1, min(wl.BH, 2.0e10 * 16 // (4.0 * T * d * d))))
        idx = np.unique(np.linspace(0, wl.BH - 1, nsl).round().astype(int))
        heads = idx % H
        t1 = time.perf_counter()
        Zo, Wref, bref, nth = oracle.linear_ln(x["K"][idx], x["Q"][idx], x["V"][idx],
                                               None if x["eta"] is None else x["eta"][idx],
                                               x["eta_scalar"], W0.reshape(-1, d, d)[idx],
                                               b0.reshape(-1, d)[idx], lnw[heads], lnb[heads],
                                               eps, wl.chunk, return_threads=True)
        tcpu = time.perf_counter() - t1
        cpu = {"value": round(len(idx) * T / H / tcpu, 1), "unit": "tokens/s", "cores": int(nth),
               "kind": "oracle",
               "sample": "%d of %d (batch, head) slices, full T=%d, fp64 per-token primal "
                         "loop with LayerNorm, %.2f s" % (len(idx), wl.BH, T, tcpu)}
        errs = {}
        for name, g, r in (("Z", Z, Zo), ("W", Wo, Wref), ("b", bo, bref)):
            gg = g.float().cpu().numpy().reshape(wl.BH, -1)[idx]
            rr = r.reshape(len(idx), -1)
            den = np.maximum(np.abs(rr).max(axis=1), 1e-6)
            errs[name] = float("%.3e" % (np.abs(gg - rr).max(axis=1) / den).max())
        parity = {"max_rel_err": errs, "slices_checked": int(len(idx))}
        log("oracle: %d slices in %.2f s; parity %s" % (len(idx), tcpu, parity))
    peak = BF16_PEAK_TFS if wl.io == "bf16" else FP32_PEAK_TFS
    rec = {
        "metric": LN_METRIC,
        "value": round(B * T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # bf16 I/O: products on the bf16 matrix cores (fp32 operands split hi + lo),
        # priced against the dense bf16 peak; fp32 I/O: the fp32 matrix peak
        "dtype": "bf16x2" if wl.io == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name + "_ln", "scan": "ttt_linear_ln_fwd", "batch": B,
                   "heads": H, "seq_len": T, "head_dim": d, "chunk": wl.chunk, "io": wl.io,
                   "parallelism": "single_gpu"},
        "roofline": {"bound": "mfma", "achieved": round(tfs, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tfs / peak, 4), "traffic": None,
                     "kernel_ms": round(ms_event, 5), "algorithmic_flops": flops},
        "cpu_baseline": cpu,
        "parity": parity,
        "head_tokens_per_s": round(B * H * T / (ms_step * 1e-3), 1),
    }
    print(json.dumps(rec), flush=True)


def varlen_main(args, wl, x, seed):
    """Packed documents with a reset at each: the workload's B x T tokens per head,
    packed head-major and cut into documents of seeded lengths drawn uniformly
    from [T/4, 7T/4] (the last one takes the rest), each with its own W0."""
    import torch
    from test_sequence_layers_ttt_amd import ttt
    dev = torch.device("cuda:0")
    B, H, T, d = wl.B, wl.H, wl.T, wl.d
    total_T = B * T
    rng = np.random.default_rng([seed, 99])
    lengths = []
    while sum(lengths) < total_T:
        lengths.append(int(min(rng.integers(T // 4, 7 * T // 4 + 1), total_T - sum(lengths))))
    n_docs = len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    io = torch.bfloat16 if wl.io == "bf16" else torch.float32

    def packed(a):   # [B*H, T, d] -> [H, B*T, d]
        return np.ascontiguousarray(a.reshape(B, H, T, -1).transpose(1, 0, 2, 3).reshape(H, B * T, -1))

    t = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    K, Q, V = (t(packed(x[k]), io) for k in ("K", "Q", "V"))
    eta = None if x["eta"] is None else t(packed(x["eta"][..., None])[..., 0])
    W0 = t(rng.standard_normal((n_docs, H, d, d), dtype=np.float32) * np.float32(wl.state_std))
    cu_d = t(cu, torch.int32)
    Z = torch.empty_like(K)
    W_out = torch.empty_like(W0)
    io_code = ttt.DTYPE_BF16 if wl.io == "bf16" else ttt.DTYPE_F32
    plan = ttt.linear_select_plan_varlen(n_docs, H, total_T, d, wl.chunk, io_code)
    log("varlen: %d documents (lengths %d..%d) x %d heads, plan %s" % (
        n_docs, min(lengths), max(lengths), H, ttt.plan_name(plan)))
    stream = torch.cuda.current_stream(dev)

    def step():
        ttt.linear_fwd_varlen(K, Q, V, eta, W0, cu_d, wl.chunk, eta_scalar=x["eta_scalar"],
                              Z=Z, W_out=W_out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_event = ev0.elapsed_time(ev1) / args.steps
    ms_step = wall * 1e3 / args.steps
    log("timed %d varlen calls: %.4f ms/call (events), %.4f ms/call (wall)" % (
        args.steps, ms_event, ms_step))
    esz = 2 if wl.io == "bf16" else 4
    abytes = float(H) * total_T * (4 * d * esz + (4 if eta is not None else 0)) + \
        float(n_docs) * H * 2 * d * d * 4
    gbs = abytes / (ms_event * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(total_T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.io == "bf16" and plan == ttt.PLAN_MFMA else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name + "_varlen", "scan": "ttt_linear_fwd_varlen",
                   "documents": n_docs, "heads": H, "total_tokens": total_T, "head_dim": d,
                   "chunk": wl.chunk, "plan": ttt.plan_name(plan), "parallelism": "single_gpu"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel_ms": round(ms_event, 5), "algorithmic_bytes": abytes},
        "cpu_baseline": None,
        "parity": None,
        "head_tokens_per_s": round(H * total_T / (ms_step * 1e-3), 1),
    }
    print(json.dumps(rec), flush=True)


def decode_main(args, wl, x):
    """Decode: each call continues every sequence by n tokens.  The calls are
    captured once in a HIP graph (one per state copy) and the graph is replayed,
    so the events time the GPU rather than the host's launch rate."""
    import torch
    from test_sequence_layers_ttt_amd import ttt
    dev = torch.device("cuda:0")
    n = args.decode
    B, H, T, d = wl.B, wl.H, wl.T, wl.d
    io = torch.bfloat16 if wl.io == "bf16" else torch.float32

    def dev_t(a, shape, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).reshape(shape).to(dt).contiguous()

    seq = {k: dev_t(x[k], (B, H, T, d), io) for k in ("K", "Q", "V")}
    seq["eta"] = None if x["eta"] is None else dev_t(x["eta"], (B, H, T))
    # token groups [g*n, (g+1)*n) of the sequences, each a contiguous [B, H, n, d]
    ngroups = max(1, min(64, T // n))
    groups = []
    for g in range(ngroups):
        sl = slice(g * n, (g + 1) * n)
        groups.append({k: (None if v is None else v[:, :, sl].contiguous())
                       for k, v in seq.items()})
    W0 = dev_t(x["W0"], (B, H, d, d))
    state_bytes = 2 * W0.numel() * 4
    ncopies = max(1, min(1024, int(math.ceil(args.rotate_bytes / state_bytes))))
    states = [(W0.clone(), torch.zeros_like(W0)) for _ in range(ncopies)]
    pos = [0] * ncopies
    Z = torch.empty((B, H, n, d), dtype=io, device=dev)
    log("decode: %d tokens per call, %d state copies of %.1f MB" % (
        n, ncopies, state_bytes / 1e6))

    def call(i, stream):
        c = i % ncopies
        g = groups[(i // ncopies) % ngroups]
        Wc, G = states[c]
        _, pos[c] = ttt.linear_step(g["K"], g["Q"], g["V"], g["eta"], Wc, G, pos[c], wl.chunk,
                                    eta_scalar=x["eta_scalar"], Z=Z, stream=stream)

    # eager calls first (they also advance every copy to a mid-chunk position)
    stream = torch.cuda.current_stream(dev)
    for i in range(max(args.warmup, ncopies)):
        call(i, stream)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for c in range(ncopies):
            call(c, cap)
    torch.cuda.synchronize()
    reps = max(1, args.steps // ncopies)
    graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(reps):
        graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    calls = reps * ncopies
    ms_event = ev0.elapsed_time(ev1) / calls
    ms_step = wall * 1e3 / calls
    log("timed %d decode calls in %d graph replays: %.5f ms/call (events), %.5f ms/call "
        "(wall)" % (calls, reps, ms_event, ms_step))
    abytes = decode_bytes(wl, n)
    gbs = abytes / (ms_event * 1e-3) / 1e9
    rec = {
        "metric": DECODE_METRIC,
        "value": round(B * n / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": calls,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name + "_decode%d" % n, "scan": "ttt_linear_step",
                   "batch": B, "heads": H, "tokens_per_call": n, "head_dim": d,
                   "chunk": wl.chunk, "io": wl.io, "state_dtype": "f32",
                   "launch": "hip_graph", "parallelism": "single_gpu"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel_ms": round(ms_event, 5), "algorithmic_bytes": abytes},
        # the oracle's per-token cost is the scan's; its baseline is the scan line's
        "cpu_baseline": None,
        "parity": None,
        "head_tokens_per_s": round(B * H * n / (ms_step * 1e-3), 1),
    }
    print(json.dumps(rec), flush=True)


def copy_bandwidth(dev, nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Read + write GB/s of a plain 1 GiB device-to-device copy (torch's copy kernel)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


def copy_calibration(nbytes: int, steps: int):
    """A plain device copy of known size, for scaling the FETCH_SIZE/WRITE_SIZE
    counters (run under rocprofv3 --pmc)."""
    import torch
    n = nbytes // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "steps": steps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="linear_b16_1x32")
    ap.add_argument("--plan", default="auto", choices=sorted(PLANS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-slices", type=int, default=0,
                    help="slices the oracle times (0 = pick a bounded sample)")
    ap.add_argument("--rotate-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--copy-calibration", type=int, default=0)
    ap.add_argument("--decode", type=int, default=0,
                    help="time ttt_linear_step continuing every sequence by N tokens")
    ap.add_argument("--ln", action="store_true",
                    help="TTT-Linear with the inner bias and LayerNorm + residual inside f")
    ap.add_argument("--varlen", action="store_true",
                    help="TTT-Linear over the workload's tokens packed as documents with resets")
    ap.add_argument("--momentum", type=float, default=None,
                    help="TTT-Linear with a momentum state of this beta (chunk-start reads)")
    ap.add_argument("--read-start", action="store_true",
                    help="TTT-Linear with the chunk-start read order")
    ap.add_argument("--bwd", action="store_true",
                    help="time ttt_linear_bwd (the backward pass) on the workload")
    ap.add_argument("--decode-batch", type=int, default=0,
                    help="batch size of the decode line (default: the workload's)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from test_sequence_layers_ttt_amd import inputs, ttt

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return

    wl = inputs.WORKLOADS[args.workload]
    seed = inputs.WORKLOAD_SEEDS[wl.name]
    if args.ln:
        if wl.model != "linear":
            raise SystemExit("--ln needs a TTT-Linear workload")
        ln_main(args, wl, inputs.make_inputs(wl, seed), seed)
        return
    if args.varlen:
        if wl.model != "linear":
            raise SystemExit("--varlen needs a TTT-Linear workload")
        varlen_main(args, wl, inputs.make_inputs(wl, seed), seed)
        return
    if args.bwd:
        if wl.model != "linear":
            raise SystemExit("--bwd needs a TTT-Linear workload")
        bwd_main(args, wl, inputs.make_inputs(wl, seed), seed)
        return
    if args.decode:
        if wl.model != "linear" or args.decode > wl.T:
            raise SystemExit("--decode needs a TTT-Linear workload with T >= N")
        # a decode call reads only its own n tokens: generate the first few groups
        wl = wl.with_(T=min(wl.T, 64 * args.decode), B=args.decode_batch or wl.B)
        decode_main(args, wl, inputs.make_inputs(wl, seed))
        return
    dev = torch.device("cuda:0")
    plan_req = PLANS[args.plan]
    io_code = ttt.DTYPE_BF16 if wl.io == "bf16" else ttt.DTYPE_F32
    if args.momentum is not None:
        args.read_start = True   # the momentum scan reads every chunk at its start state
    read_mode = ttt.READ_CHUNK_START if args.read_start else ttt.READ_INCLUSIVE
    if args.read_start and wl.model != "linear":
        raise SystemExit("--read-start applies to TTT-Linear")
    if wl.model == "linear":
        plan = ttt.linear_select_plan(wl.B, wl.H, wl.T, wl.d, wl.chunk, io_code, plan_req,
                                      read_mode)
    else:
        plan = ttt.mlp_select_plan(wl.B, wl.H, wl.T, wl.d, wl.chunk, io_code, plan_req)
    if plan < 0:
        raise SystemExit("plan %s cannot run %s" % (args.plan, wl.name))
    plan_name = ttt.plan_name(plan)
    log("workload %s plan %s" % (wl.name, plan_name))

    t0 = time.time()
    x = inputs.make_inputs(wl, seed)
    log("inputs generated in %.1f s" % (time.time() - t0))

    io = torch.bfloat16 if wl.io == "bf16" else torch.float32
    B, H, T, d = wl.B, wl.H, wl.T, wl.d

    def dev_t(a, shape, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).reshape(shape).to(dt).contiguous()

    base = {k: dev_t(x[k], (B, H, T, d), io) for k in ("K", "Q", "V")}
    base["eta"] = None if x["eta"] is None else dev_t(x["eta"], (B, H, T))
    if wl.model == "linear":
        base["W0"] = dev_t(x["W0"], (B, H, d, d))
    else:
        base["W1"] = dev_t(x["W1"], (B, H, wl.hidden, d))
        base["W2"] = dev_t(x["W2"], (B, H, d, wl.hidden))
        base["b1"] = None if x["b1"] is None else dev_t(x["b1"], (B, H, wl.hidden))
        base["b2"] = None if x["b2"] is None else dev_t(x["b2"], (B, H, d))

    def out_set():
        o = {"Z": torch.empty((B, H, T, d), dtype=io, device=dev)}
        if wl.model == "linear":
            o["W"] = torch.empty_like(base["W0"])
        else:
            o["W1"] = torch.empty_like(base["W1"])
            o["W2"] = torch.empty_like(base["W2"])
            o["b1"] = None if base["b1"] is None else torch.empty_like(base["b1"])
            o["b2"] = None if base["b2"] is None else torch.empty_like(base["b2"])
        return o

    set_bytes = sum(t.numel() * t.element_size() for t in base.values() if t is not None)
    set_bytes += sum(t.numel() * t.element_size() for t in out_set().values() if t is not None)
    ncopies = max(1, min(64, int(math.ceil(args.rotate_bytes / set_bytes))))
    sets = [({k: (None if v is None else v.clone()) for k, v in base.items()}, out_set())
            for _ in range(ncopies)]
    nbytes_ws = (ttt.linear_workspace_bytes if wl.model == "linear" else ttt.mlp_workspace_bytes)(
        B, H, T, d, wl.chunk, io_code, plan)
    ws = torch.empty(max(nbytes_ws, 1), dtype=torch.uint8, device=dev) if nbytes_ws else None
    log("rotating over %d copies of %.1f MB (workspace %.1f MB)" % (
        ncopies, set_bytes / 1e6, nbytes_ws / 1e6))
    stream = torch.cuda.current_stream(dev)

    mom_out = torch.empty_like(base["W0"]) if args.momentum is not None else None

    def step(i):
        a, o = sets[i % ncopies]
        if args.momentum is not None:
            ttt.linear_fwd_momentum(a["K"], a["Q"], a["V"], a["eta"], a["W0"], None,
                                    args.momentum, wl.chunk, eta_scalar=x["eta_scalar"],
                                    Z=o["Z"], W_out=o["W"], Mom_out=mom_out, workspace=ws,
                                    plan=plan_req, stream=stream)
        elif wl.model == "linear":
            ttt.linear_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W0"], wl.chunk,
                           eta_scalar=x["eta_scalar"], Z=o["Z"], W_out=o["W"], workspace=ws,
                           plan=plan_req, stream=stream, read_mode=read_mode)
        else:
            ttt.mlp_fwd(a["K"], a["Q"], a["V"], a["eta"], a["W1"], a["b1"], a["W2"], a["b2"],
                        wl.chunk, eta_scalar=x["eta_scalar"], Z=o["Z"], W1_out=o["W1"],
                        b1_out=o["b1"], W2_out=o["W2"], b2_out=o["b2"], workspace=ws,
                        plan=plan_req, stream=stream)

    # Diagnostics first: the device copy rate, then the distribution of single calls
    # (each call between its own events, max(K, 50) calls).  They run before the
    # warm-up and the timed steps, so the timed region does not fall on the lower
    # core clock the GPU shows over its first few tens of calls after idling.
    copy_gbs = copy_bandwidth(dev)
    per_call = []
    for i in range(max(args.steps, 50)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step(i)
        e1.record(stream)
        per_call.append((e0, e1))
    torch.cuda.synchronize()
    call_ms = sorted(e0.elapsed_time(e1) for e0, e1 in per_call)
    log("single calls: median %.4f ms, min %.4f ms; 1 GiB device copy %.0f GB/s" % (
        call_ms[len(call_ms) // 2], call_ms[0], copy_gbs))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_event = ev0.elapsed_time(ev1) / args.steps
    ms_step = wall * 1e3 / args.steps
    log("timed %d steps: %.4f ms/step (events), %.4f ms/step (wall)" % (
        args.steps, ms_event, ms_step))

    tokens = B * T
    value = tokens / (ms_step * 1e-3)
    abytes = algorithmic_bytes(wl)
    aflops = algorithmic_flops(wl, args.read_start)
    achieved_gbs = abytes / (ms_event * 1e-3) / 1e9
    achieved_tfs = aflops / (ms_event * 1e-3) / 1e12
    traffic = None if args.read_start else traffic_from_profiles(wl, plan_name)
    # the large-chunk plan is a matrix-core workload with the inclusive read; with the
    # chunk-start read its Z pass is a plain W_c Q product and HBM bounds the call
    hbm_bound = wl.model == "linear" and (plan_name != "bigchunk" or args.read_start)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(achieved_tfs, 2), "peak": BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(achieved_tfs / BF16_PEAK_TFS, 4),
                "traffic": traffic}
    roof["kernel_ms"] = round(ms_event, 5)
    roof["call_ms_median"] = round(call_ms[len(call_ms) // 2], 5)
    roof["call_ms_min"] = round(call_ms[0], 5)
    # the same achieved rate against a measured device copy instead of the datasheet
    roof["copy_gbs"] = round(copy_gbs, 1)
    if hbm_bound:
        roof["frac_of_copy"] = round(achieved_gbs / copy_gbs, 4)
    roof["algorithmic_bytes"] = abytes
    roof["algorithmic_flops"] = aflops
    # matrix-core flops the kernels execute (counter summary), which can differ from
    # the method's count: the fraction of peak they reach in the same time
    xfl = None if args.read_start else executed_flops_from_profiles(wl, plan_name)
    if xfl is not None:
        roof["executed_flops"] = xfl
        roof["frac_executed"] = round(xfl / (ms_event * 1e-3) / 1e12 / BF16_PEAK_TFS, 4)

    # parity of the first output set against the oracle, and the CPU baseline
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        nsl = args.cpu_sample_slices or wl.BH
        # bound the oracle's work to roughly 10-30 s of host time
        per_slice_fma = wl.T * (3 * wl.d * wl.d if wl.model == "linear"
                                else 7 * wl.hidden * wl.d)
        ncores = os.cpu_count() or 1
        budget = 2.0e10 * max(1, min(ncores, 16))
        if not args.cpu_sample_slices:
            nsl = int(max(1, min(wl.BH, budget // per_slice_fma)))
        idx = np.linspace(0, wl.BH - 1, nsl).round().astype(int)
        idx = np.unique(idx)
        xo = {k: (v[idx] if isinstance(v, np.ndarray) else v) for k, v in x.items()}
        t1 = time.perf_counter()
        if args.momentum is not None:
            Zo, Wo, _, nth = oracle.linear_momentum(xo["K"], xo["Q"], xo["V"], xo["eta"],
                                                    xo["eta_scalar"], xo["W0"], None,
                                                    args.momentum, wl.chunk, return_threads=True)
            refs = {"Z": Zo, "W": Wo}
        elif wl.model == "linear":
            Zo, Wo, nth = oracle.linear(xo["K"], xo["Q"], xo["V"], xo["eta"], xo["eta_scalar"],
                                        xo["W0"], wl.chunk, return_threads=True,
                                        read_start=args.read_start)
            refs = {"Z": Zo, "W": Wo}
        else:
            r = oracle.mlp(xo["K"], xo["Q"], xo["V"], xo["eta"], xo["eta_scalar"], xo["W1"],
                           xo["b1"], xo["W2"], xo["b2"], wl.chunk, return_threads=True)
            refs = {"Z": r[0], "W1": r[1], "W2": r[3]}
            nth = r[5]
        tcpu = time.perf_counter() - t1
        cpu_tok_s = (len(idx) * wl.T / wl.H) / tcpu if wl.H > 0 else 0.0
        # tokens/s counts a token when all H heads are done: sample heads / H
        cpu = {"value": round(cpu_tok_s, 1), "unit": "tokens/s", "cores": int(nth),
               "kind": "oracle",
               "sample": "%d of %d (batch, head) slices, full T=%d, fp64 per-token primal "
                         "loop, %.2f s" % (len(idx), wl.BH, wl.T, tcpu)}
        o = sets[0][1]
        errs = {}
        for k, ref in refs.items():
            g = o[k].float().cpu().numpy().reshape(wl.BH, -1)[idx]
            r2 = ref.reshape(len(idx), -1)
            den = np.maximum(np.abs(r2).max(axis=1), 1e-6)
            errs[k] = float((np.abs(g - r2).max(axis=1) / den).max())
        parity = {"max_rel_err": {k: float("%.3e" % v) for k, v in errs.items()},
                  "slices_checked": int(len(idx))}
        log("oracle: %d slices in %.2f s on %d threads; parity %s" % (
            len(idx), tcpu, nth, parity))

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # arithmetic type of the products (accumulation and state are fp32)
        "dtype": ("f32" if wl.io == "f32" or plan_name == "generic"
                  else ("f16" if wl.model == "mlp" else "bf16")),
        "data": "synthetic",
        "config": {"workload": wl.name + ("_momentum" if args.momentum is not None else
                                          ("_read_start" if args.read_start else "")),
                   "scan": "ttt_" + wl.model, "batch": B, "heads": H,
                   "seq_len": T, "head_dim": d, "chunk": wl.chunk, "plan": plan_name,
                   "state_dtype": "f32", "parallelism": "single_gpu"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": parity,
        "head_tokens_per_s": round(B * H * T / (ms_step * 1e-3), 1),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
