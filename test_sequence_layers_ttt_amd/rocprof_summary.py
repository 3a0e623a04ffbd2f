"""Summarise rocprofv3 output for the TTT kernels.

  python -m test_sequence_layers_ttt_amd.rocprof_summary stats  <dir> [--last N]   # kernel-trace --stats
  python -m test_sequence_layers_ttt_amd.rocprof_summary traffic \
        --fetch <dir> --write <dir> --copy-fetch <dir> --copy-write <dir> \
        --copy-bytes N --kernel SUBSTR[,SUBSTR...] [--json OUT --workload NAME --plan PLAN --model FAMILY]
  python -m test_sequence_layers_ttt_amd.rocprof_summary mfma <dir> [--kernel SUBSTR]

`stats` prints the per-kernel table of a `--kernel-trace --stats --output-format csv`
run (with `--last N`, also each kernel's mean over its last N dispatches: a bench
run's timed steps come last).  `traffic` averages FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the
kernels whose name contains each SUBSTR, sums them over the substrings (one
library call launches each kernel once), scales each by bytes / counter-reading
of a plain device copy of known size, and optionally writes the JSON that bench.py
reads as the roofline's `traffic` (tagged with the kernel-source hash, so it is
ignored once the kernels change).  `mfma` tabulates matrix-core busy cycles and
executed matrix-core flops per kernel from a `--pmc SQ_VALU_MFMA_BUSY_CYCLES
SQ_INSTS_VALU_MFMA_MOPS_<type> GRBM_GUI_ACTIVE ...` run.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys


def _csv(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit("no *%s under %s" % (suffix, d))
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def last_dispatches(d, n):
    """Per kernel name, the mean and min duration of its last n dispatches in the
    kernel trace (the timed steps of a bench run, which come last)."""
    rows = _csv(d, "kernel_trace.csv")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    by = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print("| kernel | dispatches (last) | avg us | min us |")
    print("|---|---|---|---|")
    for name, ds in sorted(by.items(), key=lambda kv: -sum(kv[1][-n:])):
        tail = ds[-n:]
        short = name if len(name) <= 90 else name[:87] + "..."
        print("| %s | %d | %.2f | %.2f |" % (short, len(tail), sum(tail) / len(tail), min(tail)))


def stats(d):
    rows = _csv(d, "kernel_stats.csv")
    print("| kernel | calls | avg us | min us | max us | % |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        name = r["Name"]
        if len(name) > 90:
            name = name[:87] + "..."
        print("| %s | %s | %.2f | %.2f | %.2f | %.1f |" % (
            name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))


def counter_avg(d, counter, substr):
    rows = _csv(d, "counter_collection.csv")
    vals = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        if substr not in r.get("Kernel_Name", ""):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit("no %s rows for kernels matching %r in %s" % (counter, substr, d))
    return sum(vals.values()) / len(vals), len(vals)


def per_call(d, counter, kernels):
    """Sum over the comma-separated kernel substrings of each kernel's mean reading
    per dispatch: the counter per library call when a call launches each once."""
    tot, ns = 0.0, []
    for k in kernels.split(","):
        v, n = counter_avg(d, counter, k)
        tot += v
        ns.append(n)
    return tot, min(ns)


def traffic(a):
    f_k, nf = per_call(a.fetch, "FETCH_SIZE", a.kernel)
    w_k, nw = per_call(a.write, "WRITE_SIZE", a.kernel)
    cf, _ = counter_avg(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cw, _ = counter_avg(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    sf = a.copy_bytes / (cf * 1024.0)
    sw = a.copy_bytes / (cw * 1024.0)
    fetch_b = f_k * 1024.0 * sf
    write_b = w_k * 1024.0 * sw
    out = {"fetch_kib_raw": f_k, "write_kib_raw": w_k, "dispatches": [nf, nw],
           "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes": a.copy_bytes,
           "fetch_scale": sf, "write_scale": sw,
           "hbm_fetch_bytes_per_launch": fetch_b, "hbm_write_bytes_per_launch": write_b,
           "hbm_bytes_per_launch": fetch_b + write_b}
    print(json.dumps(out, indent=1))
    if a.json:
        sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
        import bench
        out.update({"workload": a.workload, "plan": a.plan, "kernel": a.kernel,
                    "kernel_hash": bench.kernel_hash(a.model)})
        with open(a.json, "w") as fh:
            json.dump(out, fh, indent=1)


def mfma(a):
    """Matrix-core use per kernel from SQ_VALU_MFMA_BUSY_CYCLES (busy cycles summed
    over every SIMD), SQ_INSTS_VALU_MFMA_MOPS_<type> (512 flops each) and
    GRBM_GUI_ACTIVE (GPU-busy cycles summed over the 8 XCDs)."""
    rows = _csv(a.dir, "counter_collection.csv")
    per = {}
    for r in rows:
        name = r.get("Kernel_Name", "")
        if a.kernel not in name:
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        c = per.setdefault(name, {}).setdefault(r["Counter_Name"], {})
        c[key] = c.get(key, 0.0) + float(r["Counter_Value"])
    out = []
    for name, cs in per.items():
        mean = {c: sum(v.values()) / len(v) for c, v in cs.items()}
        mops = [c for c in mean if c.startswith("SQ_INSTS_VALU_MFMA_MOPS_")]
        cycles = mean["GRBM_GUI_ACTIVE"] / a.xcds
        busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"]
        flops = 512.0 * sum(mean[c] for c in mops)
        us = cycles / (a.clock_ghz * 1e3)
        out.append({"kernel": name, "dispatches": len(next(iter(cs.values()))),
                    "gpu_busy_us": us, "mfma_busy_frac": busy / (cycles * a.simds),
                    "mfma_flops": flops, "mops_counters": mops,
                    "tflops_while_busy": flops / (us * 1e-6) / 1e12 if us > 0 else 0.0,
                    "sq_waves": mean.get("SQ_WAVES")})
    print("| kernel | dispatches | GPU-busy us | MFMA busy (of all SIMD cycles) | executed matrix-core GFLOP | TFLOP/s |")
    print("|---|---|---|---|---|---|")
    for o in out:
        n = o["kernel"]
        n = n if len(n) <= 90 else n[:87] + "..."
        print("| %s | %d | %.1f | %.3f | %.2f | %.1f |" % (
            n, o["dispatches"], o["gpu_busy_us"], o["mfma_busy_frac"], o["mfma_flops"] / 1e9,
            o["tflops_while_busy"]))
    if a.json:
        sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
        import bench
        rec = {"kernels": out, "mfma_flops_per_call": sum(o["mfma_flops"] for o in out),
               "workload": a.workload, "plan": a.plan, "kernel_hash": bench.kernel_hash(a.model),
               "model": a.model}
        with open(a.json, "w") as fh:
            json.dump(rec, fh, indent=1)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--last", type=int, default=0,
                   help="also average each kernel's last N dispatches from the kernel trace")
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--json")
    t.add_argument("--workload", default="")
    t.add_argument("--plan", default="")
    t.add_argument("--model", default="linear_b16",
                   help="kernel family whose source hash tags the JSON (bench.KERNEL_SOURCES)")
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    m.add_argument("--kernel", default="ttt")
    m.add_argument("--xcds", type=int, default=8)
    m.add_argument("--simds", type=int, default=256 * 4)
    m.add_argument("--clock-ghz", type=float, default=2.4)
    m.add_argument("--json")
    m.add_argument("--workload", default="")
    m.add_argument("--plan", default="")
    m.add_argument("--model", default="bigchunk")
    a = ap.parse_args()
    if a.cmd == "stats":
        stats(a.dir)
        if a.last:
            print()
            last_dispatches(a.dir, a.last)
    elif a.cmd == "mfma":
        mfma(a)
    else:
        traffic(a)


if __name__ == "__main__":
    main()
