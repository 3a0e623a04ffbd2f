"""Summarise rocprofv3 output for the TTT kernels.

  python -m test_sequence_layers_ttt_amd.rocprof_summary stats  <dir>   # kernel-trace --stats
  python -m test_sequence_layers_ttt_amd.rocprof_summary traffic \
        --fetch <dir> --write <dir> --copy-fetch <dir> --copy-write <dir> \
        --copy-bytes N --kernel SUBSTR [--json OUT --workload NAME --plan PLAN --model M]

`stats` prints the per-kernel table of a `--kernel-trace --stats --output-format csv`
run.  `traffic` averages FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the
kernels whose name contains SUBSTR, scales each by bytes / counter-reading of a
plain device copy of known size, and optionally writes the JSON that bench.py
reads as the roofline's `traffic` (tagged with the kernel-source hash, so it is
ignored once the kernels change).
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


def traffic(a):
    f_k, nf = counter_avg(a.fetch, "FETCH_SIZE", a.kernel)
    w_k, nw = counter_avg(a.write, "WRITE_SIZE", a.kernel)
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


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--json")
    t.add_argument("--workload", default="")
    t.add_argument("--plan", default="")
    t.add_argument("--model", default="linear")
    a = ap.parse_args()
    if a.cmd == "stats":
        stats(a.dir)
    else:
        traffic(a)


if __name__ == "__main__":
    main()
