"""Summaries of rocprofv3 CSV output for the profiles/ directory.

    python -m sparse_moe_expert_fp32_amd.profsum trace STATS_CSV OUT_MD --cmd "..."
    python -m sparse_moe_expert_fp32_amd.profsum traffic FETCH_CSV WRITE_CSV OUT_JSON \\
        --kernel REGEX --copy-bytes N --flops-per-launch F --cmd "..."

`trace` turns a --kernel-trace --stats kernel_stats.csv into a markdown table.
`traffic` takes two --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch),
averages them per dispatch of each kernel the pattern matches, sums those (the
launches of one stage), and scales each by the ratio between
the known size of a device-to-device copy and what the same counter read for
that copy (the copy kernel reads and writes exactly copy-bytes).
"""
from __future__ import annotations

import argparse
import csv
import json
import re
from collections import defaultdict


# kernels launched together as one stage of the layer (one launch per tile
# class); the trace summary adds a line with their summed average per stage
STAGES = {"gate/up expert GEMM (grouped_gemm_kernel<0, ...>, all tile classes)": r"grouped_gemm_kernel<0,",
          "down expert GEMM (grouped_gemm_kernel<1, ...>, all tile classes)": r"grouped_gemm_kernel<1,",
          "backward dH + SwiGLU (grouped_gemm_t_kernel<0, ...>, all tile classes)": r"grouped_gemm_t_kernel<0,",
          "backward dX_perm (grouped_gemm_t_kernel<1, ...>, all tile classes)": r"grouped_gemm_t_kernel<1,"}


def trace(stats_csv: str, out_md: str, cmd: str, top: int = 30):
    rows = list(csv.DictReader(open(stats_csv)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# Kernel trace summary", "", f"Command: `{cmd}`", "",
             "| kernel | calls | avg us | min us | max us | share |",
             "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        name = re.sub(r"\(.*", "", r["Name"])[:90]
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / total * 100:.1f}% |")
    lines += ["", "Per-stage sums (average of each launch in the stage, added):", ""]
    for label, rx in STAGES.items():
        sel = [r for r in rows if re.search(rx, r["Name"])]
        if sel:
            us = sum(float(r["AverageNs"]) for r in sel) / 1e3
            lines.append(f"- {label}: {us:.1f} us ({len(sel)} launches)")
    open(out_md, "w").write("\n".join(lines) + "\n")


def _dispatches(path: str, counter: str):
    acc = defaultdict(lambda: defaultdict(float))
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        acc[r["Kernel_Name"]][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in acc.items()}


def traffic(fetch_csv, write_csv, out_json, kernel, copy_bytes, flops_per_launch, cmd,
            sources_hash):
    f = _dispatches(fetch_csv, "FETCH_SIZE")
    w = _dispatches(write_csv, "WRITE_SIZE")
    pick = lambda d, rx: next(v for k, v in d.items() if re.search(rx, k))
    copy_rx = r"copyBuffer"
    mean = lambda v: sum(v) / len(v)
    # every kernel name the pattern matches is one launch of the stage (one
    # per tile class): per-dispatch means, summed over the launches
    allm = lambda d, rx: [v for k, v in d.items() if re.search(rx, k)]
    kf = sum(mean(v) for v in allm(f, kernel))
    kw = sum(mean(v) for v in allm(w, kernel))
    # the probe is the largest copy dispatch (the others are small uploads)
    cf, cw = max(pick(f, copy_rx)), max(pick(w, copy_rx))
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    rec = {
        "kernel": kernel, "command": cmd, "sources_hash": sources_hash,
        "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw,
        "copy_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "bytes_per_launch": kf * 1024.0 * f_scale + kw * 1024.0 * w_scale,
        "flops_per_launch": flops_per_launch,
    }
    json.dump(rec, open(out_json, "w"), indent=1)
    return rec


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv"); t.add_argument("out_md"); t.add_argument("--cmd", required=True)
    r = sub.add_parser("traffic")
    r.add_argument("fetch_csv"); r.add_argument("write_csv"); r.add_argument("out_json")
    r.add_argument("--kernel", required=True); r.add_argument("--copy-bytes", type=int, required=True)
    r.add_argument("--flops-per-launch", type=float, default=None)
    r.add_argument("--cmd", required=True)
    a = ap.parse_args()
    if a.what == "trace":
        trace(a.stats_csv, a.out_md, a.cmd)
    else:
        import os
        import sys
        sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
        import bench
        print(json.dumps(traffic(a.fetch_csv, a.write_csv, a.out_json, a.kernel, a.copy_bytes,
                                 a.flops_per_launch, a.cmd, bench.kernel_sources_hash()),
                         indent=1))


if __name__ == "__main__":
    main()
