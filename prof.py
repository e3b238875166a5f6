"""Profiling helpers for the benchmark: a plain copy kernel of known size
(to calibrate the HBM byte counters), and summaries of rocprofv3 output.

  python prof.py copy [--mib 1024] [--reps 5]
      an elementwise copy (int8 negation) of a known number of bytes, run under
      rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) for the scale factor
  python prof.py trace DIR [--out FILE] [--cmd "..."]
      markdown table of a rocprofv3 --kernel-trace --stats directory
  python prof.py traffic --workload NAME --kernel SUBSTR
      --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR [--copy-mib 1024]
      HBM bytes per launch of the kernel (FETCH_SIZE + WRITE_SIZE, each
      scaled by what the counter reads for the copy), recorded in
      profiles/traffic.json under the current kernel source hash
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))


def _csvs(d: str, pattern: str):
    return sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))


def counter_per_dispatch(d: str, kernel_substr: str, counter: str):
    """Mean of a counter over the dispatches whose kernel name contains
    kernel_substr (rocprofv3 --pmc CSV output)."""
    vals = []
    for f in _csvs(d, "*counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
                    vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {kernel_substr!r} under {d}")
    return statistics.mean(vals), len(vals)


def cmd_copy(a):
    import torch
    # an elementwise kernel (not a DMA-engine memcpy) that reads and writes
    # exactly n bytes: int8 negation
    n = a.mib << 20
    src = torch.ones(n, dtype=torch.int8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(a.reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": a.reps}))


def cmd_trace(a):
    rows = []
    for f in _csvs(a.dir, "*kernel_stats.csv"):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {a.dir}")
    lines = []
    if a.cmd:
        lines += ["Command:", "", "```", a.cmd, "```", ""]
    lines += ["| kernel | calls | total ms | average us | min us | max us | % |",
              "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"]
        if len(name) > 90:
            name = name[:87] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    txt = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(txt)
    print(txt)


def cmd_traffic(a):
    sys.path.insert(0, ROOT)
    import bench
    copy_bytes = float(a.copy_mib << 20)
    cf, _ = counter_per_dispatch(a.copy_fetch, a.copy_kernel, "FETCH_SIZE")
    cw, _ = counter_per_dispatch(a.copy_write, a.copy_kernel, "WRITE_SIZE")
    kf, nf = counter_per_dispatch(a.fetch, a.kernel, "FETCH_SIZE")
    kw, nw = counter_per_dispatch(a.write, a.kernel, "WRITE_SIZE")
    # counters read in KiB; the copy moves copy_bytes each way
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    rec = {
        "kernel_source_hash": bench.kernel_source_hash(a.workload),
        "kernel": a.kernel,
        "fetch_bytes_per_launch": kf * 1024.0 * f_scale,
        "write_bytes_per_launch": kw * 1024.0 * w_scale,
        "bytes_per_launch": kf * 1024.0 * f_scale + kw * 1024.0 * w_scale,
        "fetch_kib_raw": kf, "write_kib_raw": kw, "dispatches": [nf, nw],
        "copy_scale": {"fetch": f_scale, "write": w_scale, "copy_mib": a.copy_mib},
    }
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = {}
    if os.path.exists(path):
        with open(path) as fh:
            data = json.load(fh)
    data[a.workload] = rec
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    print(json.dumps({a.workload: rec}, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=5)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--out")
    t.add_argument("--cmd")
    f = sub.add_parser("traffic")
    f.add_argument("--workload", required=True)
    f.add_argument("--kernel", required=True)
    f.add_argument("--fetch", required=True)
    f.add_argument("--write", required=True)
    f.add_argument("--copy-fetch", required=True)
    f.add_argument("--copy-write", required=True)
    f.add_argument("--copy-kernel", default="neg_kernel")
    f.add_argument("--copy-mib", type=int, default=1024)
    a = ap.parse_args()
    {"copy": cmd_copy, "trace": cmd_trace, "traffic": cmd_traffic}[a.cmd_name](a)


if __name__ == "__main__":
    main()
