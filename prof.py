"""Profiling helpers for the benchmark: a plain copy kernel of known size
(to calibrate the HBM byte counters), and summaries of rocprofv3 output.

  python prof.py copy [--mib 1024] [--reps 5]
      an elementwise copy (int8 negation) of a known number of bytes, run under
      rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) for the scale factor
  python prof.py trace DIR [--out FILE] [--cmd "..."]
      markdown table of a rocprofv3 --kernel-trace --stats directory
  python prof.py counters DIR [DIR ...] --kernel SUBSTR [--ms T] [--out FILE]
      markdown table of a kernel's rocprofv3 --pmc counters (per-dispatch
      means) with matrix-core busy, wait and issue fractions read off them
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


def counter_means(dirs, kernel_substr):
    """Per-dispatch mean of every counter of the kernels whose name contains
    kernel_substr, over one or more rocprofv3 --pmc output directories."""
    vals = {}
    for d in dirs:
        for f in _csvs(d, "*counter_collection.csv"):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if kernel_substr in r["Kernel_Name"]:
                        vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: statistics.mean(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}


def cmd_counters(a):
    """Markdown table of the counters of one kernel and the ratios read off
    them: matrix-core busy (SQ_VALU_MFMA_BUSY_CYCLES per SIMD over the GPU's
    active cycles), waves' cycles waiting on LDS, any wait, VMEM issue, the
    texture address / data units' busy fractions.  GRBM_GUI_ACTIVE reads as
    the sum over the chip's XCDs (it grows at XCDs x the shader clock), so
    the active cycles are GRBM_GUI_ACTIVE / xcds."""
    m, n = counter_means(a.dirs, a.kernel)
    if not m:
        raise SystemExit(f"no counter rows for kernels matching {a.kernel!r}")
    lines = []
    if a.cmd:
        lines += ["Command:", "", "```", a.cmd, "```", ""]
    lines += [f"Kernel: `{a.kernel}` (per-dispatch means over {max(n.values())} dispatches)", "",
              "| counter | per dispatch |", "|---|---:|"]
    for k in sorted(m):
        lines.append(f"| {k} | {m[k]:.4g} |")
    simds = a.cus * 4
    derived = []
    gui = m.get("GRBM_GUI_ACTIVE")
    if gui:
        gui = gui / a.xcds
    if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
        derived.append(("matrix-core busy, fraction of SIMD-cycles", m["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * simds)))
    wc = m.get("SQ_WAVE_CYCLES")
    if wc:
        for k, label in (("SQ_WAIT_INST_LDS", "wave-cycles waiting on LDS issue"),
                         ("SQ_WAIT_ANY", "wave-cycles waiting on anything"),
                         ("SQ_WAIT_INST_ANY", "wave-cycles waiting to issue any instruction"),
                         ("SQ_ACTIVE_INST_VMEM", "wave-cycles issuing vector-memory instructions"),
                         ("SQ_ACTIVE_INST_LDS", "wave-cycles issuing LDS instructions"),
                         ("SQ_ACTIVE_INST_VALU", "wave-cycles issuing VALU instructions")):
            if k in m:
                derived.append((label + ", fraction", m[k] / wc))
    if "SQ_INST_LEVEL_VMEM" in m and "SQ_INSTS_VMEM" in m and m["SQ_INSTS_VMEM"]:
        derived.append(("average vector-memory instruction latency, cycles", m["SQ_INST_LEVEL_VMEM"] / m["SQ_INSTS_VMEM"]))
    if "SQ_LDS_BANK_CONFLICT" in m and "SQ_ACTIVE_INST_LDS" in m and m["SQ_ACTIVE_INST_LDS"]:
        derived.append(("LDS bank-conflict cycles per LDS-active cycle", m["SQ_LDS_BANK_CONFLICT"] / m["SQ_ACTIVE_INST_LDS"]))
    if gui:
        for k in ("TA_TA_BUSY", "TD_TD_BUSY"):
            if k in m:
                derived.append((f"{k}, fraction of compute-unit active cycles", m[k] / (gui * a.cus)))
        if a.ms:
            derived.append((f"GRBM_GUI_ACTIVE / {a.xcds} / kernel time (shader clock), MHz", gui / (a.ms * 1e3)))
    if derived:
        lines += ["", "| derived | value |", "|---|---:|"] + [f"| {k} | {v:.4g} |" for k, v in derived]
    txt = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(txt)
    print(txt)


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
    k = sub.add_parser("counters")
    k.add_argument("dirs", nargs="+")
    k.add_argument("--kernel", required=True)
    k.add_argument("--cus", type=int, default=256)
    k.add_argument("--xcds", type=int, default=8)
    k.add_argument("--ms", type=float, default=None, help="kernel time per dispatch, for the clock estimate")
    k.add_argument("--out")
    k.add_argument("--cmd")
    a = ap.parse_args()
    {"copy": cmd_copy, "trace": cmd_trace, "traffic": cmd_traffic, "counters": cmd_counters}[a.cmd_name](a)


if __name__ == "__main__":
    main()
