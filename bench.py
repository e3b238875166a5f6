"""Benchmark of the grouped matmul on one MI355X.

A step is one pass of the whole hot path for a 128-expert top-8 MoE layer in
bf16: the up-projection forward gmm (lhs [262144,1408] x rhs [128,1408,1408],
an NT product) followed by the down-projection backward dlhs gmm (dout
[262144,1408] x the forward weight [128,1408,704] read in place, an NN
product).  Each gmm call is one kernel launch that builds the group offsets
and tile table, zero-fills inactive rows and runs the MFMA tiles.  Inputs are
seeded synthetic tensors already resident in HBM.

Prints one JSON line: TFLOP/s over the timed steps (algorithmic FLOPs, i.e.
2 * active rows * N * K), the roofline of the dominant kernel measured with
HIP events on the launch stream, and the CPU oracle timed on a bounded sample
of the same workload.

  python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}   # dense MFMA TFLOP/s (MI355X)
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the sources each workload's kernel is built from: committed counter
# readings stay valid until one of them changes
KERNEL_SOURCES_COMMON = ("gmm_params.hpp", "gmm_device.hpp", "gmm_kernels.hip", "gmm_launch.hpp")
KERNEL_SOURCES = {
    "tiny_fp32": (),
    "moe_fwd_bf16": ("gmm_big.hpp",),
    "moe_dlhs_bf16": ("gmm_big.hpp",),
    "decode_fp8w": ("gmm_big.hpp", "gmm_stream.hpp", "gmm_stream.hip"),
    "w8a8_fp8": ("gmm_big.hpp", "gmm_w8a8.hpp", "gmm_w8a8.hip"),
    "tgmm_bf16": ("gmm_big.hpp", "gmm_tgmm.hpp", "gmm_tgmm_tiles.hpp"),
    "quant_fp8": ("gmm_quant.hip",),
}
# workloads whose weights fit in the caches between calls: each timed call
# starts from evicted L2 / Infinity Cache (a 512 MB read outside the events)
EVICT = {"decode_fp8w", "tiny_fp32"}


def kernel_source_hash(workload: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES_COMMON + KERNEL_SOURCES.get(workload, ()):
        with open(os.path.join(ROOT, "moe_grouped_matrix_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None
    when there are none for this workload or the kernels changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash(workload):
        return None
    return rec.get("bytes_per_launch")


def build_cases(workload: str, device):
    import workloads
    if workload in workloads.TGMM_FULL:
        return [workloads.TGMM_FULL[workload](device=device)]
    if workload in workloads.QUANT_FULL:
        return [workloads.QUANT_FULL[workload](device=device)]
    names = {"fwd+dlhs": ["moe_fwd_bf16", "moe_dlhs_bf16"]}.get(workload, [workload])
    return [workloads.FULL[n](device=device) for n in names]


def is_tgmm(case) -> bool:
    return hasattr(case, "rhs") and not hasattr(case, "transpose_rhs")


def is_quant(case) -> bool:
    return hasattr(case, "x") and not hasattr(case, "rhs")


def op_peak(case):
    import torch
    if is_quant(case):
        return "bf16", PEAK["bf16"]
    if case.lhs.dtype == torch.float8_e4m3fn:
        return "fp8", PEAK["fp8"]
    if case.lhs.dtype == torch.float32:
        return "f32", PEAK["f32"]
    return "bf16", PEAK["bf16"]


def _host():
    """The host the CPU baseline ran on: logical CPUs and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"os_cpu_count": os.cpu_count(), "cpu_model": model}


# workloads whose CPU baseline is also timed on one thread (the microsecond-
# scale ones, where a caller might weigh a single host core against the GPU)
SINGLE_THREAD = {"tiny_fp32", "decode_fp8w"}


def cpu_baseline(cases, target_s: float = 20.0):
    """Time the oracle on a bounded sample of each case: a few rows of a few
    groups, packed into a sub-problem with the same K, N and weights (every
    row costs the same arithmetic as in the full problem)."""
    import numpy as np
    import torch

    import oracle
    import workloads

    oracle.build(force=False)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    if any(is_tgmm(c) for c in cases):
        return cpu_baseline_tgmm(cases, target_s)
    if any(is_quant(c) for c in cases):
        return cpu_baseline_quant(cases, target_s)
    def sample(rows_per):
        flops_total = secs_total = 0.0
        descr = []
        for case in cases:
            sizes = case.sizes_list()
            groups = [g for g in range(case.group_offset, case.group_offset + case.num_active)
                      if sizes[g] > 0][:32]
            o = np.concatenate([[0], np.cumsum(sizes)])
            idx, sub_sizes = [], []
            for g in groups:
                n = min(rows_per, sizes[g])
                idx.extend(range(int(o[g]), int(o[g]) + n))
                sub_sizes.append(n)
            idx_t = torch.tensor(idx, device=case.lhs.device)
            h_idx = torch.tensor([g - case.group_offset for g in groups], device=case.lhs.device)
            sub = workloads.Case(
                case.name, case.lhs.index_select(0, idx_t).cpu(), case.rhs.index_select(0, h_idx).cpu(),
                torch.tensor(sub_sizes, dtype=torch.int32), transpose_rhs=case.transpose_rhs,
                rhs_scale=None if case.rhs_scale is None else case.rhs_scale.index_select(0, h_idx).cpu(),
                rhs_bias=None if case.rhs_bias is None else case.rhs_bias.index_select(0, h_idx).cpu(),
                lhs_scale=None if case.lhs_scale is None else case.lhs_scale.index_select(0, idx_t).cpu(),
                out_dtype=case.out_dtype)
            t0 = time.perf_counter()
            oracle.gmm_reference(sub.lhs, sub.rhs, sub.group_sizes, transpose_rhs=sub.transpose_rhs,
                                 rhs_scale=sub.rhs_scale, rhs_bias=sub.rhs_bias, lhs_scale=sub.lhs_scale)
            secs_total += time.perf_counter() - t0
            flops_total += 2.0 * len(idx) * case.N * case.K
            descr.append(f"{case.name}: {len(idx)} rows of {len(groups)} groups")
        return flops_total, secs_total, descr

    # calibrate, then size the sample to ~target_s (re-measuring while the
    # sample ran well short of it: per-group setup dominates small samples)
    rows_per = 16
    for phase in ("calibrate", "calibrate", "measure"):
        flops_total, secs_total, descr = sample(rows_per)
        if phase == "calibrate":
            scale = target_s / max(secs_total, 1e-3)
            rows_per = max(1, int(rows_per * scale))
            if secs_total > 0.5 * target_s:
                break
    res = {"value": flops_total / secs_total / 1e12, "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle",
           "sample": "; ".join(descr) + f" (fp64 oracle, {secs_total:.1f} s)"}
    res.update(_host())
    if all(c.name in SINGLE_THREAD for c in cases):
        # the same kind of sample on one thread, sized for a few seconds
        rows_1 = max(1, int(rows_per * 3.0 / max(secs_total * threads, 1e-3)))
        oracle.set_threads(1)
        try:
            f1, s1, d1 = sample(rows_1)
        finally:
            oracle.set_threads(threads)
        res["single_thread"] = {"value": f1 / s1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                                "sample": "; ".join(d1) + f" (fp64 oracle, {s1:.1f} s)"}
    return res


def cpu_baseline_tgmm(cases, target_s: float = 20.0):
    """Time the oracle's tgmm on a bounded sample: whole output rows (h, k)
    of a spread of groups, each costing rows_h * N multiply-adds exactly as
    in the full problem."""
    import numpy as np

    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    case = cases[0]
    sizes = case.sizes_list()
    lhs, rhs, gs = case.lhs.cpu(), case.rhs.cpu(), case.group_sizes.cpu()
    groups = [h for h in range(case.num_active) if sizes[case.group_offset + h] > 0]
    groups = groups[::max(1, len(groups) // 16)]
    per = 2
    for phase in ("calibrate", "calibrate", "measure"):
        sel = [(h, (7 * j + h) % case.K) for h in groups for j in range(per)]
        t0 = time.perf_counter()
        oracle.tgmm_reference(lhs, rhs, gs, group_offset=case.group_offset, num_active=case.num_active,
                              select=sel)
        secs = time.perf_counter() - t0
        flops = sum(2.0 * sizes[case.group_offset + h] * case.N for h, _ in sel)
        if phase == "calibrate":
            per = max(1, int(per * target_s / max(secs, 1e-3)))
            if secs > 0.5 * target_s:
                break
    return dict({"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                 "sample": f"{case.name}: {len(sel)} output rows (h, k) of {len(groups)} groups "
                           f"(fp64 oracle, {secs:.1f} s)"}, **_host())


def cpu_baseline_quant(cases, target_s: float = 20.0):
    """Time the oracle's quantiser on a bounded sample of whole rows (every
    row costs what it costs in the full problem), in algorithmic GB/s."""
    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    case = cases[0]
    rows = 4096
    for phase in ("calibrate", "calibrate", "measure"):
        n = min(rows, case.M)
        x = case.x[:n].cpu()
        t0 = time.perf_counter()
        oracle.quant_fp8_reference(x, case.block)
        secs = time.perf_counter() - t0
        if phase == "calibrate":
            rows = max(1, int(n * target_s / max(secs, 1e-3)))
            if secs > 0.5 * target_s or n == case.M:
                break
    byts = n * case.K * 3 + n * (case.K // case.block) * 4
    return dict({"value": byts / secs / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
                 "sample": f"{case.name}: {n} of {case.M} rows (binary32 oracle, {secs:.1f} s)"}, **_host())


class ClockSampler:
    """Samples the shader clock and socket power with amd-smi (read-only
    queries) from a shell loop started as a child process before this
    process touches the GPU; the samples taken while the timed steps run
    are kept."""

    LOOP = "while true; do date +T%s.%N; amd-smi metric -c -p 2>/dev/null; sleep 0.2; done"

    def __init__(self):
        import shutil
        import subprocess
        import tempfile
        self.proc = None
        self.path = None
        # a profiler's preloaded library has initialised the GPU already: no
        # child process may be started from here then
        profiled = "rocprof" in os.environ.get("LD_PRELOAD", "") or any(
            k.startswith("ROCPROF") for k in os.environ)
        if profiled or shutil.which("amd-smi") is None:
            return
        fd, self.path = tempfile.mkstemp(prefix="bench_clock_", suffix=".txt")
        self.fh = os.fdopen(fd, "w")
        try:
            self.proc = subprocess.Popen(["bash", "-c", self.LOOP], stdout=self.fh, stderr=subprocess.DEVNULL)
        except OSError:
            self.fh.close()
            os.unlink(self.path)
            self.path = None

    def stop(self):
        if self.proc is not None and self.proc.poll() is None:
            self.proc.terminate()
            try:
                self.proc.wait(timeout=10)
            except Exception:
                self.proc.kill()
            self.fh.close()

    def summary(self, t0: float, t1: float):
        """Mean clock and power over samples stamped in [t0, t1] (epoch s)."""
        import re
        if self.path is None:
            return None
        with open(self.path) as fh:
            txt = fh.read()
        os.unlink(self.path)
        clk, pw = [], []
        # each reading follows a line "T<epoch seconds>"
        parts = re.split(r"^T(\d+\.\d+)\s*$", txt, flags=re.M)
        for stamp, block in zip(parts[1::2], parts[2::2]):
            ts = float(stamp)
            if not (t0 <= ts <= t1):
                continue
            # the graphics clock of each XCD (GFX_0 .. GFX_7); the listing
            # also holds memory, video and SoC clocks
            c = [int(x) for x in re.findall(r"GFX_\d+:\s*CLK:\s*(\d+) MHz", block)]
            p = re.findall(r"SOCKET_POWER:\s*(\d+) W", block)
            if c:
                clk.append(sum(c) / len(c))
            if p:
                pw.append(int(p[0]))
        if not clk:
            return None
        return {"sclk_mhz": round(statistics.mean(clk)), "samples": len(clk),
                "socket_power_w": round(statistics.mean(pw)) if pw else None}


def make_launcher(cases, dev, gmm_amd):
    """Outputs for each case and launch(i), which queues case i's call on
    the current stream."""
    import torch

    def out_of(c):
        if is_quant(c):
            return (torch.empty((c.M, c.K), dtype=torch.float8_e4m3fn, device=dev),
                    torch.empty((c.M, c.K // c.block), dtype=torch.float32, device=dev))
        shape = (c.num_active, c.K, c.N) if is_tgmm(c) else (c.M, c.N)
        return torch.empty(shape, dtype=c.out_dtype, device=dev)

    outs = [out_of(c) for c in cases]
    offs = [torch.tensor([c.group_offset], dtype=torch.int32, device=dev) if getattr(c, "group_offset", 0) else None
            for c in cases]

    def launch(i):
        c = cases[i]
        if is_quant(c):
            gmm_amd.quant_fp8(c.x, q=outs[i][0], scale=outs[i][1])
            return
        if is_tgmm(c):
            gmm_amd.tgmm(c.lhs, c.rhs, c.group_sizes, num_active=c.num_active, group_offset=offs[i], out=outs[i])
            return
        gmm_amd.gmm(c.lhs, c.rhs, c.group_sizes, rhs_scale=c.rhs_scale, rhs_bias=c.rhs_bias,
                    lhs_scale=c.lhs_scale, group_offset=offs[i], transpose_rhs=c.transpose_rhs,
                    out=outs[i])

    return launch, outs


class Evictor:
    """Reads 512 MB (twice the Infinity Cache) between timed calls, outside
    the events: a write would leave the caches full of dirty lines whose
    write-back the timed kernel then pays."""

    def __init__(self, dev):
        import torch
        self.scratch = torch.ones(512 << 18, dtype=torch.float32, device=dev)
        self.sink = torch.empty(1, dtype=torch.float32, device=dev)

    def __call__(self):
        import torch
        torch.sum(self.scratch, dim=0, keepdim=True, out=self.sink)


def time_steps(fns, steps: int, warmup: int, evict=None):
    """Run `steps` steps of the launches in fns (one after another) after
    `warmup` untimed ones, with a HIP event pair on the launch stream around
    every launch.  Returns (per-launch milliseconds [len(fns)][steps], wall
    seconds of the timed steps, epoch seconds at their start)."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
          for _ in range(steps)]
    torch.cuda.synchronize()
    epoch0 = time.time()
    t0 = time.perf_counter()
    for s in range(steps):
        for i, f in enumerate(fns):
            if evict is not None:
                evict()
            ev[s][i][0].record(stream)
            f()
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [[ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)] for i in range(len(fns))], wall, epoch0


def summarize(case, ms):
    """Median / p10 / p90 of one case's launch times and its rates: TFLOP/s
    and the fraction of the dtype's MFMA peak, algorithmic GB/s and the
    fraction of HBM peak."""
    med = statistics.median(ms)
    qs = statistics.quantiles(ms, n=10) if len(ms) > 1 else [med] * 9
    d = {"median_ms": med, "p10_ms": qs[0], "p90_ms": qs[-1], "launches": len(ms)}
    gbs = case.algorithmic_bytes() / (med * 1e-3) / 1e9
    if not is_quant(case):
        kind, pk = op_peak(case)
        tf = case.flops() / (med * 1e-3) / 1e12
        d.update({"tflops": tf, "peak_tflops": pk, "peak_dtype": kind, "frac_peak": tf / pk})
        if hasattr(case, "active_rows"):
            d["active_rows"] = case.active_rows()
    d.update({"gbs_algorithmic": gbs, "algorithmic_bytes": case.algorithmic_bytes(), "frac_hbm": gbs / HBM_PEAK_GBS})
    d["bound"] = "hbm" if case.name in MEM_BOUND else "mfma"
    return d


# workloads bound by HBM bandwidth (their roofline is bytes)
MEM_BOUND = {"decode_fp8w", "quant_fp8"}
# the other configurations, timed after the headline steps of a default run,
# each in its own protocol: (workload, timed calls, warm-up calls)
DETAIL_WORKLOADS = (("decode_fp8w", 500, 5), ("tiny_fp32", 500, 5), ("w8a8_fp8", 20, 3),
                    ("tgmm_bf16", 20, 3), ("quant_fp8", 20, 3))


def detail_workload(name, steps, warmup, dev, gmm_amd):
    import torch
    cases = build_cases(name, dev)
    launch, outs = make_launcher(cases, dev, gmm_amd)
    evict = Evictor(dev) if name in EVICT else None
    ms, _, _ = time_steps([lambda: launch(0)], steps, warmup, evict)
    if gmm_amd.device_flags() != 0:
        raise RuntimeError(f"{name}: device data flags set")
    d = summarize(cases[0], ms[0])
    d["evicted_caches"] = evict is not None
    d["traffic"] = measured_traffic(name)
    del cases, outs, evict
    torch.cuda.empty_cache()
    return d


def speed_gate(fwd, dlhs, steps, warmup, gmm_amd):
    """The transposed-RHS kernel's speed test on the MaxText PR page
    "Megablox: transposed-RHS gmm_v2 kernel for the backward dlhs" (Tests;
    Context: the wi and wo weight-transpose copies it removes): the backward
    dlhs reading the forward weight in place (NN) against an explicit
    transpose copy of the weight followed by the NT product on the copy, at
    the wi shape (the up-projection's weight [128,1408,1408]; the forward's
    activations stand in for its output gradient) and the wo shape (the
    down-projection's dlhs workload).  The copy is timed on its own."""
    import torch
    res = {}
    for tag, lhs, w, gs in (("wi", fwd.lhs, fwd.rhs, fwd.group_sizes), ("wo", dlhs.lhs, dlhs.rhs, dlhs.group_sizes)):
        # W as the forward stores it: the dlhs contracts its dim 1 (NN)
        M, Kc, Nc = lhs.shape[0], w.shape[1], w.shape[2]
        out_nn = torch.empty((M, Nc), dtype=torch.bfloat16, device=lhs.device)
        out_nt = torch.empty_like(out_nn)
        wt = torch.empty((w.shape[0], Nc, Kc), dtype=w.dtype, device=w.device)

        def nn():
            gmm_amd.gmm(lhs, w, gs, transpose_rhs=True, out=out_nn)

        def copy():
            wt.copy_(w.transpose(1, 2))

        def nt():
            gmm_amd.gmm(lhs, wt, gs, transpose_rhs=False, out=out_nt)

        ms, _, _ = time_steps([nn, copy, nt], steps, warmup)
        med = [statistics.median(x) for x in ms]
        torch.cuda.synchronize()
        res[tag] = {"weight": list(w.shape), "dlhs": [M, Nc],
                    "nn_in_place_ms": med[0], "transpose_copy_ms": med[1], "nt_on_copy_ms": med[2],
                    "copy_plus_nt_ms": med[1] + med[2], "speedup_vs_copy_plus_nt": (med[1] + med[2]) / med[0],
                    "copy_bytes": 2 * w.numel() * w.element_size(),
                    "copy_gbs": 2 * w.numel() * w.element_size() / (med[1] * 1e-3) / 1e9,
                    "nn_equals_nt_bitwise": bool(torch.equal(out_nn, out_nt))}
        del out_nn, out_nt, wt
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50; 500 for the microsecond-scale tiny_fp32 and decode_fp8w)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="fwd+dlhs",
                    help="fwd+dlhs (default) or one of tiny_fp32, moe_fwd_bf16, moe_dlhs_bf16, "
                         "decode_fp8w, w8a8_fp8, tgmm_bf16 (the weight gradient), "
                         "quant_fp8 (the activation quantiser)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail", action="store_true",
                    help="default workload only: skip the other configurations and the speed gate")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 500 if args.workload in ("tiny_fp32", "decode_fp8w") else 50

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    clock = ClockSampler()  # before the first GPU call: it starts a child process
    import atexit
    atexit.register(clock.stop)

    import torch

    import moe_grouped_matrix_amd as gmm_amd

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cases = build_cases(args.workload, dev)
    launch, outs = make_launcher(cases, dev, gmm_amd)
    fns = [(lambda i=i: launch(i)) for i in range(len(cases))]

    evict = Evictor(dev) if args.workload in EVICT else None
    per_kernel_ms, wall, epoch0 = time_steps(fns, args.steps, args.warmup, evict)
    if gmm_amd.device_flags() != 0:
        raise RuntimeError("device data flags set")
    # the timed steps are too short for the clock sampler (about one reading
    # a second): the same steps keep running, untimed, for a few seconds and
    # the readings over both spans describe the clock under this load
    epoch1 = time.time()
    if clock.proc is not None:
        while time.time() - epoch1 < 3.0:
            for f in fns:
                f()
            torch.cuda.synchronize()
        epoch1 = time.time()
    clock.stop()

    flops = [c.flops() for c in cases]
    step_flops = sum(flops)
    # with eviction between calls the wall clock includes the scratch reads:
    # the job's rate is then taken from the kernels' own event times
    gpu_s = sum(sum(x) for x in per_kernel_ms) * 1e-3
    quant = all(is_quant(c) for c in cases)
    if quant:  # an HBM-bound pass: its rate is bytes, not FLOPs
        step_bytes = sum(c.algorithmic_bytes() for c in cases)
        value = step_bytes * args.steps / (gpu_s if evict else wall) / 1e9
    else:
        value = step_flops * args.steps / (gpu_s if evict else wall) / 1e12

    # dominant kernel: the case with the largest total event time
    tot = [sum(x) for x in per_kernel_ms]
    d = max(range(len(cases)), key=lambda i: tot[i])
    dc = cases[d]
    avg_ms = statistics.mean(per_kernel_ms[d])
    kind, peak = op_peak(dc)
    if dc.name in MEM_BOUND:
        achieved = dc.algorithmic_bytes() / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        achieved = flops[d] / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak}
    roof["traffic"] = measured_traffic(dc.name)
    roof["kernel"] = dc.name
    roof["avg_launch_ms"] = avg_ms
    clk = clock.summary(epoch0, epoch1)
    if clk:
        # the chip runs below its 2.4 GHz peak clock when power-limited:
        # the fraction of the peak at the observed clock, for context
        clk["frac_of_peak_at_sclk"] = roof["frac"] * 2400.0 / clk["sclk_mhz"] if roof["bound"] == "mfma" else None
    roof["clock"] = clk

    detail = {c.name: summarize(c, per_kernel_ms[i]) for i, c in enumerate(cases)}
    if args.workload == "fwd+dlhs" and not args.no_detail:
        detail["p4_speed_gate"] = speed_gate(cases[0], cases[1], 20, 3, gmm_amd)

    if quant:
        metric = f"activation quantiser GB/s, {args.workload}"
    elif args.workload == "fwd+dlhs":
        metric = "grouped-GEMM TFLOP/s and % MFMA peak, 128-expert bf16 fwd+dlhs"
    else:
        metric = f"grouped-GEMM TFLOP/s, {args.workload}"

    def shape_of(c):
        if is_quant(c):
            return {"M": c.M, "K": c.K, "block": c.block, "op": "quant_fp8"}
        return {"M": c.M, "K": c.K, "N": c.N, "G": int(c.group_sizes.numel()), "Ga": c.num_active,
                "transpose_rhs": getattr(c, "transpose_rhs", None), "op": "tgmm" if is_tgmm(c) else "gmm"}

    if quant:
        dtype = "bf16 -> fp8-e4m3"
    elif any(c.rhs.dtype == torch.float8_e4m3fn and c.lhs.dtype == torch.bfloat16 for c in cases):
        dtype = "bf16 x fp8-e4m3"
    else:
        dtype = {"bf16": "bf16", "fp8": "fp8-e4m3", "f32": "f32"}[op_peak(cases[0])[0]]
    line = {
        "metric": metric,
        "value": value,
        "unit": "GB/s" if quant else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": (gpu_s if evict else wall) / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; normal values)" if quant else "synthetic (seeded; router group sizes, normal values)",
        "config": {"workload": " + ".join(c.name for c in cases),
                   "shapes": [shape_of(c) for c in cases],
                   "frac_of_peak": value / (HBM_PEAK_GBS if quant else PEAK[op_peak(cases[0])[0]])},
        "roofline": roof,
        "detail": detail,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cases)
    else:
        line["cpu_baseline"] = None
    if args.workload == "fwd+dlhs" and not args.no_detail:
        # the other configurations, after the headline's inputs are freed
        del cases, outs, fns, launch
        torch.cuda.empty_cache()
        for name, steps, warm in DETAIL_WORKLOADS:
            detail[name] = detail_workload(name, steps, warm, dev, gmm_amd)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
