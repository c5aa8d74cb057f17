#!/usr/bin/env python3
"""Benchmark of the SVDQuant W4A4 linear (and the W8A8 linear) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload mlp_up] [--no-cpu-baseline]

One step is one pass of the linear's device path over one batch: the fused
activation quantization (svdq_quantize_act: smoothing divide, group absmax,
INT4 codes, low-rank down-projection) followed by the W4A4 GEMM with its
fused low-rank up-projection and bias (svdq_w4a4_linear). The codes travel in
the FP6 container (gfx950's FP6 MFMA); the same step on the compact INT4
container (i8 MFMA) is timed beside it. Weights are prepared once beforehand
by the library's host preparation (and re-encoded by svdq_repack_codes) and
stay resident in HBM; inputs are resident before the timed region starts.

Prints ONE JSON line. `value` is TOPS counted as 2 M N K operations per step
over the whole step (both kernels). The roofline object describes the
dominant kernel (the GEMM) against the dense peak of the MFMA type it runs on
(FP6); "pct_int8_roofline" gives the same throughput against the int8 MFMA
peak. The W8A8 linear on the attention shape is timed the same way and
reported under "w8a8", and the MXFP4 variant of the W4A4 linear on the same
workload under "mxfp4". The W4A16 linear (the awq_w4a16 layer type) on an
adaLN-modulation shape is reported under "w4a16" with its own HBM roofline:
it is a skinny GEMM whose cost is one read of the packed weight. Its rate is
taken the way a model runs such layers, one per block with distinct weights:
a HIP graph of launches round-robin over 16 copies of the weight (twice the
last-level cache), replayed back to back between two HIP events.

HBM traffic of the GEMM comes from two rocprofv3 counter runs (FETCH_SIZE,
then WRITE_SIZE) of this script with --calibrate-copy --no-mlp --no-w8a8 (so
that each kernel runs at one shape), which adds a plain
elementwise kernel of known size (a negation, N bytes in, N bytes out) whose
counter readings give the scale from counter units to bytes:

    bench.py --summarize-pmc DIR_FETCH DIR_WRITE  > profiles/<summary>.txt

writes the summary that later runs read; it records a hash of the GEMM's
sources, and `traffic` is null once those sources have changed.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA, published
FP6_PEAK_TFLOPS = 10100.0  # MI355X dense FP6/FP4 MFMA, published
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published

METRIC = "W4A4+lowrank linear TOPS & % int8 MFMA roofline at M=4608,K=3072,N=12288"

CSRC = os.path.join(ROOT, "bit_quantized_linear_amd", "csrc")
GEMM_SOURCES = ("w4a4_fp6_gemm.hip", "device_common.h", "quant_common.h", "gelu.h")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "svdq_w4a4_linear_fp6_mlp_up_4608x3072x12288_traffic.txt")
COPY_BYTES = 256 << 20  # calibration kernel: reads and writes this many bytes
GEMM_KERNEL_KEY = "w4a4_fp6_kernel<0, 128>"
COPY_KERNEL_KEY = "neg_kernel"
W16_SOURCES = ("w4a16.hip", "device_common.h")
W16_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "w4a16_linear_modulation_2x3072x18432_traffic.txt")
W16_KERNEL_KEY = "w4a16_kernel"
MX_SOURCES = ("mx_gemm.hip", "device_common.h")
MX_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "svdq_mx_linear_mlp_up_4608x3072x12288_traffic.txt")
MX_KERNEL_KEY = "mx_linear_kernel"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="mlp_up")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-w8a8", action="store_true")
    p.add_argument("--no-mlp", action="store_true")
    p.add_argument("--no-w4a16", action="store_true")
    p.add_argument("--no-mx", action="store_true")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the attention-projection and video configurations")
    p.add_argument("--cpu-rows", type=int, default=4608,
                   help="token rows of the workload the CPU oracle is timed on")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain elementwise kernel of known size (for counter runs)")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="print the traffic summary from two rocprofv3 --pmc output folders (no GPU)")
    p.add_argument("--pmc-kernel", choices=("fp6_gemm", "w4a16", "mx_gemm"), default="fp6_gemm",
                   help="kernel whose traffic --summarize-pmc reports")
    p.add_argument("--summarize-trace", metavar="DIR",
                   help="print per-kernel durations from a rocprofv3 --kernel-trace output folder, one "
                        "line per kernel and grid shape")
    p.add_argument("--summarize-counters", nargs="+", metavar=("KERNEL", "DIR"),
                   help="print a summary of a kernel's SQ/TA/TD/TCC counters from rocprofv3 --pmc "
                        f"output folders; KERNEL is one of {', '.join(COUNTER_KERNELS)}")
    return p.parse_args()


def gemm_source_hash(sources=GEMM_SOURCES):
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _counter_means(folder, counter, kernel_key=GEMM_KERNEL_KEY):
    """Mean per-dispatch value of `counter` for the kernel and the calibration kernel."""
    vals = {"gemm": [], "copy": []}
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") != counter:
                    continue
                name = r.get("Kernel_Name", "")
                key = "gemm" if kernel_key in name else "copy" if COPY_KERNEL_KEY in name else None
                if key:
                    vals[key].append(float(r["Counter_Value"]))
    if not vals["gemm"] or not vals["copy"]:
        raise SystemExit(f"{folder}: no {counter} rows for both kernels")
    return {k: sum(v) / len(v) for k, v in vals.items()}


def summarize_pmc(fetch_dir, write_dir, which="fp6_gemm"):
    """Text summary of a kernel's HBM traffic per launch (printed to stdout)."""
    if which == "w4a16":
        key, sources = W16_KERNEL_KEY, W16_SOURCES
        M, K, N = 2, 3072, 18432
        algo = w4a16_bytes(M, K, N)
        title = f"# HBM traffic of w4a16_linear, modulation M={M} K={K} N={N}"
    elif which == "mx_gemm":
        key, sources = MX_KERNEL_KEY, MX_SOURCES
        M, K, N, r = 4608, 3072, 12288, 32
        algo = mx_gemm_bytes(M, N, K, r)
        title = f"# HBM traffic of svdq_mx_linear (MXFP4), mlp_up M={M} K={K} N={N} rank={r}"
    else:
        key, sources = GEMM_KERNEL_KEY, GEMM_SOURCES
        M, K, N, r = 4608, 3072, 12288, 32
        algo = algorithmic_gemm_bytes(M, N, K, r)
        title = f"# HBM traffic of svdq_w4a4_linear (FP6 container), mlp_up M={M} K={K} N={N} rank={r}"
    fe = _counter_means(fetch_dir, "FETCH_SIZE", key)
    wr = _counter_means(write_dir, "WRITE_SIZE", key)
    # the calibration kernel moves COPY_BYTES each way: counter units -> bytes
    f_scale = COPY_BYTES / fe["copy"]
    w_scale = COPY_BYTES / wr["copy"]
    fetch_b = fe["gemm"] * f_scale
    write_b = wr["gemm"] * w_scale
    lines = [
        title,
        f"kernel_source_sha256_16: {gemm_source_hash(sources)}",
        f"calibration: elementwise negation of {COPY_BYTES} bytes (reads and writes that many)",
        f"FETCH_SIZE kernel mean per dispatch (counter units): {fe['gemm']:.1f}",
        f"FETCH_SIZE calibration kernel (counter units): {fe['copy']:.1f}  -> {f_scale:.2f} bytes/unit",
        f"WRITE_SIZE kernel mean per dispatch (counter units): {wr['gemm']:.1f}",
        f"WRITE_SIZE calibration kernel (counter units): {wr['copy']:.1f}  -> {w_scale:.2f} bytes/unit",
        f"fetch_bytes_per_launch: {fetch_b:.0f}",
        f"write_bytes_per_launch: {write_b:.0f}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"algorithmic_bytes_per_launch: {algo}",
        f"traffic_over_algorithmic: {(fetch_b + write_b) / algo:.3f}",
    ]
    print("\n".join(lines))


# Kernels --summarize-counters knows: key in the kernel name, sources whose
# hash the summary records, the workload, and the MFMA operations one launch
# must perform (with the counter that counts them), or None.
COUNTER_KERNELS = {
    "fp6_gemm": (GEMM_KERNEL_KEY, GEMM_SOURCES,
                 "svdq_w4a4_linear (FP6 container), mlp_up M=4608 K=3072 N=12288 rank=32",
                 2 * 4608 * 3072 * 12288, "SQ_INSTS_VALU_MFMA_MOPS_F6F4"),
    "int4_gemm": ("w4a4_int4_kernel", ("w4a4_gemm.hip", "device_common.h"),
                  "svdq_w4a4_linear (INT4 container), mlp_up M=4608 K=3072 N=12288 rank=32",
                  2 * 4608 * 3072 * 12288, "SQ_INSTS_VALU_MFMA_MOPS_I8"),
    "act": ("quantize_act_kernel<1, 2>", ("act_quant.hip", "quant_common.h", "device_common.h"),
            "svdq_quantize_act (FP6 container), mlp_up M=4608 K=3072 rank=32", None, None),
    "mx_gemm": (MX_KERNEL_KEY, MX_SOURCES, "svdq_mx_linear (MXFP4), mlp_up M=4608 K=3072 N=12288 rank=32",
                2 * 4608 * 3072 * 12288, "SQ_INSTS_VALU_MFMA_MOPS_F6F4"),
    "w8a8_gemm": ("w8a8_gemm256_kernel", ("w8a8.hip", "device_common.h", "quant_common.h"),
                  "w8a8_linear GEMM, attention projection M=4608 K=3072 N=3072",
                  2 * 4608 * 3072 * 3072, "SQ_INSTS_VALU_MFMA_MOPS_I8"),
}
# grid sizes (work-items) of the workloads above where the kernel also runs
# at other shapes in the same bench run: the up-projection's 36 x 96 blocks of
# 256 threads; the activation pass's 72 blocks of 64 rows x 8 K parts of 256
# threads
COUNTER_GRIDS = {"fp6_gemm": 36 * 96 * 256, "act": 72 * 8 * 256}
XCDS, CUS, SIMDS = 8, 256, 1024  # MI355X


def _dispatch_counters(folder, key, grid=None):
    """{(folder, dispatch): {counter: value, "_ns": duration}} for the
    dispatches of the kernel whose name contains `key`, restricted to the
    given grid size (work-items) or else to the one that occurs most often
    (the workload named in the summary)."""
    rows = []
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += [r for r in csv.DictReader(fh) if key in r.get("Kernel_Name", "")]
    if not rows:
        raise SystemExit(f"{folder}: no dispatches of {key}")
    grids = {}
    for r in rows:
        grids[r["Grid_Size"]] = grids.get(r["Grid_Size"], 0) + 1
    grid = str(grid) if grid is not None else max(grids, key=grids.get)
    out = {}
    for r in rows:
        if r["Grid_Size"] != grid:
            continue
        d = out.setdefault((folder, r["Dispatch_Id"]), {"_ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out, grid


def summarize_counters(which, folders):
    """Text summary of one kernel's counters (printed to stdout): per-dispatch
    means of every counter in the folders (one rocprofv3 --pmc pass each) and
    the figures derived from them. Counter values are totals over the chip
    (rocprofv3 sums the per-XCD / per-SE instances); GRBM_GUI_ACTIVE counts
    the dispatch's cycles once per XCD, so its sum over the 8 XCDs is divided
    by 8. Busy fractions are of every SIMD's (or CU's) cycles over that span."""
    key, sources, workload, ops, mops_counter = COUNTER_KERNELS[which]
    lines = [f"# counters of {workload}", f"kernel_source_sha256_16: {gemm_source_hash(sources)}"]
    derived = []
    for folder in folders:
        disp, grid = _dispatch_counters(folder, key, COUNTER_GRIDS.get(which))
        names = sorted({c for d in disp.values() for c in d if c != "_ns"})
        mean = {c: sum(d.get(c, 0.0) for d in disp.values()) / len(disp) for c in names + ["_ns"]}
        lines.append(f"pass {os.path.basename(os.path.normpath(folder))}: {len(disp)} dispatches, grid size {grid}, "
                     f"{mean['_ns'] / 1e3:.1f} us per dispatch under collection")
        for c in names:
            lines.append(f"  {c}: {mean[c]:.0f}")
        cyc = mean.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
        if not cyc:
            continue
        lines.append(f"  kernel_cycles (GRBM_GUI_ACTIVE / {XCDS}): {cyc:.0f} "
                     f"({cyc / (mean['_ns'] * 1e-3):.0f} MHz over the collected duration)")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            b = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS
            derived.append(f"mfma_busy_cycles_per_simd: {b:.0f} (fraction of kernel_cycles {b / cyc:.3f})")
        if "SQ_ACTIVE_INST_VALU" in mean:
            b = 4 * mean["SQ_ACTIVE_INST_VALU"] / SIMDS
            derived.append(f"valu_busy_cycles_per_simd: {b:.0f} (fraction of kernel_cycles {b / cyc:.3f}; "
                           "SQ_ACTIVE_INST_VALU is in quad-cycles)")
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in mean:
            derived.append(f"mfma_valu_coexec_fraction: {mean['SQ_VALU_MFMA_COEXEC_CYCLES'] / (cyc * SIMDS):.3f}")
        if "SQ_WAVES" in mean and "SQ_INSTS_VALU" in mean:
            derived.append(f"valu_instructions_per_wave: {mean['SQ_INSTS_VALU'] / mean['SQ_WAVES']:.0f}")
        if "SQ_WAVES" in mean and "SQ_INSTS_MFMA" in mean:
            derived.append(f"mfma_instructions_per_wave: {mean['SQ_INSTS_MFMA'] / mean['SQ_WAVES']:.0f}")
        if "SQ_LDS_BANK_CONFLICT" in mean and "SQ_LDS_IDX_ACTIVE" in mean:
            c, a = mean["SQ_LDS_BANK_CONFLICT"], mean["SQ_LDS_IDX_ACTIVE"]
            derived.append(f"lds_bank_conflict_cycles_per_access_cycle: {c / max(a - c, 1.0):.3f}")
            derived.append(f"lds_bank_conflict_fraction_of_cu_cycles: {c / (cyc * CUS):.3f}")
        if mops_counter and mops_counter in mean and ops:
            done = mean[mops_counter] * 512
            derived.append(f"mfma_ops_counted: {done:.4g} (algorithmic {ops:.4g}, ratio {done / ops:.3f})")
        for c, unit in (("TA_TA_BUSY_sum", "ta"), ("TD_TD_BUSY_sum", "td")):
            if c in mean:
                derived.append(f"{unit}_busy_fraction: {mean[c] / (cyc * CUS):.3f}")
        if "TCC_HIT_sum" in mean and "TCC_MISS_sum" in mean:
            h, m = mean["TCC_HIT_sum"], mean["TCC_MISS_sum"]
            derived.append(f"l2_hit_rate: {h / max(h + m, 1.0):.3f}")
    print("\n".join(lines + ["derived:"] + ["  " + d for d in derived]))


def summarize_trace(folder):
    """Per-kernel durations from a kernel trace (printed to stdout): one line
    per kernel and grid shape (a kernel that runs at several shapes gets one
    line per shape), in order of first launch. The name is the kernel's
    without its namespaces and argument list."""
    groups = {}
    for f in glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"].replace("(anonymous namespace)::", "")
                name = name[5:] if name.startswith("void ") else name
                if name.endswith(")"):  # drop the argument list: the "(" matching the last ")"
                    depth, i = 0, len(name) - 1
                    while i >= 0:
                        depth += {")": 1, "(": -1}.get(name[i], 0)
                        if depth == 0:
                            break
                        i -= 1
                    name = name[:i]
                name = name.replace("svdq::", "").replace("at::native::", "")
                shape = "x".join(r[f"Grid_Size_{a}"] for a in "XYZ") + "/" + r["Workgroup_Size_X"]
                g = groups.setdefault((name, shape), {"first": int(r["Dispatch_Id"]), "us": []})
                g["first"] = min(g["first"], int(r["Dispatch_Id"]))
                g["us"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if not groups:
        raise SystemExit(f"{folder}: no kernel trace")
    print(f"{'kernel':58s} {'grid/block':>20s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}")
    for (name, shape), g in sorted(groups.items(), key=lambda kv: kv[1]["first"]):
        us = g["us"]
        print(f"{name[:58]:58s} {shape:>20s} {len(us):6d} {sum(us) / len(us):9.1f} {min(us):9.1f} {max(us):9.1f}")


def w4a16_bytes(M, K, N):
    """Bytes the W4A16 linear must move at least once: the packed weight
    container (codes and scales, padded to whole 32-column units), bf16 X,
    bias and Y."""
    cpairs, pairs = (N + 31) // 32, (K // 64 + 1) // 2
    return cpairs * pairs * 2304 + M * K * 2 + N * 2 + M * N * 2


def read_traffic_summary(path=TRAFFIC_SUMMARY, sources=GEMM_SOURCES):
    """(traffic bytes per launch, details) from a committed summary, or
    (None, reason) when it is missing or the kernel's sources changed since."""
    if not os.path.exists(path):
        return None, "no counter summary"
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != gemm_source_hash(sources):
        return None, "kernel changed since the counters were taken"
    return float(kv["traffic_bytes_per_launch"]), {
        "fetch_bytes": float(kv["fetch_bytes_per_launch"]), "write_bytes": float(kv["write_bytes_per_launch"]),
        "source": os.path.relpath(path, ROOT)}


def algorithmic_gemm_bytes(M, N, K, r):
    """Bytes the GEMM must move at least once: both FP6 code matrices (3/4
    byte per code), both scale matrices, T and L2 (bf16), bias, bf16 Y."""
    return (M + N) * (K // 4 * 3) + (K // 64) * (M + N) * 4 + (M + N) * r * 2 + N * 2 + M * N * 2


def mx_gemm_bytes(M, N, K, r):
    """The same for the MXFP4 linear: E2M1 codes (1/2 byte each), E8M0 block
    scales (one byte per 32 codes), T, L2, bias and bf16 Y."""
    return (M + N) * (K // 2) + (K // 32) * (M + N) + (M + N) * r * 2 + N * 2 + M * N * 2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def time_steps(fns, steps, warmup):
    """Run `fns` in order per step; returns (ms_per_step, [ms per fn per step],
    wall ms per step, [ms of each step]).

    The whole timed region is bracketed by a device synchronize on both sides;
    HIP events recorded between the launches on the same stream give each
    kernel's average duration inside the timed region."""
    import torch

    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for s in range(steps):
        ev[s][0].record()
        for i, f in enumerate(fns):
            f()
            ev[s][i + 1].record()
    end.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    total = start.elapsed_time(end) / steps
    per = [sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps for i in range(len(fns))]
    each = [ev[s][0].elapsed_time(ev[s][-1]) for s in range(steps)]
    return total, per, wall, each


def time_cold(fns, reps):
    """Per-step ms with the 256 MB last-level cache flushed before each step
    by writing a 1 GiB buffer (untimed); returns the list of step times."""
    import torch

    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    out = []
    for _ in range(reps):
        flush.fill_(1.0)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for f in fns:
            f()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    del flush
    return out


def cpu_baseline(case, X, W, bias, rows):
    """The oracle, untuned, on a bounded sample: the first `rows` token rows of
    the same workload (same K, N, rank). Preparation is untimed and skips the
    SVD (the timed forward's cost does not depend on the factors' values)."""
    from oracle import svdquant as sq

    K, N, r = case.K, case.N, case.rank
    Wv = W["values"]
    a = sq.channel_absmax(X["values"][:rows])
    s = sq.smoothing_factors(a, Wv)
    rng = np.random.default_rng(0)
    L1s = sq.bf16_round(rng.standard_normal((K, r)) * 1e-2)
    L2 = sq.bf16_round(rng.standard_normal((r, N)) * 1e-2)
    prep = sq.prepare_from_factors(Wv, s, L1s, L2)
    Xs = X["values"][:rows]
    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        blas_threads = None
    # repeated until about 10 s of CPU work have been timed (at most 5 passes)
    reps, t0 = 0, time.perf_counter()
    while True:
        sq.forward(Xs, prep, bias["values"], "bf16")
        reps += 1
        if time.perf_counter() - t0 >= 10.0 or reps == 5:
            break
    dt = (time.perf_counter() - t0) / reps
    ops = 2.0 * rows * N * K
    cores = len(os.sched_getaffinity(0))
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": blas_threads or cores,
            "host_cores": cores, "kind": "oracle", "seconds": dt, "passes": reps,
            "sample": f"oracle forward (numpy fp64: quantize, per-group exact dgemms, scales, "
                      f"low-rank, bias) on the first {rows} of {case.M} token rows, K={K}, N={N}, r={r}; "
                      f"mean of {reps} passes"}


def cpu_baseline_w8a8(case, X, W, bias):
    """The W8A8 oracle, untuned, on the whole W8A8 workload (quantize X, exact
    fp64 product of the codes, scale, bias, bf16), repeated until about 3 s."""
    from oracle import w8a8 as o8

    qw, sw = o8.prepare_weights(W["values"])
    reps, t0 = 0, time.perf_counter()
    while True:
        o8.forward(X["values"], qw, sw, bias["values"])
        reps += 1
        if time.perf_counter() - t0 >= 3.0 or reps == 5:
            break
    dt = (time.perf_counter() - t0) / reps
    ops = 2.0 * case.M * case.N * case.K
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle", "seconds": dt, "passes": reps,
            "sample": f"oracle W8A8 forward on the whole workload M={case.M} K={case.K} N={case.N}"}


def time_cold_read_flush(fn, reps):
    """Per-launch ms of `fn` with the caches flushed by reading 1 GiB right
    before (no synchronize in between: the read keeps the stream busy while
    the events and the launch are enqueued)."""
    import torch

    big = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    out = []
    for _ in range(reps):
        torch.cuda.synchronize()
        big.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    del big
    return out


def cpu_baseline_w4a16(case, X, W, bias):
    """The W4A16 oracle, untuned, on the whole workload (quantize W, dequantize,
    fp64 product, bias, bf16), the forward repeated until about 3 s."""
    from oracle import w4a16 as o16

    qw, sw = o16.prepare_weights(W["values"])
    reps, t0 = 0, time.perf_counter()
    while True:
        o16.forward(X["values"], qw, sw, bias["values"])
        reps += 1
        if time.perf_counter() - t0 >= 3.0 or reps == 20:
            break
    dt = (time.perf_counter() - t0) / reps
    nbytes = case.K * case.N // 2 + case.K // 64 * case.N * 4
    return {"value": nbytes / dt / 1e9, "unit": "GB/s of packed weight", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle", "seconds": dt, "passes": reps,
            "sample": f"oracle W4A16 forward (dequantize + fp64 matmul + bias + bf16) on the whole workload "
                      f"M={case.M} K={case.K} N={case.N}"}


def w4a4_config_line(name, steps, warmup):
    """One SVDQuant W4A4 step (activation pass with its workspace + FP6 GEMM)
    on another configuration of the same layer type, with the library's own
    preparation: time, TOPS, % of the int8 and FP6 peaks, activation GB/s."""
    import torch

    from bit_quantized_linear_amd import binding as b
    from bit_quantized_linear_amd import workloads as wl

    case = wl.CASES[name]
    M, K, N, r = case.M, case.K, case.N, case.rank
    X, W, bias = wl.activations(case), wl.weight(case), wl.bias(case)
    Xd = torch.from_numpy(X["bits"].view(np.int16)).cuda()
    amax = torch.zeros(K, dtype=torch.float32, device="cuda")
    b.svdq_channel_absmax(Xd, amax)
    prep = b.svdq_prepare_weights(W["bits"], amax.cpu().numpy(), r)

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()

    s_d, l1_d, l2_d, sw_d, b_d = up(prep["s"]), up(prep["l1t"]), up(prep["l2t"]), up(prep["sw"]), up(bias["bits"])
    qw6 = up(b.svdq_repack_codes(prep["qw"], K, b.QFMT_FP6))
    qx6 = torch.empty((M, b.svdq_qrow_bytes(K, b.QFMT_FP6)), dtype=torch.uint8, device="cuda")
    sx = torch.empty((K // 64, M), dtype=torch.float32, device="cuda")
    T = torch.empty((M, r), dtype=torch.int16, device="cuda")
    Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    ws = torch.empty(max(16, b.svdq_act_workspace_bytes(M, K, r)), dtype=torch.uint8, device="cuda")

    def act():
        b.svdq_quantize_act(Xd, s_d, l1_d, qx6, sx, T, r, qfmt=b.QFMT_FP6, workspace=ws)

    def gemm():
        b.svdq_w4a4_linear(qx6, sx, T, qw6, sw_d, l2_d, b_d, Y, M, N, K, r, qfmt=b.QFMT_FP6)

    ms, per, _, each = time_steps([act, gemm], steps, warmup)
    ops = 2.0 * M * N * K
    tops, gemm_tops = ops / (ms * 1e-3) / 1e12, ops / (per[1] * 1e-3) / 1e12
    act_bytes = M * K * 2 + r * K * 2 + K * 4 + M * (K // 4 * 3) + (K // 64) * M * 4 + M * r * 2
    finite = bool(torch.isfinite(Y.view(torch.bfloat16).float()).all().item())
    log(f"[bench] {name}: step {ms:.4f} ms (act {per[0]:.4f} ms, gemm {per[1]:.4f} ms) -> {tops:.1f} TOPS")
    return {"workload": f"{name}: SVDQuant W4A4 linear M={M} K={K} N={N} rank={r} group=64, FP6 container",
            "ms_per_step": round(ms, 5), "step_ms_median": round(float(np.median(each)), 5),
            "TOPS": round(tops, 2), "pct_int8_roofline": round(100.0 * tops / INT8_PEAK_TOPS, 2),
            "act_ms": round(per[0], 5), "act_GB/s": round(act_bytes / (per[0] * 1e-3) / 1e9, 1),
            "act_frac_hbm": round(act_bytes / (per[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "gemm_ms": round(per[1], 5), "gemm_TOPS": round(gemm_tops, 2),
            "gemm_pct_int8_roofline": round(100.0 * gemm_tops / INT8_PEAK_TOPS, 2),
            "gemm_frac_fp6_peak": round(gemm_tops / FP6_PEAK_TFLOPS, 4), "outputs_finite": finite}


def library_int8_gemm_ms(M, K, N, steps, warmup):
    """Time per call of the library int8 GEMM (torch._int_mm, hipBLASLt on
    this platform) on the same shape and operand layout as the W8A8 GEMM
    (codes [M, K] row-major times the weight codes [N, K] row-major, i.e.
    their transpose as a view), or None where it is not available. Context
    for the W8A8 GEMM's time, not part of any step."""
    import torch

    try:
        g = torch.Generator(device="cuda").manual_seed(7)
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
        w = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
        ms, _, _, _ = time_steps([lambda: torch._int_mm(a, w.t())], steps, warmup)
        return round(ms, 5)
    except (RuntimeError, AttributeError):
        return None


def w8a8_config_line(name, steps, warmup):
    """The W8A8 tensorwise linear on a configuration (library preparation)."""
    import torch

    from bit_quantized_linear_amd import binding as b
    from bit_quantized_linear_amd import workloads as wl

    c8 = wl.CASES[name]
    X8, W8, b8 = wl.activations(c8), wl.weight(c8), wl.bias(c8)
    qw8, sw8 = b.w8a8_prepare_weights(W8["bits"])

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()

    X8d, qw8d, b8d = up(X8["bits"]), up(qw8), up(b8["bits"])
    ws = torch.empty(b.w8a8_workspace_bytes(c8.M, c8.K), dtype=torch.uint8, device="cuda")
    Y8 = torch.empty((c8.M, c8.N), dtype=torch.int16, device="cuda")

    def w8():
        b.w8a8_linear(X8d, qw8d, sw8, b8d, ws, Y8)

    ms8, _, _, each = time_steps([w8], steps, warmup)
    ops8 = 2.0 * c8.M * c8.N * c8.K
    lib = library_int8_gemm_ms(c8.M, c8.K, c8.N, steps, warmup)
    log(f"[bench] {name}: {ms8:.4f} ms (library int8 GEMM alone on the same shape: {lib} ms)")
    return {"workload": f"{name}: W8A8 tensorwise M={c8.M} K={c8.K} N={c8.N}",
            "ms": round(ms8, 5), "step_ms_median": round(float(np.median(each)), 5),
            "TOPS": round(ops8 / (ms8 * 1e-3) / 1e12, 2),
            "pct_int8_roofline": round(100.0 * ops8 / (ms8 * 1e-3) / 1e12 / INT8_PEAK_TOPS, 2),
            "library_int8_gemm_ms": lib}


def measured_peaks():
    """This chip's matrix-core rates under load (back-to-back MFMAs on every
    SIMD: FP6 32x32x64, int8 32x32x32, bf16 32x32x16), the shader clock under
    that load, and the HBM copy bandwidth (a 1 GiB device-to-device copy, read
    plus write bytes)."""
    import torch

    from bit_quantized_linear_amd import binding as b

    blocks, iters = 4 * 256, 2000
    out = torch.empty(8 * blocks, dtype=torch.int64, device="cuda")
    res = {}
    for kind, name in ((0, "fp6"), (1, "int8"), (2, "bf16")):
        b.svdq_debug_mfma_rate(kind, blocks, 50, out)  # warm-up
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.svdq_debug_mfma_rate(kind, blocks, iters, out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        spans = out.view(-1, 2).cpu().numpy().astype(np.float64)
        clock_mhz = float(np.median(spans[:, 0] / spans[:, 1]) * 100.0)
        res[name] = {"TOPS": round(b.svdq_debug_mfma_ops(kind, blocks, iters) / (ms * 1e-3) / 1e12, 1),
                     "shader_clock_MHz": round(clock_mhz, 0)}
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    res["hbm_copy_GB/s"] = round(2 * src.numel() * 4 / (ms * 1e-3) / 1e9, 1)
    del src, dst
    log(f"[bench] measured: fp6 {res['fp6']['TOPS']} TOPS, int8 {res['int8']['TOPS']} TOPS, "
        f"bf16 {res['bf16']['TOPS']} TFLOPS at {res['fp6']['shader_clock_MHz']} MHz; "
        f"HBM copy {res['hbm_copy_GB/s']} GB/s")
    return res


def cpu_baseline_one_core(case, X, W, bias, rows):
    """The same oracle forward with its BLAS limited to one thread, on a
    smaller sample of the same workload (`rows` token rows)."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # noqa: BLE001
        return None
    with threadpool_limits(limits=1):
        res = cpu_baseline(case, X, W, bias, rows)
    res["cores"] = 1
    return res


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, which=args.pmc_kernel)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        if len(args.summarize_counters) < 2 or args.summarize_counters[0] not in COUNTER_KERNELS:
            raise SystemExit(f"--summarize-counters KERNEL DIR [DIR ...], KERNEL one of {', '.join(COUNTER_KERNELS)}")
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1:])
        return
    if args.gpus != 1:
        print(json.dumps({"error": f"--gpus {args.gpus}: this benchmark runs on one GPU only "
                                   "(--gpus must be 1); there is no multi-GPU path"}))
        sys.exit(2)
    import torch

    from bit_quantized_linear_amd import binding as b
    from bit_quantized_linear_amd import workloads as wl

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.cuda.current_device()
    st = b.svdq_check_device(dev)
    if st != b.SVDQ_OK:
        print(json.dumps({"error": f"device check failed: {b.status_string(st)}"}))
        sys.exit(1)

    case = wl.CASES[args.workload]
    M, K, N, r = case.M, case.K, case.N, case.rank
    log(f"[bench] workload {case.name}: M={M} K={K} N={N} rank={r}")
    X = wl.activations(case)
    W = wl.weight(case)
    bias = wl.bias(case)

    # calibration statistic on the device, preparation on the host (library)
    t0 = time.perf_counter()
    Xd = torch.from_numpy(X["bits"].view(np.int16)).cuda()
    amax = torch.zeros(K, dtype=torch.float32, device="cuda")
    b.svdq_channel_absmax(Xd, amax)
    torch.cuda.synchronize()
    amax_h = amax.cpu().numpy()
    t1 = time.perf_counter()
    prep = b.svdq_prepare_weights(W["bits"], amax_h, r)
    prep_s = time.perf_counter() - t1
    log(f"[bench] host prepare {prep_s:.1f}s (calibration + prepare {time.perf_counter() - t0:.1f}s)")

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).cuda()

    s_d, l1_d, l2_d = up(prep["s"]), up(prep["l1t"]), up(prep["l2t"])
    qw_d, sw_d, b_d = up(prep["qw"]), up(prep["sw"]), up(bias["bits"])
    qw6_d = up(b.svdq_repack_codes(prep["qw"], K, b.QFMT_FP6))
    qx = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    qx6 = torch.empty((M, b.svdq_qrow_bytes(K, b.QFMT_FP6)), dtype=torch.uint8, device="cuda")
    sx = torch.empty((K // 64, M), dtype=torch.float32, device="cuda")
    T = torch.empty((M, r), dtype=torch.int16, device="cuda")
    Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    # the activation pass's workspace: K split across blocks at this batch
    act_ws = torch.empty(max(16, b.svdq_act_workspace_bytes(M, K, r)), dtype=torch.uint8, device="cuda")

    def act6():
        b.svdq_quantize_act(Xd, s_d, l1_d, qx6, sx, T, r, qfmt=b.QFMT_FP6, workspace=act_ws)

    def gemm6():
        b.svdq_w4a4_linear(qx6, sx, T, qw6_d, sw_d, l2_d, b_d, Y, M, N, K, r, qfmt=b.QFMT_FP6)

    def act4():
        b.svdq_quantize_act(Xd, s_d, l1_d, qx, sx, T, r, qfmt=b.QFMT_INT4, workspace=act_ws)

    def gemm4():
        b.svdq_w4a4_linear(qx, sx, T, qw_d, sw_d, l2_d, b_d, Y, M, N, K, r, qfmt=b.QFMT_INT4)

    ms4, per4, _, _ = time_steps([act4, gemm4], args.steps, args.warmup)
    log(f"[bench] int4 container: step {ms4:.4f} ms (act {per4[0]:.4f} ms, gemm {per4[1]:.4f} ms)")
    ms, per, wall, each = time_steps([act6, gemm6], args.steps, args.warmup)
    cold = time_cold([act6, gemm6], max(5, min(args.steps, 20)))
    ops = 2.0 * M * N * K
    tops = ops / (ms * 1e-3) / 1e12
    gemm_tops = ops / (per[1] * 1e-3) / 1e12
    act_bytes = M * K * 2 + r * K * 2 + K * 4 + M * (K // 4 * 3) + (K // 64) * M * 4 + M * r * 2
    act_gbs = act_bytes / (per[0] * 1e-3) / 1e9
    y_finite = bool(torch.isfinite(Y.view(torch.bfloat16).float()).all().item())
    log(f"[bench] step {ms:.4f} ms (act {per[0]:.4f} ms, gemm {per[1]:.4f} ms) -> {tops:.1f} TOPS")
    traffic, traffic_detail = read_traffic_summary()
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()

    out = {
        "metric": METRIC,
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4",
        "dtype_detail": "int4 x int4 codes multiplied exactly on the FP6 MFMA, fp32 group scaling and "
                        "accumulation, bf16 low-rank branch, bf16 output",
        "data": "synthetic (seeded N(0,1) activations with outlier channels, N(0,0.02) weights "
                "with heavy columns, random init; no checkpoint)",
        "config": {"workload": f"{case.name}: SVDQuant W4A4 linear M={M} K={K} N={N} rank={r} group=64",
                   "M": M, "K": K, "N": N, "rank": r, "group": 64, "parallelism": "single GPU"},
        "pct_int8_roofline": round(100.0 * tops / INT8_PEAK_TOPS, 2),
        "kernels": {
            "svdq_quantize_act": {"ms": round(per[0], 5), "GB/s": round(act_gbs, 1),
                                  "frac_hbm": round(act_gbs / HBM_PEAK_GBS, 4),
                                  "algorithmic_bytes": act_bytes},
            "svdq_w4a4_linear": {"ms": round(per[1], 5), "TOPS": round(gemm_tops, 2),
                                 "pct_int8_roofline": round(100.0 * gemm_tops / INT8_PEAK_TOPS, 2)},
        },
        "int4_container": {"ms_per_step": round(ms4, 5), "TOPS": round(ops / (ms4 * 1e-3) / 1e12, 2),
                           "act_ms": round(per4[0], 5), "gemm_ms": round(per4[1], 5),
                           "gemm_TOPS": round(ops / (per4[1] * 1e-3) / 1e12, 2),
                           "gemm_pct_int8_roofline": round(100.0 * ops / (per4[1] * 1e-3) / 1e12 / INT8_PEAK_TOPS, 2)},
        "roofline": {"bound": "mfma", "kernel": "svdq_w4a4_linear (FP6 container)", "mfma_dtype": "fp6",
                     "achieved": round(gemm_tops, 2), "peak": FP6_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tops / FP6_PEAK_TFLOPS, 4), "traffic": traffic,
                     "traffic_detail": traffic_detail,
                     "algorithmic_bytes": algorithmic_gemm_bytes(M, N, K, r),
                     "algorithmic_ops": ops},
        "wall_ms_per_step": round(wall, 5),
        "step_ms_median": round(float(np.median(each)), 5),
        "step_ms_min": round(float(np.min(each)), 5),
        "cold_step_ms_median": round(float(np.median(cold)), 5),
        "cold_step_ms_min": round(float(np.min(cold)), 5),
        "outputs_finite": y_finite,
    }

    if not args.no_mx:
        # the MXFP4 variant on the same workload and the same smoothing and
        # low-rank factors: E2M1 codes with E8M0 block-32 scales
        t1 = time.perf_counter()
        mxw = b.svdq_mx_prepare_residual(W["bits"], prep["s"], prep["l1t"], prep["l2t"])
        mx_prep_s = time.perf_counter() - t1
        mqw, muw = up(mxw["qw"]), up(mxw["uw"])
        mqx = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
        mux = torch.empty((K // 32, b.svdq_mx_scale_ld(M)), dtype=torch.uint8, device="cuda")

        def actmx():
            b.svdq_mx_quantize_act(Xd, s_d, l1_d, mqx, mux, T, r, workspace=act_ws)

        def gemmmx():
            b.svdq_mx_linear(mqx, mux, T, mqw, muw, l2_d, b_d, Y, M, N, K, r)

        msmx, permx, _, eachmx = time_steps([actmx, gemmmx], args.steps, args.warmup)
        mx_tops = ops / (msmx * 1e-3) / 1e12
        mx_gemm_tops = ops / (permx[1] * 1e-3) / 1e12
        traffic_mx, traffic_mx_detail = read_traffic_summary(MX_TRAFFIC_SUMMARY, MX_SOURCES)
        out["mxfp4"] = {
            "workload": f"{case.name}: SVDQuant W4A4 linear, MXFP4 variant (E2M1, E8M0 per 32 along K), "
                        f"M={M} K={K} N={N} rank={r}",
            "ms_per_step": round(msmx, 5), "TOPS": round(mx_tops, 2),
            "pct_int8_roofline": round(100.0 * mx_tops / INT8_PEAK_TOPS, 2),
            "step_ms_median": round(float(np.median(eachmx)), 5),
            "act_ms": round(permx[0], 5), "gemm_ms": round(permx[1], 5),
            "roofline": {"bound": "mfma", "kernel": "svdq_mx_linear", "mfma_dtype": "fp4",
                         "achieved": round(mx_gemm_tops, 2), "peak": FP6_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(mx_gemm_tops / FP6_PEAK_TFLOPS, 4), "traffic": traffic_mx,
                         "traffic_detail": traffic_mx_detail, "algorithmic_ops": ops,
                         "algorithmic_bytes": mx_gemm_bytes(M, N, K, r)},
            "prepare_residual_library_s": round(mx_prep_s, 3),
        }
        log(f"[bench] mxfp4: step {msmx:.4f} ms (act {permx[0]:.4f} ms, gemm {permx[1]:.4f} ms) "
            f"-> {mx_tops:.1f} TOPS")

    if not args.no_mlp:
        # the whole MLP of the workload: up-projection, GELU, down-projection
        # (12288 -> 3072), unfused (GELU as its own pass, the down-projection's
        # activation pass reading GELU(y_up)) and fused (the up-projection's
        # epilogue emits the down-projection's codes, scales and T)
        cd = wl.MLP_DOWN
        Nd, Kd, rd = cd.N, cd.K, cd.rank
        Wd, bd = wl.mlp_down_weight(), wl.mlp_down_bias()
        gemm6()
        G = torch.empty_like(Y)
        b.svdq_debug_gelu_bf16(Y, G)
        amax_d = torch.zeros(Kd, dtype=torch.float32, device="cuda")
        b.svdq_channel_absmax(G, amax_d)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        prep_d = b.svdq_prepare_weights(Wd["bits"], amax_d.cpu().numpy(), rd)
        mlp_prep_s = time.perf_counter() - t1
        sd_d, l1d_d, l2d_d, bd_d = up(prep_d["s"]), up(prep_d["l1t"]), up(prep_d["l2t"]), up(bd["bits"])
        qwd6 = up(b.svdq_repack_codes(prep_d["qw"], Kd, b.QFMT_FP6))
        swd = up(prep_d["sw"])
        qxd = torch.empty((M, b.svdq_qrow_bytes(Kd, b.QFMT_FP6)), dtype=torch.uint8, device="cuda")
        sxd = torch.empty((Kd // 64, M), dtype=torch.float32, device="cuda")
        Td = torch.empty((M, rd), dtype=torch.int16, device="cuda")
        Yd = torch.empty((M, Nd), dtype=torch.int16, device="cuda")
        ws = torch.empty(b.svdq_mlp_workspace_bytes(M, Kd, rd), dtype=torch.uint8, device="cuda")
        act_ws_d = torch.empty(max(16, b.svdq_act_workspace_bytes(M, Kd, rd)), dtype=torch.uint8, device="cuda")

        def gelu():
            b.svdq_debug_gelu_bf16(Y, G)

        def act_d():
            b.svdq_quantize_act(G, sd_d, l1d_d, qxd, sxd, Td, rd, qfmt=b.QFMT_FP6, workspace=act_ws_d)

        def fused():
            b.svdq_w4a4_linear_gelu_quantize(qx6, sx, T, qw6_d, sw_d, l2_d, b_d, M, N, K, r, sd_d, l1d_d, rd,
                                             qxd, sxd, Td, None, ws)

        def gemm_d():
            b.svdq_w4a4_linear(qxd, sxd, Td, qwd6, swd, l2d_d, bd_d, Yd, M, Nd, Kd, rd, qfmt=b.QFMT_FP6)

        ms_u, per_u, _, _ = time_steps([act6, gemm6, gelu, act_d, gemm_d], args.steps, args.warmup)
        ms_f, per_f, _, each_f = time_steps([act6, fused, gemm_d], args.steps, args.warmup)
        ops2 = 2.0 * ops
        out["mlp_pair"] = {
            "workload": f"MLP of the {case.name} workload: up M={M} K={K} N={N}, GELU, down K={Kd} N={Nd}, "
                        f"ranks {r}/{rd}, FP6 container",
            "fused_ms": round(ms_f, 5), "fused_TOPS": round(ops2 / (ms_f * 1e-3) / 1e12, 2),
            "fused_step_ms_median": round(float(np.median(each_f)), 5),
            "fused_parts_ms": {"act_up": round(per_f[0], 5), "up_gelu_quantize": round(per_f[1], 5),
                               "down_linear": round(per_f[2], 5)},
            "unfused_ms": round(ms_u, 5), "unfused_TOPS": round(ops2 / (ms_u * 1e-3) / 1e12, 2),
            "unfused_parts_ms": {"act_up": round(per_u[0], 5), "up_linear": round(per_u[1], 5),
                                 "gelu": round(per_u[2], 5), "act_down": round(per_u[3], 5),
                                 "down_linear": round(per_u[4], 5)},
            "speedup": round(ms_u / ms_f, 3),
            "prepare_down_library_s": round(mlp_prep_s, 2),
        }
        log(f"[bench] mlp pair: fused {ms_f:.4f} ms (up+gelu+quant {per_f[1]:.4f}), unfused {ms_u:.4f} ms "
            f"(up {per_u[1]:.4f}, gelu {per_u[2]:.4f}, act_down {per_u[3]:.4f}, down {per_u[4]:.4f})")

    if not args.no_w8a8:
        c8 = wl.CASES["w8a8_attn"]
        X8 = wl.activations(c8)
        W8 = wl.weight(c8)
        b8 = wl.bias(c8)
        qw8, sw8 = b.w8a8_prepare_weights(W8["bits"])
        X8d, qw8d, b8d = up(X8["bits"]), up(qw8), up(b8["bits"])
        ws = torch.empty(b.w8a8_workspace_bytes(c8.M, c8.K), dtype=torch.uint8, device="cuda")
        Y8 = torch.empty((c8.M, c8.N), dtype=torch.int16, device="cuda")

        def w8():
            b.w8a8_linear(X8d, qw8d, sw8, b8d, ws, Y8)

        ms8, _, _, _ = time_steps([w8], args.steps, args.warmup)
        ops8 = 2.0 * c8.M * c8.N * c8.K
        lib8 = library_int8_gemm_ms(c8.M, c8.K, c8.N, args.steps, args.warmup)
        out["w8a8"] = {"workload": f"W8A8 tensorwise M={c8.M} K={c8.K} N={c8.N}",
                       "ms": round(ms8, 5), "TOPS": round(ops8 / (ms8 * 1e-3) / 1e12, 2),
                       "pct_int8_roofline": round(100.0 * ops8 / (ms8 * 1e-3) / 1e12 / INT8_PEAK_TOPS, 2),
                       "library_int8_gemm_ms": lib8}
        log(f"[bench] w8a8 {ms8:.4f} ms (library int8 GEMM alone on the same shape: {lib8} ms)")
        if not args.no_cpu_baseline:
            out["w8a8"]["cpu_baseline"] = cpu_baseline_w8a8(c8, X8, W8, b8)
            log(f"[bench] w8a8 cpu baseline {out['w8a8']['cpu_baseline']['seconds']:.1f}s")

    if not args.no_configs:
        # the other configurations of the same layer types: the attention
        # projection (4608 x 3072 -> 3072) and the video-scale linear (32760 x
        # 5120 -> 5120, its row tail included), W4A4 and W8A8
        out["attn_proj"] = w4a4_config_line("attn_proj", args.steps, args.warmup)
        out["video"] = w4a4_config_line("video", max(5, args.steps // 4), max(2, args.warmup // 2))
        out["video_w8a8"] = w8a8_config_line("video_w8a8", max(5, args.steps // 4), max(2, args.warmup // 2))
        torch.cuda.empty_cache()

    if not args.no_w4a16:
        c16 = wl.CASES["modulation"]
        X16 = wl.activations(c16)
        W16 = wl.weight(c16)
        b16 = wl.bias(c16)
        t1 = time.perf_counter()
        packed16 = b.w4a16_prepare_weights(W16["bits"])
        prep16_s = time.perf_counter() - t1
        X16d, p16d, b16d = up(X16["bits"]), up(packed16), up(b16["bits"])
        Y16 = torch.empty((c16.M, c16.N), dtype=torch.int16, device="cuda")

        def w16():
            b.w4a16_linear(X16d, p16d, b16d, Y16, c16.N)

        ms16, _, _, _ = time_steps([w16], max(args.steps, 100), args.warmup)
        cold16 = time_cold_read_flush(w16, 30)
        cold_ms = float(np.median(cold16))
        # HBM-streaming rate: a model has one such layer per block, each with
        # its own weights, so the layer is launched round-robin over 16 copies
        # of the container (512 MB, twice the last-level cache): every launch
        # reads its weights from HBM. The launches are captured once in a HIP
        # graph and replayed back to back; HIP events around each replay on
        # the replay stream give the average launch duration.
        copies = [p16d.clone() for _ in range(16)]
        rounds = 2
        gstream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=gstream):
            for _ in range(rounds):
                for cp in copies:
                    b.w4a16_linear(X16d, cp, b16d, Y16, c16.N)
        graph.replay()
        torch.cuda.synchronize()
        rr = []
        with torch.cuda.stream(gstream):
            for _ in range(20):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(gstream)
                graph.replay()
                e1.record(gstream)
                gstream.synchronize()
                rr.append(e0.elapsed_time(e1) / (rounds * len(copies)))
        hbm_ms = float(np.median(rr))
        del graph, copies
        bytes16 = w4a16_bytes(c16.M, c16.K, c16.N)
        assert bytes16 == packed16.size + c16.M * c16.K * 2 + c16.M * c16.N * 2 + c16.N * 2
        traffic16, traffic16_detail = read_traffic_summary(W16_TRAFFIC_SUMMARY, W16_SOURCES)
        gbs = bytes16 / (hbm_ms * 1e-3) / 1e9
        out["w4a16"] = {
            "workload": f"{c16.name}: W4A16 linear M={c16.M} K={c16.K} N={c16.N} group=64 "
                        "(adaLN modulation: 6 x 3072 outputs of a batch of 2 conditioning vectors)",
            "ms_per_launch": round(hbm_ms, 5),
            "ms_single_layer_back_to_back_events": round(ms16, 5),
            "ms_single_layer_cold_events_median": round(cold_ms, 5),
            "roofline": {"bound": "hbm", "kernel": "w4a16_linear", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "timing": "HIP graph of 32 launches round-robin over 16 weight copies (512 MB), "
                                   "events around each replay, median of 20 replays",
                         "algorithmic_bytes": bytes16, "traffic": traffic16,
                         "traffic_detail": traffic16_detail},
            "prepare_library_s": round(prep16_s, 3),
        }
        log(f"[bench] w4a16 {hbm_ms * 1e3:.2f} us per launch from HBM ({gbs:.0f} GB/s); single layer: "
            f"back to back {ms16 * 1e3:.2f} us, cold {cold_ms * 1e3:.2f} us (events, incl. launch gaps)")
        if not args.no_cpu_baseline:
            out["w4a16"]["cpu_baseline"] = cpu_baseline_w4a16(c16, X16, W16, b16)
            log(f"[bench] w4a16 cpu baseline {out['w4a16']['cpu_baseline']['seconds']:.3f}s")

    try:
        out["measured_peaks"] = measured_peaks()
    except Exception as e:  # noqa: BLE001 -- reported, never fatal to the bench line
        out["measured_peaks"] = {"error": str(e)}

    out["prepare"] = {"library_s": round(prep_s, 3),
                      "what": "svdq_prepare_weights on the host: smoothing, rank-r SVD, bf16 factors, "
                              "residual, INT4 group codes and scales"}
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle) on {args.cpu_rows} rows ...")
        out["cpu_baseline"] = cpu_baseline(case, X, W, bias, args.cpu_rows)
        log(f"[bench] cpu baseline {out['cpu_baseline']['seconds']:.1f}s")
        one = cpu_baseline_one_core(case, X, W, bias, max(64, args.cpu_rows // 16))
        if one is not None:
            out["cpu_baseline_one_core"] = one
            log(f"[bench] cpu baseline, one core: {one['value']:.4f} TOPS ({one['seconds']:.1f}s per pass)")
        from oracle import svdquant as sq

        t1 = time.perf_counter()
        sq.prepare_weights(W["values"], amax_h, r)
        out["prepare"]["oracle_s"] = round(time.perf_counter() - t1, 3)
        out["prepare"]["oracle_cores"] = len(os.sched_getaffinity(0))
        log(f"[bench] oracle prepare {out['prepare']['oracle_s']:.1f}s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
