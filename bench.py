"""Throughput of the KV-cache translation hot path on one MI355X.

One step = token alignment + layer map + translation of every receiver
layer, K and V, of the long-context cross-family workload: sender 36 layers,
receiver 32 layers, 8 KV heads x 128 on both sides, 32768 receiver tokens
over a shared synthetic string (sender tokens 1..8 characters, receiver
1..6), three sender taps per receiver layer flattened to 3072 features,
3072 -> 1024 maps per layer and role (dense + rank-16 folded, bf16), sender
keys stored rotated (base 5e5) and rotated back, outputs rotated at the
receiver position (base 1e6), 1% outlier channels x20.  Inputs are seeded
synthetic tensors resident in HBM before timing.

Prints one JSON line.  ``value`` = receiver tokens translated per second
(all layers, K+V).  ``roofline`` reports the dominant kernel (the grouped
GEMM with its fused epilogue, one launch per step covering both roles: fp16
operands for the rotated-back keys, bf16 for the values) against the
bf16/fp16 dense matrix-core peak, timed with HIP events on the launch stream inside each
timed step.  ``traffic`` is the HBM bytes per launch read from the committed
rocprofv3 counter summary when the kernel sources still match it, else null.
``cpu_baseline`` times the CPU oracle on a bounded row sample of the same
workload.  ``also`` reports the per-head workload (32 -> 80 layers, 4096
tokens, fp32 128 x 128 maps) against the HBM peak, ``also_perhead_rope`` the
same with keys stored rotated on both sides; ``also_cfg3``,
``also_fp32_maps``, ``also_key_norm`` (the 32k setting with the receiver's
key normalisation) and ``also_fit`` other flattened settings and the ridge
fit.

Profiling helpers: ``--no-also`` runs the headline step alone and
``--perhead-only`` the per-head workload alone, so each kernel is profiled on
one workload; ``--calibration-copy`` first runs a plain 1 GiB device copy
(1 GiB read + 1 GiB written) so a rocprofv3 counter run of the same command
sees a kernel of known traffic; ``--pmc-summary FETCH.csv WRITE.csv`` turns
the counter CSVs of a FETCH_SIZE run and a WRITE_SIZE run into the per-launch
traffic summary kept under profiles/, ``--trace-summary STATS.csv LOG`` a
kernel-trace statistics file and the bench output of the same run into the
trace summary.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from cross_model_kv_kvx_amd import kvx, synth  # noqa: E402

PEAK_MFMA_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
PEAK_FP64_TFLOPS = 78.6          # MI355X dense fp64 (matrix and vector)
CALIB_BYTES = 1 << 30            # bytes read (and written) by the calibration copy
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "flat_gemm_kernel": ["kvx_flat.hip", "kvx_common.hpp", "kvx_internal.hpp"],
    "perhead_kernel": ["kvx_perhead.hip", "kvx_common.hpp", "kvx_internal.hpp"],
    "fit_from_caches": ["kvx_fit.hip", "kvx_fit.hpp", "kvx_align.hip", "kvx_common.hpp", "kvx_internal.hpp"],
}
FIT_TRACE_FILE = "fit_from_caches__calibration_64x65536__trace.md"
TRAFFIC_FILES = {
    "flat_gemm_kernel": "flat_gemm_kernel__crossfamily_rope_32k__traffic.md",
    "perhead_kernel": "perhead_kernel__32to80_4k__traffic.md",
}
TRACE_FILES = {
    "flat_gemm_kernel": "flat_gemm_kernel__crossfamily_rope_32k__trace.md",
    "perhead_kernel": "perhead_kernel__32to80_4k__trace.md",
}
# bench.py arguments of the profiled runs of each kernel: the headline step
# alone (default step counts), or the per-head workload alone, so every
# dispatch of the kernel in the profile belongs to the workload the summary
# names; the last field is the number of leading dispatches that are warm-up
PROFILE_ARGS = {
    "flat_gemm_kernel": ("flat", "--no-cpu-baseline --no-also", 3),
    "perhead_kernel": ("ph", "--perhead-only", 40),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "cross_model_kv_kvx_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel):
    """HBM bytes per launch from the committed counter summary, or None when
    the summary is missing or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILES, TRAFFIC_FILES[kernel])
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_h = re.search(r"source hash: `([0-9a-f]+)`", text)
    m_b = re.search(r"HBM bytes per launch \(mean\): `([0-9.eE+-]+)`", text)
    if not m_h or not m_b or m_h.group(1) != source_hash(kernel):
        return None
    return float(m_b.group(1))


def committed_clock_mhz(kernel):
    """Average clock under the kernel (GRBM_GUI_ACTIVE per XCD over the
    dispatches' duration) from the committed unit-counter summary, or None
    when the summary is missing or the kernel sources changed since."""
    path = os.path.join(PROFILES, UNITS_FILES[kernel])
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_h = re.search(r"source hash: `([0-9a-f]+)`", text)
    m_c = re.search(r"-> ([0-9.]+) MHz average clock", text)
    if not m_h or not m_c or m_h.group(1) != source_hash(kernel):
        return None
    return float(m_c.group(1))


def calibration_copy(dev):
    """A plain device copy of known size: CALIB_BYTES read, CALIB_BYTES written
    per dispatch (an elementwise multiply by one, run twice)."""
    src = torch.empty(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev).normal_()
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def pmc_summary(fetch_csv, write_csv):
    """Markdown traffic summaries from a FETCH_SIZE and a WRITE_SIZE counter run
    (rocprofv3 --pmc ... --output-format csv) of a --calibration-copy command."""
    def per_kernel(path, counter):
        rows = sorted((r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter),
                      key=lambda r: int(r["Dispatch_Id"]))
        vals = {}
        for r in rows:
            name = r["Kernel_Name"]
            key = None
            if "flat_gemm_kernel" in name:
                key = "flat_gemm_kernel"
            elif "perhead_kernel" in name:
                key = "perhead_kernel"
            elif "MulFunctor" in name and len(vals.get("copy", [])) < 2:
                key = "copy"  # the calibration copy runs first, twice
            if key:
                vals.setdefault(key, []).append(float(r["Counter_Value"]) * 1024.0)  # KiB -> bytes
        return vals
    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    if "copy" not in f or "copy" not in w:
        raise SystemExit("no calibration copy in the counter files (run the command with --calibration-copy)")
    kf = CALIB_BYTES / float(np.median(f["copy"]))
    kw = CALIB_BYTES / float(np.median(w["copy"]))
    out = {}
    for kernel in ("flat_gemm_kernel", "perhead_kernel"):
        if kernel not in f or kernel not in w:
            continue
        fb = np.array(f[kernel]) * kf
        wb = np.array(w[kernel]) * kw
        n = min(fb.size, wb.size)
        tot = fb[:n] + wb[:n]
        tag, bargs, _ = PROFILE_ARGS[kernel]
        out[kernel] = (f"# HBM traffic: {kernel}\n\n"
                       f"source hash: `{source_hash(kernel)}`\n\n"
                       "Commands (from the repository root, `cd /tmp && export TMPDIR=/tmp` first, paths "
                       "relative to the repository), then this summary:\n\n```\n"
                       f"rocprofv3 --pmc FETCH_SIZE -d gpurun_out/prof/{tag}_fetch -o fetch --output-format csv -- "
                       f"python3 bench.py --calibration-copy {bargs}\n"
                       f"rocprofv3 --pmc WRITE_SIZE -d gpurun_out/prof/{tag}_write -o write --output-format csv -- "
                       f"python3 bench.py --calibration-copy {bargs}\n"
                       f"python3 bench.py --pmc-summary gpurun_out/prof/{tag}_fetch/fetch_counter_collection.csv "
                       f"gpurun_out/prof/{tag}_write/write_counter_collection.csv\n```\n\n"
                       f"Counters: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), one rocprofv3 run each.\n"
                       f"Calibration: a plain copy of {CALIB_BYTES} bytes read and written reads "
                       f"FETCH_SIZE {np.median(f['copy']):.0f} B and WRITE_SIZE {np.median(w['copy']):.0f} B, "
                       f"so the factors are {kf:.4f} (fetch) and {kw:.4f} (write).\n\n"
                       f"| dispatches | fetch bytes (mean) | write bytes (mean) |\n|---|---|---|\n"
                       f"| {n} | {fb[:n].mean():.4g} | {wb[:n].mean():.4g} |\n\n"
                       f"HBM bytes per launch (mean): `{tot.mean():.6g}`\n")
    return out


def trace_summary(trace_dir, bench_log):
    """Markdown summaries of a rocprofv3 --kernel-trace --stats run of one of
    the profiled commands: per-dispatch durations of the kernel from the
    kernel trace (warm-up dispatches excluded: mean, median, min), the
    statistics file as rocprofv3 wrote it, and the live HIP-event launch time
    that bench.py printed in the same run."""
    stats = list(csv.DictReader(open(os.path.join(trace_dir, "trace_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(os.path.join(trace_dir, "trace_kernel_trace.csv"))))
    line = next(l for l in open(bench_log) if l.startswith("{"))
    res = json.loads(line)
    out = {}
    for kernel in ("flat_gemm_kernel", "perhead_kernel"):
        disp = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in trace
                      if f"kvx::{kernel}" in r["Kernel_Name"])
        if not disp:
            continue
        tag, bargs, skip = PROFILE_ARGS[kernel]
        dur = np.array([(e - b) / 1e3 for b, e in disp])  # us
        timed = dur[skip:] if dur.size > skip else dur
        roof = res["roofline"] if kernel == "flat_gemm_kernel" else res["also"]["roofline"]
        work = roof.get("flops_per_launch") or roof["algorithmic_bytes_per_launch"]
        scale = 1e12 if roof["unit"] == "TFLOP/s" else 1e9
        frac_prof = work / (float(np.median(timed)) * 1e-6) / scale / roof["peak"]
        tab = "\n".join(f"| {r['Name'].removeprefix('void ')[:70]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                        f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {r['Percentage']} |"
                        for r in stats[:14])
        out[kernel] = (f"# Kernel trace: {kernel}\n\n"
                       f"source hash: `{source_hash(kernel)}`\n\n"
                       "Commands (from the repository root, `cd /tmp && export TMPDIR=/tmp` first, paths "
                       "relative to the repository), then this summary:\n\n```\n"
                       f"rocprofv3 --kernel-trace --stats -d gpurun_out/prof/{tag}_trace -o trace --output-format csv "
                       f"-- python3 bench.py {bargs} > gpurun_out/prof/{tag}_trace.log\n"
                       f"python3 bench.py --trace-summary gpurun_out/prof/{tag}_trace gpurun_out/prof/{tag}_trace.log\n"
                       "```\n\n"
                       f"{kernel}: {dur.size} dispatches; the first {min(skip, dur.size)} are warm-up.\n\n"
                       f"| dispatches | mean us | median us | min us | max us |\n|---|---|---|---|---|\n"
                       f"| all {dur.size} | {dur.mean():.1f} | {np.median(dur):.1f} | {dur.min():.1f} | {dur.max():.1f} |\n"
                       f"| timed {timed.size} | {timed.mean():.1f} | {np.median(timed):.1f} | {timed.min():.1f} | "
                       f"{timed.max():.1f} |\n\n"
                       f"Same run, live HIP-event timing in bench.py: {roof['launch_ms'] * 1e3:.1f} us per launch, "
                       f"{roof['achieved']:.1f} {roof['unit']} algorithmic, frac {roof['frac']:.4f} of "
                       f"{roof['peak']:.0f}.\n"
                       f"From the profile's timed median: frac {frac_prof:.4f} "
                       f"({100 * (frac_prof / roof['frac'] - 1):+.1f}% against the bench line).\n\n"
                       "Kernel statistics of the run as rocprofv3 wrote them (all dispatches, input generation "
                       "and warm-up included; top 14):\n\n| kernel | calls | avg us | min us | max us | % time |\n"
                       f"|---|---|---|---|---|---|\n{tab}\n")
    return out


def _kernel_table(seg):
    per = {}
    for r in seg:
        name = r["Kernel_Name"].split("(")[0].removeprefix("void ")
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
        c, t = per.get(name, (0, 0.0))
        per[name] = (c + 1, t + d)
    span = (int(seg[-1]["End_Timestamp"]) - int(seg[0]["Start_Timestamp"])) / 1e6
    busy = sum(t for _, t in per.values())
    rows = "\n".join(f"| {n[:60]} | {c} | {t:.2f} | {1e3 * t / c:.1f} |"
                     for n, (c, t) in sorted(per.items(), key=lambda kv: -kv[1][1]))
    return span, busy, "| kernel | calls | total ms | mean us |\n|---|---|---|---|\n" + rows + "\n"


def _phase_table(seg, cuts):
    """Kernel time per phase: ``cuts`` are (phase name, index of its first
    dispatch in seg), in order."""
    out = []
    for k, (name, i0) in enumerate(cuts):
        i1 = cuts[k + 1][1] if k + 1 < len(cuts) else len(seg)
        t = sum((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6 for r in seg[i0:i1])
        out.append(f"| {name} | {i1 - i0} | {t:.2f} |")
    return "| phase | dispatches | ms |\n|---|---|---|\n" + "\n".join(out) + "\n"


def fit_trace_summary(trace_dir, bench_log):
    """Markdown summary of a rocprofv3 --kernel-trace run of ``bench.py
    --fit-only``: the kernels of the last kvx_fit_ridge_caches call and of
    the last kvx_fit_recolor_caches call, per kernel and per phase, beside
    the same run's fit_ms of each.  A call from the caches starts with the
    alignment's run compaction; the ridge call ends with its last output
    store, the Recolor call (the only one that forms weighted feature sums)
    with its last bias kernel."""
    trace = sorted(csv.DictReader(open(os.path.join(trace_dir, "trace_kernel_trace.csv"))),
                   key=lambda r: int(r["Start_Timestamp"]))
    res = json.loads(next(l for l in open(bench_log) if l.startswith("{")))

    def has(seg, key):
        return any(key in r["Kernel_Name"] for r in seg)

    def first(seg, key):
        return next(i for i, r in enumerate(seg) if key in r["Kernel_Name"])

    def last(seg, key):
        return max(i for i, r in enumerate(seg) if key in r["Kernel_Name"])

    starts = [i for i, r in enumerate(trace) if "kvx::runs_flags_scan" in r["Kernel_Name"]]
    segs = [trace[a:(starts[k + 1] if k + 1 < len(starts) else len(trace))] for k, a in enumerate(starts)]
    ridge = [g for g in segs if not has(g, "kvx::fitc_sx_kernel") and has(g, "kvx::fit_store_kernel")][-1]
    # a ridge call ends before the next call's first Gram
    ridge = ridge[:first(ridge, "kvx::gram_kernel")] if has(ridge, "kvx::gram_kernel") else ridge
    ridge = ridge[:last(ridge, "kvx::fit_store_kernel") + 1]
    rc = [g for g in segs if has(g, "kvx::fitc_sx_kernel")][-1]
    rc = rc[:last(rc, "kvx::fit_bias_final_kernel") + 1]

    out = (f"# Kernel trace: the fits from the calibration caches\n\n"
           f"source hash: `{source_hash('fit_from_caches')}`\n\n"
           "Commands (from the repository root, `cd /tmp && export TMPDIR=/tmp` first, paths relative to the "
           "repository), then this summary:\n\n```\n"
           "rocprofv3 --kernel-trace --stats -d gpurun_out/prof/fit_trace -o trace --output-format csv "
           "-- python3 bench.py --fit-only > gpurun_out/prof/fit_trace.log\n"
           "python3 bench.py --fit-trace-summary gpurun_out/prof/fit_trace gpurun_out/prof/fit_trace.log\n"
           "```\n\n")
    fit = res["also_fit"]
    span, busy, table = _kernel_table(ridge)
    cuts = [("Gram from the runs (run compaction, gathers, run sums, Gram)", 0),
            ("fp64 solve (lambda, Cholesky, two triangular solves)", first(ridge, "kvx::lambda_batched_kernel")),
            ("outputs", first(ridge, "kvx::fit_store_kernel"))]
    out += (f"## Ridge (kvx_fit_ridge_caches)\n\nWorkload: {fit['workload']}.\n\n"
            f"Last timed call: {len(ridge)} dispatches, {span:.2f} ms from its first to its last kernel, "
            f"{busy:.2f} ms of kernel time.  Same run, bench.py's host clock around the call: "
            f"{fit['fit_ms']:.2f} ms (mean of the timed calls).\n\n" + _phase_table(ridge, cuts) + "\n" + table)
    rec = res["also_recolor"]
    span, busy, table = _kernel_table(rc)
    cuts = [("moments (Gram from the runs, feature sums, Y^T Y, target sums, centring)", 0),
            ("factors (Cholesky of both, Z0 = L_x^-1 S_xy, E = L_y^-1)", first(rc, "kvx::potrf_diag")),
            # Z0^T Z0 is the product just before the first mirroring
            ("polar iteration (S = E Z0^T Z0 E^T, scale, Newton-Schulz steps)",
             first(rc, "kvx::sym_from_lower") - 1),
            ("map and bias (R = E^T S^-1/2 L_y^T, Z0 R, back-substitution, outputs)",
             last(rc, "kvx::frob_final") + 1)]
    out += (f"\n## Recolor (kvx_fit_recolor_caches)\n\nWorkload: {rec['workload']}.\n\n"
            f"Last timed call: {len(rc)} dispatches, {span:.2f} ms from its first to its last kernel, "
            f"{busy:.2f} ms of kernel time, {rec['polar_iterations']} polar iterations.  Same run, bench.py's "
            f"host clock around the call: {rec['fit_ms']:.2f} ms (mean of the timed calls).\n\n"
            + _phase_table(rc, cuts) + "\n" + table)
    return out


UNITS_FILES = {
    "flat_gemm_kernel": "flat_gemm_kernel__crossfamily_rope_32k__units.md",
    "perhead_kernel": "perhead_kernel__32to80_4k__units.md",
}
UNIT_COUNTERS = ("GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE "
                 "SQ_WAIT_INST_LDS SQ_VMEM_TA_CMD_FIFO_FULL TA_TA_BUSY TA_ADDR_STALLED_BY_TD_CYCLES TD_TD_BUSY "
                 "TD_TC_STALL")


def units_summary(counter_csv, bench_log):
    """Markdown summaries of one rocprofv3 --pmc run of the unit-activity
    counters over a profiled command: per-dispatch means, the average clock
    (GRBM_GUI_ACTIVE is summed over the 8 XCDs), busy fractions per unit, and
    the matrix-core ceiling at that clock beside the bench line's fraction of
    the published peak (which assumes 2.4 GHz)."""
    rows = list(csv.DictReader(open(counter_csv)))
    line = next(l for l in open(bench_log) if l.startswith("{"))
    res = json.loads(line)
    out = {}
    for kernel in ("flat_gemm_kernel", "perhead_kernel"):
        mine = [r for r in rows if kernel in r["Kernel_Name"]]
        if not mine:
            continue
        tag, bargs, skip = PROFILE_ARGS[kernel]
        per, dur = {}, {}
        for r in mine:
            d = int(r["Dispatch_Id"])
            per.setdefault(r["Counter_Name"], {}).setdefault(d, 0.0)
            per[r["Counter_Name"]][d] += float(r["Counter_Value"])
            dur[d] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        ids = sorted(per["GRBM_GUI_ACTIVE"])
        timed = ids[skip:] if len(ids) > skip else ids
        mean = {c: float(np.mean([v[i] for i in timed if i in v])) for c, v in per.items()}
        roof = res["roofline"] if kernel == "flat_gemm_kernel" else res["also"]["roofline"]
        t_s = float(np.mean([dur[i] for i in timed]))
        cyc = mean["GRBM_GUI_ACTIVE"] / 8.0
        mhz = cyc / t_s / 1e6
        lines = [f"| {c} | {v:.4g} |" for c, v in sorted(mean.items())]
        frac = [f"cycles per XCD (GRBM_GUI_ACTIVE / 8): {cyc:.4g} over the dispatches' mean duration "
                f"{t_s * 1e6:.1f} us (profiler timestamps) -> {mhz:.0f} MHz average clock"]
        for c, units in (("SQ_VALU_MFMA_BUSY_CYCLES", 1024), ("TA_TA_BUSY", 256), ("TD_TD_BUSY", 256),
                         ("TD_TC_STALL", 256), ("SQ_LDS_IDX_ACTIVE", 256), ("SQ_LDS_BANK_CONFLICT", 256),
                         ("SQ_VMEM_TA_CMD_FIFO_FULL", 256), ("SQ_BUSY_CU_CYCLES", 256)):
            if c in mean:
                frac.append(f"{c} per unit ({units} units): {mean[c] / units:.4g} cycles = "
                            f"{mean[c] / units / cyc:.3f} of the cycles")
        if roof["unit"] == "TFLOP/s":
            ceil = roof["peak"] * mhz / 2400.0
            ach = roof["flops_per_launch"] / t_s / 1e12
            frac.append(f"matrix-core ceiling at the measured clock: {roof['peak']:.0f} x {mhz:.0f} / 2400 = "
                        f"{ceil:.0f} TFLOP/s; over the same dispatches' mean duration the launch reaches "
                        f"{ach:.1f} TFLOP/s = {ach / ceil:.3f} of that ceiling and {ach / roof['peak']:.3f} of the "
                        f"published {roof['peak']:.0f} (counter collection lengthens the dispatches: the kernel-trace "
                        "summary gives the undisturbed time)")
        out[kernel] = (f"# Unit activity: {kernel}\n\n"
                       f"source hash: `{source_hash(kernel)}`\n\n"
                       "Commands (from the repository root, `cd /tmp && export TMPDIR=/tmp` first, paths "
                       "relative to the repository), then this summary:\n\n```\n"
                       f"rocprofv3 --pmc {UNIT_COUNTERS} -d gpurun_out/prof/{tag}_units -o units "
                       f"--output-format csv -- python3 bench.py {bargs} > gpurun_out/prof/{tag}_units.log\n"
                       f"python3 bench.py --units-summary gpurun_out/prof/{tag}_units/units_counter_collection.csv "
                       f"gpurun_out/prof/{tag}_units.log\n```\n\n"
                       f"Values: each counter summed over its instances per dispatch, mean over the "
                       f"{len(timed)} timed dispatches (the first {min(skip, len(ids))} are warm-up).  Fractions "
                       "assume each counter is summed over its units: GRBM_GUI_ACTIVE over 8 XCDs, "
                       "SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs, the TA, TD and per-CU SQ counters over 256 CUs; "
                       "each is divided by the cycles per XCD.\n\n"
                       "| counter | mean per dispatch |\n|---|---|\n" + "\n".join(lines) + "\n\n"
                       + "\n".join(f"- {f}" for f in frac) + "\n")
    return out


def measured_peaks(dev):
    """What this chip sustains (the probes of the library): HBM copy, read
    and fill streams over 4 GiB, and back-to-back bf16 matrix-core products
    on every compute unit for about 100 ms."""
    n = 1 << 29  # 2 GiB of fp32 in each copy buffer
    a = torch.empty(n, dtype=torch.float32, device=dev)
    b = torch.empty(n, dtype=torch.float32, device=dev)
    a.fill_(1.0)
    ms_c = kvx.probe_hbm("copy", a, b, iters=5)
    del b
    big = torch.empty(2 * n, dtype=torch.float32, device=dev)
    big.fill_(1.0)
    ms_r = kvx.probe_hbm("read", big, iters=5)
    ms_f = kvx.probe_hbm("fill", big, iters=5)
    del a, big
    torch.cuda.empty_cache()
    ms_m, fl = kvx.probe_mfma(reps=100000, iters=8, device=dev)
    gib4 = float(8 * n)
    return {"hbm_copy_GBs": gib4 / (ms_c * 1e-3) / 1e9, "hbm_read_GBs": gib4 / (ms_r * 1e-3) / 1e9,
            "hbm_fill_GBs": gib4 / (ms_f * 1e-3) / 1e9, "mfma_bf16_TFLOPs": fl / (ms_m * 1e-3) / 1e12,
            "note": "copy = 2 GiB read + 2 GiB written per launch; read and fill over 4 GiB; matrix cores: "
                    "4 independent 32x32x16 bf16 chains per wave, 8 waves per compute unit, ~100 ms"}


def library_gemm(dev, rows):
    """What the vendor library's dense bf16 products reach on this machine, as
    torch.matmul runs them (hipBLASLt): one 8192 x 8192 x 8192 product, and
    the headline's 64 products without its gather, epilogue or rotation (rows
    x 3072 by 3072 x 1024, one map each, 1024 outputs per row instead of the
    translation's expansion to every receiver row), timed with events on the
    current stream.  A reference for an achievable GEMM rate here; nothing of
    the translation runs through it."""
    g = torch.Generator(device=dev)
    g.manual_seed(9)

    def timed(fn, iters):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    a = torch.randn((8192, 8192), generator=g, device=dev).to(torch.bfloat16)
    b = torch.randn((8192, 8192), generator=g, device=dev).to(torch.bfloat16)
    c = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
    ms_sq = timed(lambda: torch.matmul(a, b, out=c), 10)
    del a, b, c
    x = torch.randn((rows, 3072), generator=g, device=dev).to(torch.bfloat16)
    ws = [torch.randn((3072, 1024), generator=g, device=dev).to(torch.bfloat16).contiguous() for _ in range(64)]
    y = torch.empty((rows, 1024), dtype=torch.bfloat16, device=dev)

    def shapes():
        for w in ws:
            torch.matmul(x, w, out=y)

    ms_sh = timed(shapes, 5)
    del x, ws, y
    torch.cuda.empty_cache()
    return {"library_gemm_8192_TFLOPs": 2.0 * 8192 ** 3 / (ms_sq * 1e-3) / 1e12,
            "headline_shapes_library_ms": ms_sh,
            "headline_shapes_library_TFLOPs": 64 * 2.0 * rows * 3072 * 1024 / (ms_sh * 1e-3) / 1e12,
            "library_note": "torch.matmul (hipBLASLt) on contiguous bf16 operands: 8192^3, and 64 products of "
                            f"{rows} x 3072 by 3072 x 1024 (the headline's distinct rows and maps, no gather, no "
                            "epilogue) timed back to back"}


def flat_inputs(dev):
    c = synth.CONFIGS[4]
    seed = c["seed"]
    send_end, recv_end = synth.token_ends(c["recv_tokens"], seed)
    shp = synth.CacheShape(36, len(send_end), 8, 128)
    x = {}
    for r, role in enumerate(("k", "v")):
        x[f"{role}_send"] = synth.sender_cache(shp, seed * 100 + r, dev, outlier_frac=0.01, outlier_scale=20.0,
                                               outlier_pairs=(role == "k"))
        w, a, b_lr, b = synth.flat_maps(32, 3072, 1024, seed * 100 + 20 + r, dev, 16)
        x[f"fold_{role}"] = (w, a, b_lr)
        x[f"w_{role}"] = kvx.fold_lowrank(w, a, b_lr, torch.bfloat16)
        x[f"b_{role}"] = b
    x["send_end"] = torch.as_tensor(send_end, device=dev)
    x["recv_end"] = torch.as_tensor(recv_end, device=dev)
    x["send_end_h"], x["recv_end_h"] = send_end, recv_end
    x["shp"] = shp
    # the maps put once into the kernel layout (untimed, as a server would
    # when it loads a model pair): fp16 for the rotated-back keys, bf16 values
    x["send_desc"] = kvx.cache_desc(x["k_send"], 5e5)
    x["recv_desc"] = kvx.CacheDesc(32, len(recv_end), 8, 128, kvx.BF16, 1e6)
    for role in ("k", "v"):
        x[f"p_{role}"] = kvx.prepare_maps(x[f"w_{role}"], role, x["send_desc"], x["recv_desc"], 3)
    torch.cuda.synchronize()
    return x


def run_step(x, taps, ws, outs, events=None):
    """One step: alignment + translation with the prepared maps.  Nothing
    synchronises: the alignment leaves its validity flag on the device; with
    ``events`` (three recorded torch.cuda.Event) the translation records the
    phase events."""
    tmap = kvx.align_tokens(x["send_end"], x["recv_end"], out=outs["map"], workspace=outs["align_ws"],
                            invalid=outs["invalid"])
    kvx.translate(x["k_send"], x["v_send"], tmap, taps, x["p_k"], x["p_v"], x["b_k"], x["b_v"],
                  send_rope_base=5e5, recv_rope_base=1e6, k_recv=outs["k"], v_recv=outs["v"], workspace=ws,
                  events=events, prepared=True, w_dtype=kvx.BF16)
    return tmap


def new_events(n):
    """n trios of timing events, each recorded once (so they exist)."""
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    for trio in evs:
        for e in trio:
            e.record()
    torch.cuda.synchronize()
    return evs


def cold_measure(dev, x, taps, ws, outs, steps=10):
    """The headline step with caches cold: before each step a 512 MB scratch
    write evicts the 256 MB last-level cache and the L2s, then the step is
    timed alone (median over steps)."""
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    step_ms, gemm_ms = [], []
    evs = new_events(steps)
    for i in range(steps):
        scratch.fill_(1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_step(x, taps, ws, outs, events=evs[i])
        torch.cuda.synchronize()
        step_ms.append((time.perf_counter() - t0) * 1e3)
        gemm_ms.append(evs[i][1].elapsed_time(evs[i][2]))
    del scratch
    n_r = x["recv_end_h"].size
    t = float(np.median(step_ms))
    return {"workload": "the headline step with the last-level cache and L2s flushed before each step "
                        "(512 MB scratch write)", "tokens_per_s": n_r / (t * 1e-3), "ms_per_step": t,
            "gemm_ms": float(np.median(gemm_ms)), "steps": steps}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, target_s=15.0):
    """The oracle as it stands on a bounded sample: token alignment of the
    whole string plus translation of sampled receiver rows (all layers, K
    and V), with maps folded by the oracle (untimed setup).  Timed on one
    host core: the process is pinned to a single CPU and numpy's BLAS pool
    limited to one thread for the timed part."""
    from oracle import kvx_oracle as O
    from threadpoolctl import threadpool_limits
    wo = {}
    for role in ("k", "v"):
        wt, u, v = (t.cpu().numpy() for t in x[f"fold_{role}"])
        wo[role] = np.stack([O.bf16_bits_to_f64(O.fold_lowrank(wt[l], u[l], v[l])[1]) for l in range(32)])
    bo = {role: x[f"b_{role}"].cpu().numpy() for role in ("k", "v")}
    caches = {role: x[f"{role}_send"].cpu() for role in ("k", "v")}
    taps = O.layer_taps(36, 32, 3, 4)
    n_recv = x["recv_end_h"].size
    rng = np.random.default_rng(0)
    rows_done, t_total, n = 0, 0.0, 16
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[0]
    torch_threads = torch.get_num_threads()
    os.sched_setaffinity(0, {core})
    torch.set_num_threads(1)
    try:
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            tmap = O.token_align(x["send_end_h"], x["recv_end_h"])
            t_align = time.perf_counter() - t0
            while t_total < target_s and rows_done < n_recv:
                rows = np.sort(rng.choice(n_recv, size=n, replace=False))
                t0 = time.perf_counter()
                for role in ("k", "v"):
                    O.translate_rows(caches[role], tmap, taps, wo[role], bo[role], rows, per_head=False,
                                     recv_heads=8, recv_head_dim=128, send_rope_base=5e5 if role == "k" else 0.0,
                                     recv_rope_base=1e6 if role == "k" else 0.0)
                t_total += time.perf_counter() - t0
                rows_done += n
    finally:
        os.sched_setaffinity(0, set(allowed))
        torch.set_num_threads(torch_threads)
    per_row = t_total / rows_done
    step_s = t_align + per_row * n_recv
    return {"value": n_recv / step_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "nproc": os.cpu_count(), "cpus_allowed": len(allowed), "cpu_model": cpu_model(), "pinned_core": core,
            "sample": f"token alignment of all {n_recv} receiver tokens ({t_align:.3f} s) + translation of "
                      f"{rows_done} random receiver rows x 32 layers x K,V ({t_total:.1f} s), scaled to "
                      f"{n_recv} rows; one core (process pinned, BLAS limited to one thread)"}


def perhead_measure(dev, steps=20, rope=False):
    """Per-head workload: sender 32 layers, receiver 80, 4096 tokens,
    8 x 128 heads, fp32 128 x 128 maps (prepared once), identity token map.
    With ``rope`` the keys are stored rotated on both sides (bases 5e5 and
    1e6): the preparation rotates the sender keys back into fp16 rows first.
    Calls run back to back on the stream; each records its phase events."""
    shp = synth.CacheShape(32, 4096, 8, 128)
    x = {}
    kw = dict(send_rope_base=5e5, recv_rope_base=1e6) if rope else {}
    send = kvx.CacheDesc(32, 4096, 8, 128, kvx.BF16, kw.get("send_rope_base", 0.0))
    recv = kvx.CacheDesc(80, 4096, 8, 128, kvx.BF16, kw.get("recv_rope_base", 0.0))
    for r, role in enumerate(("k", "v")):
        x[f"{role}_send"] = synth.sender_cache(shp, 200 + r, dev, channel_scale="loguniform")
        w, x[f"b_{role}"] = synth.perhead_maps(80, 8, 128, 220 + r, dev)
        x[f"p_{role}"] = kvx.prepare_maps(w, role, send, recv, 1, per_head=True)
        del w
    taps = kvx.layer_map(32, 80, 1)
    ident = torch.arange(4096, dtype=torch.int32, device=dev)
    k = torch.empty((80, 4096, 8, 128), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    ws = torch.empty(kvx.lib().kvx_translate_prepared_workspace_size(send, recv, 1, 1, 0), dtype=torch.uint8,
                     device=dev)

    def call(ev=None):
        kvx.translate(x["k_send"], x["v_send"], ident, taps, x["p_k"], x["p_v"], x["b_k"], x["b_v"],
                      per_head=True, k_recv=k, v_recv=v, workspace=ws, events=ev, prepared=True,
                      w_dtype=kvx.F32, **kw)

    # warm-up: the first few tens of launches after the inputs are built run
    # slower (about 0.63 against 0.55 ms on one box)
    for _ in range(40):
        call()
    evs = new_events(steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        call(evs[i])
    e1.record()
    torch.cuda.synchronize()
    t_call = e0.elapsed_time(e1) / steps * 1e-3
    prep_ms = float(np.mean([t[0].elapsed_time(t[1]) for t in evs]))
    t = float(np.mean([t[1].elapsed_time(t[2]) for t in evs])) * 1e-3
    # algorithmic bytes: each sender row read once, each receiver row written
    # once, maps (fp32) and bias read once
    bytes_alg = 2 * (32 * 4096 * 1024 * 2 + 80 * 4096 * 1024 * 2 + 80 * 8 * 128 * 128 * 4 + 80 * 1024 * 4)
    traffic = committed_traffic("perhead_kernel") if not rope else None
    return {"workload": "per-head 32->80 layers, 4096 tokens, 8x128 heads, fp32 maps, bf16 caches"
                        + (", keys rotated (RoPE 5e5 -> 1e6)" if rope else ""),
            "tokens_per_s": 4096 / t_call, "call_ms": t_call * 1e3, "kernel_ms": t * 1e3, "prep_ms": prep_ms,
            "roofline": {"bound": "hbm", "achieved": bytes_alg / t / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": bytes_alg / t / 1e9 / PEAK_HBM_GBS, "traffic": traffic,
                         "traffic_over_algorithmic": None if traffic is None else traffic / bytes_alg,
                         "kernel": "perhead_kernel", "launch_ms": t * 1e3, "algorithmic_bytes_per_launch": bytes_alg}}


def flat_setting_measure(dev, n_recv, seed, rope, fp32_maps, steps=8, key_norm=False):
    """A flattened setting other than the headline one: translation of all
    32 receiver layers, K and V, from 36 sender layers with three taps, maps
    prepared once (with ``key_norm``, the receiver's key normalisation in the
    epilogue).  Each call is synchronised and timed alone."""
    send_end, recv_end = synth.token_ends(n_recv, seed)
    shp = synth.CacheShape(36, len(send_end), 8, 128)
    kw = dict(send_rope_base=5e5, recv_rope_base=1e6) if rope else {}
    send = kvx.CacheDesc(36, len(send_end), 8, 128, kvx.BF16, kw.get("send_rope_base", 0.0))
    recv = kvx.CacheDesc(32, n_recv, 8, 128, kvx.BF16, kw.get("recv_rope_base", 0.0))
    x = {}
    for r, role in enumerate(("k", "v")):
        x[f"{role}_send"] = synth.sender_cache(shp, seed * 100 + r, dev, outlier_frac=0.01 if rope else 0.0,
                                               outlier_scale=20.0 if rope else 1.0, outlier_pairs=(rope and role == "k"))
        w, a, b_lr, b = synth.flat_maps(32, 3072, 1024, seed * 100 + 20 + r, dev, 16)
        w = w if fp32_maps else kvx.fold_lowrank(w, a, b_lr, torch.bfloat16)
        x[f"p_{role}"] = kvx.prepare_maps(w, role, send, recv, 3)
        x[f"b_{role}"] = b
        del w, a, b_lr
    taps = kvx.layer_map(36, 32, 3, 4)
    tmap = kvx.align_tokens(torch.as_tensor(send_end, device=dev), torch.as_tensor(recv_end, device=dev))
    m = tmap.cpu().numpy()
    U = int(1 + np.count_nonzero(np.diff(m)))
    if key_norm:
        kw["recv_key_norm"] = synth.key_norm_weights(32, 128, seed * 100 + 30, dev)
    outs = {"k_recv": torch.empty((32, n_recv, 8, 128), dtype=torch.bfloat16, device=dev)}
    outs["v_recv"] = torch.empty_like(outs["k_recv"])
    ms, gm = [], []
    evs = new_events(steps + 2)
    for i in range(steps + 2):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        kvx.translate(x["k_send"], x["v_send"], tmap, taps, x["p_k"], x["p_v"], x["b_k"], x["b_v"], events=evs[i],
                      prepared=True, w_dtype=kvx.F32 if fp32_maps else kvx.BF16, **kw, **outs)
        torch.cuda.synchronize()
        if i >= 2:
            ms.append((time.perf_counter() - t0) * 1e3)
            gm.append(evs[i][1].elapsed_time(evs[i][2]))
    t_gemm = float(np.mean(gm))
    flops = 2.0 * U * 3072 * 1024 * 32 * 2  # algorithmic (fp32 maps execute twice: high and low halves)
    return {"workload": f"flattened{' + RoPE' if rope else ''}{' + receiver key norm' if key_norm else ''}, "
                        f"{n_recv} receiver tokens, {'fp32' if fp32_maps else 'bf16'} maps", "distinct_sender_rows": U,
            "tokens_per_s": n_recv / (float(np.mean(ms)) * 1e-3), "translate_ms": float(np.mean(ms)),
            "roofline": {"bound": "mfma", "achieved": flops / (t_gemm * 1e-3) / 1e12, "peak": PEAK_MFMA_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": flops / (t_gemm * 1e-3) / 1e12 / PEAK_MFMA_BF16_TFLOPS,
                         "kernel": "flat_gemm_kernel", "launch_ms": t_gemm, "flops_per_launch": flops,
                         "executed_flops_per_launch": flops * (2 if fp32_maps else 1), "traffic": None}}


def fit_inputs(dev):
    """The calibration setting: 32 receiver layers x K, V = 64 problems.  The
    sender (36 layers) and receiver (32 layers) calibration caches of 65536
    receiver tokens with their alignment and taps -4/0/+4, and every problem's
    65536 x 3072 gathered bf16 features and 65536 x 1024 targets (for the
    features path and Recolor)."""
    n = 65536
    send_end, recv_end = synth.token_ends(n, 5)
    shp = synth.CacheShape(36, len(send_end), 8, 128)
    taps = kvx.layer_map(36, 32, 3, 4)
    tm = kvx.align_tokens(torch.as_tensor(send_end, device=dev), torch.as_tensor(recv_end, device=dev))
    cal = {"taps": taps, "tmap": tm, "xs": [], "ys": [],
           "runs": int(1 + np.count_nonzero(np.diff(tm.cpu().numpy())))}
    for r, role in enumerate(("k", "v")):
        cal[f"{role}_send"] = send = synth.sender_cache(shp, 500 + r, dev)
        cal[f"{role}_recv"] = recv = synth.receiver_cache(synth.CacheShape(32, n, 8, 128), 550 + r, dev)
        for l in range(32):
            cal["xs"].append(kvx.gather_features(send, tm, taps[l]))
            cal["ys"].append(recv[l].reshape(n, 1024))
    return cal


def fit_measure(dev, cal, reps=2):
    """Closed-form ridge fit of the whole calibration setting, lambda =
    1e-3 tr(G)/3072: all 64 maps from the caches in one call
    (kvx_fit_ridge_caches, the Gram from the alignment's runs), and for
    comparison the same maps from gathered features in one batched call and
    one problem alone."""
    xs, ys = cal["xs"], cal["ys"]
    n = xs[0].shape[0]
    count = len(xs)
    w_outs = [torch.empty((3072, 1024), dtype=torch.float32, device=dev) for _ in range(count)]

    def timed(c):
        ws = torch.empty(kvx.lib().kvx_fit_ridge_batched_workspace_size(c, 3072, 1024), dtype=torch.uint8,
                         device=dev)
        ms = []
        for i in range(reps + 1):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            kvx.fit_ridge_batched(xs[:c], ys[:c], lambda_rel=1e-3, w_outs=w_outs[:c], workspace=ws)  # synchronous
            if i >= 1:
                ms.append((time.perf_counter() - t0) * 1e3)
        del ws
        torch.cuda.empty_cache()
        return float(np.mean(ms))

    t_one = timed(1)
    t_feat = timed(count)
    del w_outs
    torch.cuda.empty_cache()
    send, recv = kvx.cache_desc(cal["k_send"]), kvx.cache_desc(cal["k_recv"])
    ws = torch.empty(kvx.fit_ridge_caches_workspace_size(send, recv, 3), dtype=torch.uint8, device=dev)
    wk = torch.empty((32, 3072, 1024), dtype=torch.float32, device=dev)
    wv = torch.empty_like(wk)
    ms = []
    for i in range(reps + 1):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        kvx.fit_ridge_caches(cal["k_send"], cal["v_send"], cal["k_recv"], cal["v_recv"], cal["tmap"], cal["taps"],
                             lambda_rel=1e-3, w_k=wk, w_v=wv, workspace=ws)  # synchronous
        if i >= 1:
            ms.append((time.perf_counter() - t0) * 1e3)
    t = float(np.mean(ms))
    del ws, wk, wv
    torch.cuda.empty_cache()
    gram = count * 2.0 * n * (3072 * 3073 / 2 + 3072 * 1024)      # G (one triangle) and X^T Y over all rows
    solve = count * (3072.0 ** 3 / 3 + 2 * 3072.0 ** 2 * 1024)    # Cholesky + two triangular solves, fp64
    t_roof = gram / (PEAK_MFMA_BF16_TFLOPS * 1e12) + solve / (PEAK_FP64_TFLOPS * 1e12)
    return {"workload": f"ridge fit of all {count} maps (32 layers x K,V) in one call from the calibration caches: "
                        "65536 receiver tokens, 3072 bf16 sender features (taps -4/0/+4 of 36 layers) -> 1024 "
                        "outputs each, lambda = 1e-3 tr(G)/3072",
            "fit_ms": t, "problems": count, "ms_per_problem": t / count,
            "calibration_tokens_per_s": count * n / (t * 1e-3), "runs_of_the_alignment": cal["runs"],
            "features_path_fit_ms": t_feat, "features_path_one_problem_alone_ms": t_one,
            "gram_flops": gram, "solve_flops_fp64": solve, "roofline_ms": t_roof * 1e3,
            "roofline": {"bound": "mfma", "achieved": gram / (t * 1e-3) / 1e12, "peak": PEAK_MFMA_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": t_roof / (t * 1e-3),
                         "note": "frac = (Gram FLOPs of the plain definition over all 65536 rows at the bf16 peak "
                                 "+ solve FLOPs at the fp64 peak) / measured time; achieved = those Gram FLOPs "
                                 "over the whole fit time (the runs formulation executes fewer)",
                         "traffic": None}}


def fp8_measure(dev, x, taps, steps=10):
    """The headline step's translation with the maps stored as fp8 (E4M3
    codes, one fp32 scale per output; folded in fp32, quantised by the
    library): same inputs, rotations and outputs."""
    q, sc = {}, {}
    for role in ("k", "v"):
        wt, u, v = x[f"fold_{role}"]
        q[role], sc[role] = kvx.quantize_fp8(kvx.fold_lowrank(wt, u, v, torch.float32))
    tmap = kvx.align_tokens(x["send_end"], x["recv_end"])
    N_R = x["recv_end_h"].size
    U = int(1 + np.count_nonzero(np.diff(tmap.cpu().numpy())))
    k_out = torch.empty((32, N_R, 8, 128), dtype=torch.bfloat16, device=dev)
    v_out = torch.empty_like(k_out)
    send = kvx.cache_desc(x["k_send"], 5e5)
    recv = kvx.CacheDesc(32, N_R, 8, 128, kvx.BF16, 1e6)
    ws = torch.empty(kvx.translate_workspace_size(send, recv, 3, False), dtype=torch.uint8, device=dev)

    def call(stage):
        kvx.translate_fp8(x["k_send"], x["v_send"], tmap, taps, q["k"], q["v"], sc["k"], sc["v"], x["b_k"], x["b_v"],
                          send_rope_base=5e5, recv_rope_base=1e6, k_recv=k_out, v_recv=v_out, workspace=ws,
                          stage_ms=stage)

    for _ in range(2):
        call([])
    stages = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        st = []
        call(st)
        stages.append(st)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    gemm_ms = float(np.mean([s_[1] for s_ in stages]))
    flops = 2.0 * U * 3072 * 1024 * 32 * 2
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    return {"workload": "flattened + RoPE, 32768 receiver tokens, maps stored as fp8 E4M3 with per-output scales "
                        "(widened exactly to bf16 / fp16 operands)",
            "distinct_sender_rows": U, "tokens_per_s": N_R / (ms * 1e-3), "translate_ms": ms,
            "map_bytes": 2 * 32 * 1024 * (3072 + 4),
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": achieved / PEAK_MFMA_BF16_TFLOPS, "kernel": "flat_gemm_kernel (fp8 maps)",
                         "launch_ms": gemm_ms, "flops_per_launch": flops, "traffic": None}}


def recolor_measure(dev, cal, reps=2):
    """Moment-matched (Recolor) fit of the whole calibration setting in one
    call: 64 problems of 65536 rows, 3072 -> 1024, rho_x = 1e-3, from the
    caches (kvx_fit_recolor_caches: the feature moments from the
    alignment's runs), and for comparison from gathered features."""
    xs, ys = cal["xs"], cal["ys"]
    n, count = xs[0].shape[0], len(xs)
    fi, fo = 3072, 1024

    def timed(call):
        ms = []
        for i in range(reps + 1):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            call()  # synchronous
            if i >= 1:
                ms.append((time.perf_counter() - t0) * 1e3)
        return float(np.mean(ms))

    w_outs = [torch.empty((fi, fo), dtype=torch.float32, device=dev) for _ in range(count)]
    b_outs = [torch.empty(fo, dtype=torch.float32, device=dev) for _ in range(count)]
    ws = torch.empty(kvx.lib().kvx_fit_recolor_workspace_size(count, fi, fo), dtype=torch.uint8, device=dev)
    info_f, st_f = {}, []
    t_feat = timed(lambda: (st_f.clear(), kvx.fit_recolor(xs, ys, rho_x=1e-3, w_outs=w_outs, b_outs=b_outs,
                                                           workspace=ws, info=info_f, status=st_f)))
    del ws, w_outs, b_outs
    torch.cuda.empty_cache()
    send, recv = kvx.cache_desc(cal["k_send"]), kvx.cache_desc(cal["k_recv"])
    ws = torch.empty(kvx.fit_recolor_caches_workspace_size(send, recv, 3), dtype=torch.uint8, device=dev)
    wk = torch.empty((32, fi, fo), dtype=torch.float32, device=dev)
    wv = torch.empty_like(wk)
    bk = torch.empty((32, fo), dtype=torch.float32, device=dev)
    bv = torch.empty_like(bk)
    info, st = {}, []
    t = timed(lambda: (st.clear(), kvx.fit_recolor_caches(cal["k_send"], cal["v_send"], cal["k_recv"],
                                                          cal["v_recv"], cal["tmap"], cal["taps"], rho_x=1e-3,
                                                          w_k=wk, w_v=wv, b_k=bk, b_v=bv, workspace=ws,
                                                          info=info, status=st)))
    del ws, wk, wv, bk, bv
    torch.cuda.empty_cache()
    it = info["iters"]
    gram = count * 2.0 * n * (fi * (fi + 1) / 2 + fi * fo + fo * (fo + 1) / 2)   # S_xx, S_xy, S_yy on bf16 MFMA
    # the fp64 FLOPs the solve executes (symmetric results counted once)
    fp64 = count * (fi ** 3 / 3 + fo ** 3 / 3 + fi ** 2 * fo + fo ** 3 / 3       # factors, Z0 = L_x^-1 S_xy, L_y^-1
                    + fi * fo ** 2 + 2 * fo ** 3 + fo ** 3                        # S = E (Z0^T Z0) E^T
                    + it * 6 * fo ** 3                                            # steps: P, P^2 halves, Y T, T Z
                    + 4 * fo ** 3 + 2 * fi * fo ** 2 + fi ** 2 * fo)               # R = E^T Z L_y^T, Z0 R, L_x^-T
    t_roof = gram / (PEAK_MFMA_BF16_TFLOPS * 1e12) + fp64 / (PEAK_FP64_TFLOPS * 1e12)
    return {"workload": f"Recolor fit of all {count} maps (32 layers x K,V) in one call from the calibration caches: "
                        "65536 receiver tokens, 3072 bf16 sender features -> 1024 receiver outputs each, "
                        "rho_x = 1e-3",
            "fit_ms": t, "problems": count, "ms_per_problem": t / count, "polar_iterations": it,
            "statuses_ok": int(sum(1 for v in st if v == kvx.OK)),
            "calibration_tokens_per_s": count * n / (t * 1e-3),
            "features_path_fit_ms": t_feat, "features_path_polar_iterations": info_f["iters"],
            "features_path_statuses_ok": int(sum(1 for v in st_f if v == kvx.OK)),
            "gram_flops": gram, "fp64_flops": fp64, "roofline_ms": t_roof * 1e3,
            "roofline": {"bound": "fp64", "achieved": fp64 / (t * 1e-3) / 1e12, "peak": PEAK_FP64_TFLOPS,
                         "unit": "TFLOP/s", "frac": t_roof / (t * 1e-3),
                         "note": "frac = (moment FLOPs of the plain definition over all 65536 rows at the bf16 "
                                 "peak + the fp64 FLOPs the solve executes at the fp64 peak) / measured time; "
                                 "achieved = those fp64 FLOPs over the whole fit time",
                         "traffic": None}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--trace-summary", nargs=2, metavar=("TRACE_DIR", "BENCH_LOG"))
    ap.add_argument("--units-summary", nargs=2, metavar=("COUNTER_CSV", "BENCH_LOG"))
    ap.add_argument("--fit-trace-summary", nargs=2, metavar=("TRACE_DIR", "BENCH_LOG"))
    ap.add_argument("--fp8-only", action="store_true", help="measure the fp8-map translation alone")
    ap.add_argument("--fit-only", action="store_true",
                    help="measure the ridge and Recolor fits of the calibration setting alone")
    ap.add_argument("--perhead-only", action="store_true",
                    help="measure the per-head workload alone (profiling runs of the per-head kernel)")
    args = ap.parse_args()
    if args.fit_trace_summary:
        path = os.path.join(PROFILES, FIT_TRACE_FILE)
        with open(path, "w") as fh:
            fh.write(fit_trace_summary(*args.fit_trace_summary))
        print(f"wrote {path}")
        return
    if args.pmc_summary or args.trace_summary or args.units_summary:
        if args.pmc_summary:
            made, files = pmc_summary(*args.pmc_summary), TRAFFIC_FILES
        elif args.trace_summary:
            made, files = trace_summary(*args.trace_summary), TRACE_FILES
        else:
            made, files = units_summary(*args.units_summary), UNITS_FILES
        for kernel, text in made.items():
            path = os.path.join(PROFILES, files[kernel])
            with open(path, "w") as fh:
                fh.write(text)
            print(f"wrote {path}")
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the translation runs on a single device with no collectives; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calibration_copy:
        log("bench: calibration copy")
        calibration_copy(dev)
    if args.fp8_only:
        log("bench: flattened + RoPE, bf16 and fp8 maps")
        x = flat_inputs(dev)
        taps = kvx.layer_map(36, 32, 3, 4)
        print(json.dumps({"also_fp8_maps": fp8_measure(dev, x, taps)}), flush=True)
        return
    if args.fit_only:
        log("bench: calibration fits")
        cal = fit_inputs(dev)
        print(json.dumps({"also_fit": fit_measure(dev, cal), "also_recolor": recolor_measure(dev, cal)}), flush=True)
        return
    if args.perhead_only:
        log("bench: per-head workload")
        print(json.dumps({"also": perhead_measure(dev)}), flush=True)
        return
    log("bench: measured peaks")
    peaks = measured_peaks(dev)
    log("bench: building inputs")
    x = flat_inputs(dev)
    taps = kvx.layer_map(36, 32, 3, 4)
    N_R = x["recv_end_h"].size
    ws = torch.empty(kvx.lib().kvx_translate_prepared_workspace_size(x["send_desc"], x["recv_desc"], 3, 0, 0),
                     dtype=torch.uint8, device=dev)
    outs = {"map": torch.empty(N_R, dtype=torch.int32, device=dev),
            "align_ws": torch.empty(kvx.lib().kvx_align_workspace_size(N_R), dtype=torch.uint8, device=dev),
            "k": torch.empty((32, N_R, 8, 128), dtype=torch.bfloat16, device=dev)}
    outs["v"] = torch.empty_like(outs["k"])
    outs["invalid"] = torch.zeros(1, dtype=torch.int32, device=dev)
    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        run_step(x, taps, ws, outs)
    # HIP events of every timed step (before the preparation kernels, before
    # and after the translation kernel), recorded on the launch stream by the
    # library; created by one record each before timing
    evs = new_events(args.steps)
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        tmap = run_step(x, taps, ws, outs, events=evs[i])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    if int(outs["invalid"].item()) != 0:
        raise SystemExit("token alignment reported invalid offsets")
    stages = [[trio[0].elapsed_time(trio[1]), trio[1].elapsed_time(trio[2])] for trio in evs]
    ms_step = dt * 1e3 / args.steps
    m = tmap.cpu().numpy()
    U = int(1 + np.count_nonzero(np.diff(m)))
    gemm_ms = float(np.mean([s[1] for s in stages]))
    prep_ms = float(np.mean([s[0] for s in stages]))
    # one launch per step covers both roles; its algorithmic work: U distinct
    # sender rows x 3072 features x 1024 outputs x 32 layers x 2 roles
    launches = 1
    launch_ms = gemm_ms / launches
    flops = 2.0 * U * 3072 * 1024 * 32 * 2
    achieved = flops / (launch_ms * 1e-3) / 1e12
    # algorithmic bytes of a launch, both roles: the U distinct sender rows of
    # every sender layer the taps reference read once, the maps and bias read
    # once, every receiver row written once
    used_layers = len(set(int(t) for t in np.asarray(taps).ravel()))
    bytes_alg = 2 * (used_layers * U * 2048 + 32 * (3072 * 1024 * 2 + 1024 * 4) + 32 * N_R * 2048)
    traffic = committed_traffic("flat_gemm_kernel")
    res = {
        "metric": "translated KV tokens/sec (all layers, K+V) at 32k ctx; % of MFMA/HBM roofline",
        "value": N_R / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "cross-family flattened translation with RoPE: 36->32 layers, 8x128 heads, "
                               "taps -4/0/+4, 3072->1024 bf16 maps, 32768 receiver tokens",
                   "recv_tokens": N_R, "send_tokens": int(x["send_end_h"].size), "distinct_sender_rows": U,
                   "global_batch": 1, "seq_len": N_R, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_MFMA_BF16_TFLOPS, "traffic": traffic,
                     "kernel": "flat_gemm_kernel", "launches_per_step": launches, "launch_ms": launch_ms,
                     "launch_ms_median": float(np.median([s[1] for s in stages])),
                     "launch_ms_min": float(np.min([s[1] for s in stages])),
                     "flops_per_launch": flops, "algorithmic_bytes_per_launch": bytes_alg,
                     "traffic_over_algorithmic": None if traffic is None else traffic / bytes_alg,
                     "prep_ms": prep_ms},
    }
    log("bench: library GEMM reference")
    peaks.update(library_gemm(dev, U))
    res["measured_peaks"] = peaks
    res["roofline"]["frac_of_measured_peak"] = achieved / peaks["mfma_bf16_TFLOPs"]
    res["roofline"]["frac_of_library_gemm_8192"] = achieved / peaks["library_gemm_8192_TFLOPs"]
    res["roofline"]["library_same_shapes_ms"] = peaks["headline_shapes_library_ms"]
    # the matrix cores' ceiling at the clock they hold under this kernel (the
    # published peak assumes 2.4 GHz), from the committed unit-counter run
    mhz = committed_clock_mhz("flat_gemm_kernel")
    res["roofline"]["clock_mhz_under_load"] = mhz
    res["roofline"]["frac_of_clock_limited_peak"] = (
        None if mhz is None else achieved / (PEAK_MFMA_BF16_TFLOPS * mhz / 2400.0))
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(x)
    if not args.no_also:
        log("bench: per-head workload")
        res["also"] = perhead_measure(dev)
        log("bench: per-head workload, rotated keys")
        res["also_perhead_rope"] = perhead_measure(dev, rope=True)
        for key in ("also", "also_perhead_rope"):
            ro = res[key]["roofline"]
            ro["frac_of_measured_peak"] = ro["achieved"] / peaks["hbm_copy_GBs"]
        log("bench: headline step, caches flushed")
        res["also_cold"] = cold_measure(dev, x, taps, ws, outs)
        log("bench: flattened + RoPE, fp8 maps")
        res["also_fp8_maps"] = fp8_measure(dev, x, taps)
        del x, outs, ws
        torch.cuda.empty_cache()
        log("bench: flattened + RoPE + receiver key norm, 32768 tokens")
        res["also_key_norm"] = flat_setting_measure(dev, 32768, 4, rope=True, fp32_maps=False, key_norm=True)
        torch.cuda.empty_cache()
        log("bench: flattened, 8192 tokens, no RoPE")
        res["also_cfg3"] = flat_setting_measure(dev, 8192, 3, rope=False, fp32_maps=False)
        log("bench: flattened with fp32 maps, 16384 tokens")
        res["also_fp32_maps"] = flat_setting_measure(dev, 16384, 6, rope=False, fp32_maps=True)
        torch.cuda.empty_cache()
        log("bench: ridge fit")
        cal = fit_inputs(dev)
        res["also_fit"] = fit_measure(dev, cal)
        log("bench: Recolor fit")
        res["also_recolor"] = recolor_measure(dev, cal)
        del cal
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
