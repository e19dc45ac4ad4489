#!/usr/bin/env python3
"""Benchmark of the TBE hot path on one MI355X: one step = bounds check + forward + backward
(exact row-wise Adagrad) over one synthetic batch of the skewed large workload (T=32 tables of
2M x 128 fp16 rows, B=131072, L ~ Poisson(20), Zipf(0.91) over 95000 ranks per table: about
83.9M lookups, 3.03M unique rows, hottest row about 128K lookups).  By default the backward's
transpose runs inside the forward call on a second stream, concurrent with the pooling
(--hoist off: inside the backward call).

Prints one JSON line (metric, value, ..., roofline, cpu_baseline).

  python bench.py [--steps K] [--warmup W] [--workload skewed] [--no-cpu-baseline] [--hoist on|off]
  python bench.py --calib-copy      # plain copy kernel of known size (rocprofv3 byte calibration)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bwd_tbe_fwd_amd as tbe  # noqa: E402
import tbe_inputs as ti  # noqa: E402

METRIC = "TBE fwd+bwd lookups/s and achieved HBM GB/s vs peak, 1 MI355X"
HBM_PEAK_GBS = 8000.0
# MI355X dense matrix-core peaks (no sparsity), TFLOP/s
MFMA_PEAK_TFLOPS = {"fp16": 2500.0, "bf16": 2500.0, "fp32": 157.3}
MFMA_KERNELS = ("fwd_hist", "hist_bwd_partial", "dense_partial")  # the kernels mfma_flops prices
KERNELS = ["bounds_offsets", "bounds_indices", "fwd_gather", "fwd_hist", "linearize",
           "radix_upsweep", "radix_scan", "radix_downsweep", "rle", "classify", "short_run",
           "grad_accum", "long_apply", "hist_bwd_partial", "hist_bwd_apply", "dense_sample", "dense_select",
           "dense_partial", "dense_apply"]


# sources each timed kernel is built from: its counters in profiles/ are valid only while
# these files are unchanged
KERNEL_SOURCES = {
    "fwd_gather": ["forward.hip", "tbe_device.h"],
    "fwd_hist": ["forward.hip", "tbe_device.h"],
    "short_run": ["backward_kernels.h", "backward_launch.h", "tbe_device.h"],
    "grad_accum": ["backward.hip", "backward_kernels.h", "tbe_device.h"],
    "dense_partial": ["dense_backward.hip", "tbe_device.h"],
    "long_apply": ["backward_kernels.h", "backward_launch.h", "tbe_device.h"],
    "linearize": ["transpose.hip", "tbe_device.h"],
    "radix_upsweep": ["transpose.hip", "tbe_device.h"],
    "radix_downsweep": ["transpose.hip", "tbe_device.h"],
    "bounds_indices": ["bounds.hip", "tbe_device.h"],
    "bounds_offsets": ["bounds.hip", "tbe_device.h"],
    "hist_bwd_partial": ["hist_backward.hip", "tbe_device.h"],
    "hist_bwd_apply": ["hist_backward.hip", "tbe_device.h"],
    "radix_scan": ["transpose.hip", "tbe_device.h"],
    "rle": ["transpose.hip", "tbe_device.h"],
    "classify": ["transpose.hip", "tbe_device.h"],
    "dense_sample": ["dense_backward.hip", "tbe_device.h"],
    "dense_select": ["dense_backward.hip", "tbe_device.h"],
    "dense_apply": ["dense_backward.hip", "tbe_device.h"],
}


def kernel_sources_hash(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, "bwd_tbe_fwd_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def all_sources_hash() -> str:
    """sha256 over every library source file (sorted by name)."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "bwd_tbe_fwd_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()


# profile summaries in profiles/ are named for the workload they cover
PROFILE_TAG = {"skewed": "skewed_large", "histogram": "histogram", "mixed": "mixed_width",
               "uniform": "uniform", "tiny": "tiny"}


def _traffic_file(workload: str):
    path = os.path.join(ROOT, "profiles", f"{PROFILE_TAG[workload]}_traffic.json")
    try:
        with open(path) as f:
            return json.load(f)
    except (OSError, ValueError):
        return None


def measured_step_traffic(workload: str):
    """Bytes leaving L2 over one whole step (every kernel, every launch) from the committed
    counters, {"copy_calibrated": FETCH_SIZE / WRITE_SIZE scaled by the copy factors,
    "by_request_size": read and write requests weighted by their sizes}; None if any library
    source changed since they were taken."""
    prof = _traffic_file(workload)
    if not prof or prof.get("sources_sha256") != all_sources_hash():
        return None
    return prof["step"]


def measured_traffic(workload: str, kernel: str, launches_per_step: int):
    """The same per launch of one kernel (its counters summed over a step, divided by its
    launches per step), plus its L2 hit rate; None if the kernel's sources changed since."""
    prof = _traffic_file(workload)
    if not prof or kernel not in prof.get("kernels", {}):
        return None
    k = prof["kernels"][kernel]
    if k.get("sources_sha256") != kernel_sources_hash(kernel):
        return None
    n = max(1, launches_per_step)
    return {"copy_calibrated": k["copy_calibrated_bytes_per_step"] / n,
            "by_request_size": k["sized_bytes_per_step"] / n,
            "read_by_request_size": k["sized_read_bytes_per_step"] / n,
            "write_by_request_size": k["sized_write_bytes_per_step"] / n,
            "l2_hit_rate": k.get("l2_hit_rate")}


# kernel names in rocprofv3 output -> the names bench.py times them under
def kernel_group(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
    n = n.split("<")[0].split("::")[-1]
    n = n[:-len("_kernel")] if n.endswith("_kernel") else n
    for prefix, group in (("rle_", "rle"), ("classify_", "classify"), ("bounds_offsets_", "bounds_offsets")):
        if n.startswith(prefix):
            return group
    return n


def _csv_rows(d: str, suffix: str):
    import csv
    import glob
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            yield from csv.DictReader(fh)


def _counter_totals(d: str):
    """{(group, counter): [dispatches, total]} over every dispatch in a --pmc output directory."""
    tot = {}
    for row in _csv_rows(d, "counter_collection.csv"):
        k = (kernel_group(row.get("Kernel_Name", "?")), row["Counter_Name"])
        a = tot.setdefault(k, [0, 0.0])
        a[0] += 1
        a[1] += float(row["Counter_Value"])
    return tot


PROFILE_RUNS = {
    # name -> rocprofv3 options; every run profiles `python3 bench.py ...` (the workload's flags
    # appended) with the transpose in the backward call, so that no two kernels overlap
    "trace": "--kernel-trace --stats",
    "fetch": "--pmc FETCH_SIZE",
    "write": "--pmc WRITE_SIZE",
    "rd": "--pmc TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum",
    "wr": "--pmc TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum TCC_HIT_sum TCC_MISS_sum",
}
PROFILE_STEPS = 3   # counter runs: --steps 2 --warmup 1 --dominant short_run (no per-kernel scan)


def profile_commands(workload: str):
    bench_args = {"trace": f"--workload {workload} --steps 10 --warmup 2 --no-cpu-baseline --hoist off"}
    cmds = {}
    for name, opt in PROFILE_RUNS.items():
        args = bench_args.get(name, f"--workload {workload} --steps 2 --warmup 1 --no-cpu-baseline "
                                    f"--hoist off --dominant short_run")
        filt = "" if name == "trace" else " --kernel-include-regex tbe::"
        cmds[name] = (f"rocprofv3 {opt}{filt} --output-format csv -d gpurun_out/prof/{workload}_{name} "
                      f"-o run -- python3 bench.py {args}")
        if name != "trace":
            cmds["calib_" + name] = (f"rocprofv3 {opt} --kernel-include-regex calibration --output-format csv "
                                     f"-d gpurun_out/prof/calib_{name} -o run -- python3 bench.py --calib-copy")
    return cmds


def mfma_rows(workload: str, trace: list, batch=None):
    """Matrix-core utilisation of the traced kernels that use MFMA: the workload's batch drawn on
    the CPU (same seed as on the GPU), its issued flops per launch over the trace's average
    duration.  {kernel: {dtype, flops_per_launch, average_us, achieved_TFLOPs, peak_TFLOPs, frac}}"""
    if not any(kernel_group(r["Name"]) in MFMA_KERNELS for r in trace):
        return {}
    spec = ti.WORKLOADS[workload]
    bt = batch if batch is not None else ti.make_batch(spec, device="cpu")
    tables = tbe.Tables(bt.E, bt.D, bt.B, bt.w_dtype, device="cpu", pooling_hint=spec.pooling_hint)
    hist_table = tables.c.hist_table if bt.psw is None else -1
    flops = mfma_flops(bt, batch_stats(bt, hist_table))
    out = {}
    for r in trace:
        g = kernel_group(r["Name"])
        if g in flops:
            fl, dt = flops[g]
            us = float(r["AverageNs"]) / 1e3
            ach = fl / (us * 1e-6) / 1e12
            out[g] = {"dtype": dt, "flops_per_launch": fl, "average_us": us, "achieved_TFLOPs": ach,
                      "peak_TFLOPs": MFMA_PEAK_TFLOPS[dt], "frac": ach / MFMA_PEAK_TFLOPS[dt]}
    return out


def summarize_profiles(root: str, workload: str, out_dir: str = None):
    """Writes <tag>_kernel_trace.md, <tag>_hbm_counters.md and <tag>_traffic.json (into
    profiles/ by default) from the rocprofv3 output directories that profile_commands(workload)
    names, under root."""
    tag = PROFILE_TAG[workload]
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    cmds = profile_commands(workload)
    d = lambda name: os.path.join(root, f"{workload}_{name}") if not name.startswith("calib") \
        else os.path.join(root, name)
    # durations
    trace = [r for r in _csv_rows(d("trace"), "kernel_stats.csv") if "tbe::" in r["Name"]]
    # the copy of known size: 1 GiB read and written per launch, 3 launches
    n_copy = 3
    copy_b = float(1 << 30)
    cal = {}
    for name in ("fetch", "write", "rd", "wr"):
        for (g, c), (n, v) in _counter_totals(d("calib_" + name)).items():
            if g == "calibration_copy":
                cal[c] = v / n
    fetch_factor = copy_b / (cal["FETCH_SIZE"] * 1024)
    write_factor = copy_b / (cal["WRITE_SIZE"] * 1024)
    sized_rd = lambda c: 32 * c["TCC_EA0_RDREQ_32B_sum"] + 64 * c["TCC_EA0_RDREQ_64B_sum"] + 128 * c["TCC_EA0_RDREQ_128B_sum"]
    sized_wr = lambda c: 32 * (c["TCC_EA0_WRREQ_sum"] - c["TCC_EA0_WRREQ_64B_sum"]) + 64 * c["TCC_EA0_WRREQ_64B_sum"]
    cal_sized = (sized_rd(cal) / copy_b, sized_wr(cal) / copy_b)
    per = {}
    for name in ("fetch", "write", "rd", "wr"):
        for (g, c), (n, v) in _counter_totals(d(name)).items():
            per.setdefault(g, {})[c] = v / PROFILE_STEPS        # per step
            per[g]["dispatches_per_step"] = n / PROFILE_STEPS
    kernels = {}
    for g, c in per.items():
        if not all(k in c for k in ("FETCH_SIZE", "WRITE_SIZE", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_WRREQ_sum")):
            continue
        hit, miss = c.get("TCC_HIT_sum", 0.0), c.get("TCC_MISS_sum", 0.0)
        kernels[g] = {
            "dispatches_per_step": c["dispatches_per_step"],
            "fetch_kib_per_step": c["FETCH_SIZE"], "write_kib_per_step": c["WRITE_SIZE"],
            "copy_calibrated_bytes_per_step": (c["FETCH_SIZE"] * fetch_factor + c["WRITE_SIZE"] * write_factor) * 1024,
            "sized_read_bytes_per_step": sized_rd(c), "sized_write_bytes_per_step": sized_wr(c),
            "sized_bytes_per_step": sized_rd(c) + sized_wr(c),
            "read_requests_per_step": {"32B": c["TCC_EA0_RDREQ_32B_sum"], "64B": c["TCC_EA0_RDREQ_64B_sum"],
                                       "128B": c["TCC_EA0_RDREQ_128B_sum"], "all": c["TCC_EA0_RDREQ_sum"]},
            "l2_hit_rate": hit / (hit + miss) if hit + miss > 0 else None,
            "sources_sha256": kernel_sources_hash(g) if g in KERNEL_SOURCES else None,
        }
    # the benchmark's own copy (its streaming-peak figure) is not part of the step
    in_step = [k for g, k in kernels.items() if g != "calibration_copy"]
    step = {"copy_calibrated": sum(k["copy_calibrated_bytes_per_step"] for k in in_step),
            "by_request_size": sum(k["sized_bytes_per_step"] for k in in_step)}
    out = {"workload": ti.WORKLOADS[workload].name, "commands": cmds, "steps_counted": PROFILE_STEPS,
           "calibration": {"copy_bytes": copy_b, "fetch_factor": fetch_factor, "write_factor": write_factor,
                           "sized_read_over_copy": cal_sized[0], "sized_write_over_copy": cal_sized[1],
                           "copy_read_requests": {k: cal.get(k) for k in ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum",
                                                                           "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum")}},
           "kernels": kernels, "step": step, "sources_sha256": all_sources_hash()}
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"{tag}_kernel_trace.md"), "w") as f:
        f.write(f"# Kernel durations, {ti.WORKLOADS[workload].name}\n\n")
        f.write("Command (from the repository root, with `TMPDIR=/tmp` exported):\n\n    "
                + cmds["trace"] + "\n\n")
        f.write(f"{2 + len(KERNELS) + 10} steps traced: 2 warm-up, one per timed kernel name (backward on one "
                "stream), 10 timed; the transpose runs in the backward call (`--hoist off`).  In the timed "
                "steps the library's automatic backward may run kernels side by side on two streams (with "
                "the dense rows picked before the sort: the dense rows, the long runs and a second "
                "short-run grid beside the first one, both grids taking their work from a shared counter), "
                "so those durations overlap.  Library kernels only, from `run_kernel_stats.csv`.\n\n")
        f.write("| kernel | calls | average us | total ms | share of GPU time % |\n|---|---|---|---|---|\n")
        for r in trace:
            nm = r["Name"].replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
            nm = nm.replace("tbe::", "")
            f.write(f"| `{nm}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                    f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |\n")
        mf = mfma_rows(workload, trace)
        if mf:
            f.write("\nMatrix-core kernels: work as issued (every MFMA tile, zero padding included) over the "
                    "average duration above, against the dense MFMA peak of the operand type.\n\n")
            f.write("| kernel | operands | GFLOP per launch | average us | achieved TFLOP/s | peak TFLOP/s | "
                    "fraction of peak |\n|---|---|---|---|---|---|---|\n")
            for k, v in mf.items():
                f.write(f"| `{k}` | {v['dtype']} | {v['flops_per_launch'] / 1e9:.2f} | {v['average_us']:.1f} | "
                        f"{v['achieved_TFLOPs']:.1f} | {v['peak_TFLOPs']:.1f} | {v['frac']:.4f} |\n")
    out["mfma_utilisation"] = mf
    with open(os.path.join(out_dir, f"{tag}_traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    with open(os.path.join(out_dir, f"{tag}_hbm_counters.md"), "w") as f:
        f.write(f"# Bytes leaving L2, {ti.WORKLOADS[workload].name}\n\n")
        f.write("Commands (from the repository root, with `TMPDIR=/tmp` exported):\n\n")
        for k, c in cmds.items():
            if k != "trace":
                f.write(f"    {c}\n")
        f.write(f"\n{PROFILE_STEPS} steps counted (`--steps 2 --warmup 1 --dominant short_run`: no per-kernel "
                "scan), transpose in the backward call.  Figures are per step, summed over a kernel's "
                "dispatches (radix passes and the three rle / classify kernels under one name; the pre-sort "
                "sample's own small sort counts under the radix names).\n\n")
        f.write("Two byte counts:\n\n"
                "* copy-calibrated: FETCH_SIZE and WRITE_SIZE scaled by what they read for the library's "
                f"1 GiB copy (`tbe_calibration_copy`): factors x{fetch_factor:.3f} (fetch) and "
                f"x{write_factor:.3f} (write).  FETCH_SIZE prices every non-32-byte read request at 64 "
                "bytes, and the copy issues 128-byte requests, hence the factor;\n"
                "* by request size: 32 x TCC_EA0_RDREQ_32B + 64 x TCC_EA0_RDREQ_64B + 128 x "
                "TCC_EA0_RDREQ_128B read, 32 x (TCC_EA0_WRREQ - TCC_EA0_WRREQ_64B) + 64 x "
                "TCC_EA0_WRREQ_64B written: no fitted factor (on the copy it reads "
                f"{cal_sized[0]:.3f} x the bytes read and {cal_sized[1]:.3f} x the bytes written).\n\n"
                "Both count requests leaving L2 towards memory, so reads the 256 MB Infinity Cache "
                "(MALL) serves are included: they bound HBM traffic from above.  L2 hit rate = "
                "TCC_HIT / (TCC_HIT + TCC_MISS).\n\n")
        f.write("| kernel | dispatches / step | FETCH_SIZE KiB | WRITE_SIZE KiB | copy-calibrated GB | "
                "read by size GB | write by size GB | 32B / 64B / 128B read requests (M) | L2 hit rate |\n"
                "|---|---|---|---|---|---|---|---|---|\n")
        for g, k in sorted(kernels.items(), key=lambda kv: -kv[1]["sized_bytes_per_step"]):
            rq = k["read_requests_per_step"]
            hr = "" if k["l2_hit_rate"] is None else f"{k['l2_hit_rate']:.3f}"
            f.write(f"| `{g}` | {k['dispatches_per_step']:.0f} | {k['fetch_kib_per_step']:.0f} | "
                    f"{k['write_kib_per_step']:.0f} | {k['copy_calibrated_bytes_per_step'] / 1e9:.3f} | "
                    f"{k['sized_read_bytes_per_step'] / 1e9:.3f} | {k['sized_write_bytes_per_step'] / 1e9:.3f} | "
                    f"{rq['32B'] / 1e6:.2f} / {rq['64B'] / 1e6:.2f} / {rq['128B'] / 1e6:.2f} | {hr} |\n")
        f.write(f"| step | | | | {step['copy_calibrated'] / 1e9:.3f} | | | | |\n")
        f.write(f"\nStep by request size: {step['by_request_size'] / 1e9:.3f} GB.\n")
    print(f"wrote {out_dir}/{tag}_*: {len(kernels)} kernels, step {step['by_request_size'] / 1e9:.2f} GB by size")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def batch_stats(bt: ti.Batch, hist_table: int, threshold=256, chunk=256, dense_min=1024,
                dense_rows=128):
    """Host-side statistics of the drawn batch (from the inputs only), per table.  hist_table
    (or -1): the table whose backward goes through the histogram kernels, not the runs.  The
    dense hot rows are picked as the library does after the sort: per eligible table (16 <= D
    <= 128, D % 16 == 0, not the histogram table), its long runs of
    at least dense_min lookups, the dense_rows longest when more qualify (among equal lengths
    the smaller keys; dense_min 0: none).  The library's pre-sort pick counts a sample
    instead, so rows near the cut may differ."""
    idx = bt.indices.cpu().numpy().astype(np.int64)
    off = bt.offsets.cpu().numpy().astype(np.int64)
    B = bt.B
    dmin = max(dense_min, threshold) if dense_min > 0 else 0
    per = []
    for t in range(bt.T):
        lk = idx[off[t * B]:off[(t + 1) * B]]
        c = np.bincount(lk, minlength=bt.E[t])
        c = c[c > 0]
        lg = c >= threshold
        lens = np.diff(off[t * B:(t + 1) * B + 1])
        D = bt.D[t]
        # bags whose gradient slice a short run / a chunked long run reads at least once
        cnt_row = np.bincount(lk, minlength=bt.E[t])
        bag = np.repeat(np.arange(B, dtype=np.int64), lens)
        ok = (dmin > 0 and 16 <= D <= 128 and D % 16 == 0 and t != hist_table)
        cand = np.flatnonzero(lg & (c >= dmin)) if ok else np.zeros(0, dtype=np.int64)  # key order
        if cand.size > dense_rows:   # the longest; among equal lengths the smaller keys
            cand = np.sort(cand[np.lexsort((cand, -c[cand]))[:dense_rows]])
        dl = c[cand]
        dn = np.zeros(c.size, dtype=bool)
        dn[cand] = True
        gl = lg & ~dn                                                # long runs left to the chunks
        row_ids = np.flatnonzero(cnt_row)                            # touched rows, as c is ordered
        row_class = np.zeros(bt.E[t], dtype=np.int8)                 # 1 short, 2 chunked long
        row_class[row_ids[~lg]] = 1
        row_class[row_ids[gl]] = 2
        cls = row_class[lk]
        short_bags = int(np.unique(bag[cls == 1]).size)
        long_bags = int(np.unique(bag[cls == 2]).size)
        per.append(dict(D=D, N=int(lk.size), U=int(c.size), hottest=int(c.max()) if c.size else 0,
                        short_bags=short_bags, long_bags=long_bags,
                        tail=int(np.maximum(lens - 256, 0).sum()),   # lookups past a bag's first 256
                        long_runs=int(lg.sum()), long_lookups=int(c[lg].sum()),
                        short_runs=int((~lg).sum()), short_lookups=int(c[~lg].sum()),
                        chunks=int(((c[lg] + chunk - 1) // chunk).sum()),
                        dense_rows=int(dl.size), dense_lookups=int(dl.sum()),
                        gen_long_runs=int(gl.sum()), gen_long_lookups=int(c[gl].sum()),
                        gen_chunks=int(((c[gl] + chunk - 1) // chunk).sum()), hist=t == hist_table))
    tot = lambda k, only_runs=False: sum(p[k] for p in per if not (only_runs and p["hist"]))
    return dict(N=int(idx.size), TB=bt.T * B, U=tot("U"), hottest=max(p["hottest"] for p in per),
                short_runs=tot("short_runs", True), short_lookups=tot("short_lookups", True),
                long_runs=tot("long_runs", True), long_lookups=tot("long_lookups", True),
                chunks=tot("chunks", True), per_table=per)


def presort_sample(N: int):
    """The pre-sort pick of the dense rows (the library's automatic choice, from 2^26 lookups on):
    (on, sampled keys).  The sample is 64 positions in every S, S the smallest power of two >= 64
    that leaves at most 2^20 of them."""
    if N < 2 ** 26:
        return False, 0
    S = 64
    while 64 * -(-N // S) > 2 ** 20:
        S *= 2
    return True, 64 * -(-N // S)


def radix_passes(total_rows: int, E=None, n_keys: int = 0, all_keys: bool = True):
    """Radix passes over keys in [0, total_rows] at up to 9 bits a pass.  With the tables' rows E
    and the keys sorted, the library's automatic choice: each table sorted on its own on the bits
    of its largest local row id when that takes fewer bits, there are at least 2 tables and at
    most half as many tables as sort blocks (segments of whole 4096-key tiles, at most 4096
    blocks, at least two tiles a block when that still leaves 1024 blocks and twice as many
    blocks as tables, if the sort covers all n_keys: all_keys, no histogram table left out)."""
    kb = max(1, int(total_rows).bit_length())
    passes = -(-kb // 9)
    if E is None or len(E) < 2:
        return passes
    lb = max(1, int(max(E) - 1).bit_length())
    tiles = max(1, -(-int(n_keys) // 4096))
    want = min(4096, tiles)
    two = (tiles + 1) // 2
    if all_keys and want > two and two >= max(1024, 2 * len(E)):
        want = two
    per = -(-tiles // want)
    nblk = -(-max(1, int(n_keys)) // (per * 4096))
    if 2 * len(E) <= nblk and lb < kb and -(-lb // 9) <= passes:
        return -(-lb // 9)
    return passes


def algorithmic_bytes(bt: ti.Batch, st: dict, hoist: bool, dense_P: int = 24, presort: bool = False,
                      sample_keys: int = 0):
    """What each kernel must move per launch (no credit for cache reuse), summed over tables
    with their own D.  hoist: the histogram forward keeps each bag's counts (64 u16) and the
    histogram backward reads them and only the ids past a bag's first 256.  dense_P: the dense
    path's partials per table.  presort: the dense rows are picked before the sort from
    sample_keys sampled lookups, and their lookups leave the sort after its first pass (radix
    figures are then averages over the passes)."""
    s_w = bt.weights.element_size()
    s_i = bt.indices.element_size()
    s_o = bt.offsets.element_size()
    s_p = 4 if bt.psw is not None else 0          # per-sample weight per lookup
    B = bt.B
    per = st["per_table"]
    gen = [p for p in per if not p["hist"]]       # tables the generic kernels serve
    hst = [p for p in per if p["hist"]]
    runs_N = sum(p["N"] for p in gen)              # keys the sort covers
    U = sum(p["U"] for p in gen)
    passes = radix_passes(sum(bt.E), bt.E, bt.num_indices, not any(p["hist"] for p in per))
    kept, U_kept = runs_N, U                       # keys and runs past the first radix pass
    if presort:
        kept -= sum(p["dense_lookups"] for p in gen)
        U_kept -= sum(p["dense_rows"] for p in gen)
    by = {
        # per lookup: index (+ weight) + row; per bag: offset + output row
        "fwd_gather": sum(p["N"] * (s_i + s_p + p["D"] * s_w) + B * (s_o + p["D"] * 4) for p in gen),
        # per lookup: index read, key + payload written (with the pre-sort pick also its two
        # dense-slot bytes); per bag: offset
        "linearize": st["N"] * s_i + runs_N * (8 + (2 if presort else 0)) + st["TB"] * s_o,
        # per pass: keys + payloads read and written (the first pass writes only the kept keys,
        # later passes see only those)
        "radix_downsweep": (runs_N * 8 + kept * 8 + (passes - 1) * kept * 16) / passes,
        "radix_upsweep": (runs_N + (passes - 1) * kept) * 4 / passes,
        # per lookup of a short run: payload (+ weight) + fp32 gradient row; per short run:
        # descriptor, weight row read + write, Adagrad state read + write
        "short_run": sum(p["short_lookups"] * (4 + s_p + p["D"] * 4)
                         + p["short_runs"] * (16 + 2 * p["D"] * s_w + 8) for p in gen),
        # per lookup of a long run: payload (+ weight) + gradient row; per chunk: partial row
        # (the long runs the dense path takes are skipped)
        "grad_accum": sum(p["gen_long_lookups"] * (4 + s_p + p["D"] * 4) + p["gen_chunks"] * (8 + p["D"] * 4)
                          for p in gen),
        # per chunk: partial row read; per long run: descriptor, weight row r/w, state r/w
        "long_apply": sum(p["gen_chunks"] * p["D"] * 4 + p["gen_long_runs"] * (20 + 2 * p["D"] * s_w + 8)
                          for p in gen),
        # per table with dense rows: its ids (with the pre-sort pick the two dense-slot bytes
        # instead; with per-sample weights also the weights), offsets and B x D gradient slice,
        # and its partials (P per table, one row of D floats per dense row each)
        "dense_partial": sum(p["N"] * ((2 if presort else s_i) + s_p) + B * (s_o + p["D"] * 4)
                             + dense_P * p["dense_rows"] * p["D"] * 4 for p in gen if p["dense_rows"]),
        # per dense row: its P partial rows, weight row r/w, state r/w
        "dense_apply": sum(p["dense_rows"] * (dense_P * p["D"] * 4 + 2 * p["D"] * s_w + 8) for p in gen),
        "bounds_indices": st["N"] * s_i,
        "bounds_offsets": 3 * (st["TB"] + 1) * s_o,
        "rle": 3 * kept * 4 + U_kept * 8,
        "classify": U_kept * 8 + U_kept * 16,
    }
    if presort:
        # ids read and keys + payloads written at the sampled positions, the sample's own sort
        # (keys + payloads read and written per pass, keys counted) and run-length encoding,
        # the dense rows' key set (8 x 128 words a table, a power of two) and 8 KB filter filled
        words = 1024
        while words < 8 * 128 * bt.T:
            words *= 2
        by["dense_sample"] = sample_keys * (s_i + 8) + passes * sample_keys * 20 + 3 * sample_keys * 4 \
            + words * 4 + 8192
    for p in hst:
        # per lookup: index; per bag: offset + output (forward) or gradient (backward) row
        by["fwd_hist"] = p["N"] * s_i + B * (s_o + p["D"] * 4) + 64 * p["D"] * s_w
        by["hist_bwd_partial"] = p["N"] * s_i + B * (s_o + p["D"] * 4)
        if hoist:   # + the saved counts, written once and read once
            by["fwd_hist"] += B * 64 * 2
            by["hist_bwd_partial"] = p["tail"] * s_i + B * (s_o + 64 * 2 + p["D"] * 4)
    return by


def compulsory_bytes(bt: ti.Batch, st: dict, ab: dict, presort: bool = False):
    """The bytes each kernel, and the whole step, cannot avoid moving: every input byte read once
    and every output byte written once, with perfect on-chip reuse of anything read twice (a hot
    weight row, a bag's gradient slice read by several of its runs).  Kernels that read nothing
    twice (the transpose, the dense and histogram products, the applies) keep their algorithmic
    bytes `ab`.  Returns (per kernel, step).

    fwd_gather: ids (+ per-sample weights) and offsets once, each touched row once, the output
    once.  short_run: payloads (+ weights) and descriptors once, the gradient slice of every bag
    that one of its runs reads, each short-run row read and written once, its state.  grad_accum:
    payloads once, the gradient slices its chunks read, one partial row written per chunk.
    Step: ids, offsets and per-sample weights once; the output written once and the upstream
    gradient read once; every touched row read by the forward and read and written by the
    backward (separate calls: the rows leave the GPU's caches in between), its state read and
    written; plus the transpose's and the long runs' own traffic as modelled per kernel."""
    s_w = bt.weights.element_size()
    s_i = bt.indices.element_size()
    s_o = bt.offsets.element_size()
    s_p = 4 if bt.psw is not None else 0
    B = bt.B
    per = st["per_table"]
    gen = [p for p in per if not p["hist"]]
    out = dict(ab)
    out["fwd_gather"] = sum(p["N"] * (s_i + s_p) + p["U"] * p["D"] * s_w + B * (s_o + p["D"] * 4) for p in gen)
    out["short_run"] = sum(p["short_lookups"] * (4 + s_p) + p["short_runs"] * (16 + 2 * p["D"] * s_w + 8)
                           + p["short_bags"] * p["D"] * 4 for p in gen)
    out["grad_accum"] = sum(p["gen_long_lookups"] * (4 + s_p) + p["long_bags"] * p["D"] * 4
                            + p["gen_chunks"] * (8 + p["D"] * 4) for p in gen)
    width = sum(bt.D)
    mom = 8 if bt.spec.optimizer == "rowwise_adagrad" else 0
    step = (st["N"] * (s_i + s_p) + (st["TB"] + 1) * s_o + 2 * B * width * 4
            + sum(p["U"] * (3 * p["D"] * s_w + mom) for p in per))
    # the transpose (linearize's key and payload writes, the radix passes, run-length encoding,
    # classification, the pre-sort sample) and the long runs' partials (written, then read)
    passes = radix_passes(sum(bt.E), bt.E, bt.num_indices, not any(p["hist"] for p in per))
    step += (ab.get("linearize", 0) - st["N"] * s_i - st["TB"] * s_o
             + passes * (ab.get("radix_downsweep", 0) + ab.get("radix_upsweep", 0))
             + ab.get("rle", 0) + ab.get("classify", 0) + ab.get("dense_sample", 0)
             + sum(2 * p["gen_chunks"] * p["D"] * 4 for p in gen))
    if ab.get("dense_partial"):
        # the dense path's partials, written and read (its ids or slots and gradient slices are
        # counted above: the slice once for the step)
        dp = ab["dense_apply"] - sum(p["dense_rows"] * (2 * p["D"] * s_w + 8) for p in gen)
        step += 2 * dp + sum(p["N"] * (2 if presort else 0) for p in gen if p["dense_rows"])
    for p in per:
        if p["hist"]:   # the small table's saved counts (hoisted forward), written and read
            step += 2 * B * 64 * 2
    return out, step


def mfma_flops(bt: ti.Batch, st: dict):
    """Matrix-core work per launch of the kernels that use it, as issued (rows and columns of
    every MFMA tile, zero padding included): {kernel: (flops, dtype)}."""
    B = bt.B
    out = {}
    for p in st["per_table"]:
        if p["hist"]:
            D = p["D"]
            # forward: per 16-bag tile, counts (16 x 64) x table (64 x D) on 16x16x16 fp16
            out["fwd_hist"] = (((B + 15) // 16) * 16 * 64 * D * 2, "fp16")
            # backward: per 64-bag step, counts^T (64 rows x 64 bags) x grad (64 bags x 128 columns)
            # on 16x16x4 fp32 (every wave multiplies its 32 columns, padded past D)
            out["hist_bwd_partial"] = (((B + 63) // 64) * 64 * 64 * 128 * 2, "fp32")
    dense = [p for p in st["per_table"] if p["dense_rows"]]
    if dense:
        # per table and 64-bag step: ceil(rows / 16) row tiles x 64 bags x 128 columns, three
        # bf16 parts of the gradient (with per-sample weights times three parts of the weight sums)
        parts = 9 if bt.psw is not None else 3
        out["dense_partial"] = (sum(((B + 63) // 64) * ((p["dense_rows"] + 15) // 16) * 16 * 64 * 128 * 2 * parts
                                    for p in dense), "bf16")
    return out


def calib_copy():
    """The library's plain 16-byte-per-lane copy of 1 GiB, three times: rocprofv3 byte counters
    of this known-size copy calibrate FETCH_SIZE / WRITE_SIZE of the other kernels."""
    n = 1 << 30
    a = torch.zeros(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        tbe.tbe_calibration_copy(a, b, n)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n, "launches": 3}))


def copy_peak_gbps(n: int = 1 << 30, reps: int = 5) -> float:
    """What a plain streaming copy reaches on this GPU (the library's 16-byte-per-lane copy
    of 1 GiB, read + write bytes over the event-timed average)."""
    a = torch.zeros(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    tbe.tbe_calibration_copy(a, b, n)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        tbe.tbe_calibration_copy(a, b, n)
    e1.record()
    torch.cuda.synchronize()
    return 2 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(spec: ti.BatchSpec, seed: int):
    """The CPU oracle, single-threaded, on a bounded sample of the same workload: 2 of its
    tables with every bag (same B, L, id and weight recipe).  Returns lookups/s of
    forward + backward."""
    import oracle
    sample = ti.scaled(spec, T=2, name_suffix=" (2-table sample)")
    bt = ti.make_batch(sample, seed, device="cuda")
    a = dict(E=np.array(bt.E), D=np.array(bt.D), W=bt.weights.double().cpu().numpy(),
             idx=bt.indices.long().cpu().numpy(), off=bt.offsets.long().cpu().numpy(),
             grad=bt.grad_out.double().cpu().numpy(),
             psw=None if bt.psw is None else bt.psw.double().cpu().numpy(),
             mom=None if bt.momentum is None else bt.momentum.double().cpu().numpy())
    odt = {torch.float32: oracle.F32, torch.float16: oracle.F16, torch.bfloat16: oracle.BF16}[bt.w_dtype]
    del bt
    torch.cuda.empty_cache()
    ada = spec.optimizer == "rowwise_adagrad"
    t0 = time.perf_counter()
    oracle.forward(sample.T, sample.B, a["E"], a["D"], a["W"], a["idx"], a["off"], a["psw"])
    if ada:
        oracle.backward(sample.T, sample.B, a["E"], a["D"], odt, a["W"], a["idx"], a["off"], a["psw"],
                        a["grad"], oracle.ROWWISE_ADAGRAD, oracle.f32_literal(spec.lr),
                        oracle.f32_literal(spec.eps), a["mom"])
    else:
        oracle.backward(sample.T, sample.B, a["E"], a["D"], odt, a["W"], a["idx"], a["off"], a["psw"],
                        a["grad"], oracle.SGD, oracle.f32_literal(spec.lr))
    dt = time.perf_counter() - t0
    n = int(a["idx"].size)
    return {"value": n / dt, "unit": "lookups/s", "cores": 1, "kind": "oracle",
            "sample": f"2 of {spec.T} tables, all {sample.B} bags: {n} lookups, forward + transpose + "
                      f"{spec.optimizer} backward in fp64, single thread, {dt:.1f} s",
            "host": f"{host_cpu()}, {os.cpu_count()} logical CPUs visible"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="skewed", choices=sorted(ti.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bounds", default="fused", choices=["fused", "standalone", "off"],
                    help="bounds check in the step: fused into the forward gather (offsets repaired "
                         "by their own kernel), the standalone kernels, or none")
    ap.add_argument("--hoist", default="on", choices=["on", "off"],
                    help="on: the backward's transpose runs inside the forward call on a second "
                         "stream, concurrent with the pooling (tbe_forward_hoisted); off: in the "
                         "backward call")
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--dominant", default=None,
                    help="kernel to time inside the timed region (skips the one-step-per-kernel scan)")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="write profiles/ summaries of --workload from the rocprofv3 output "
                         "directories under DIR (see profile_commands) and exit; no GPU needed")
    ap.add_argument("--profile-commands", action="store_true",
                    help="print the rocprofv3 commands whose output --summarize-profiles reads")
    args = ap.parse_args()
    if args.profile_commands:
        for c in profile_commands(args.workload).values():
            print(c)
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.calib_copy:
        calib_copy()
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = ti.WORKLOADS[args.workload]
    seed = spec.seed
    t0 = time.perf_counter()
    bt = ti.make_batch(spec, seed, device=dev)
    torch.cuda.synchronize()
    log(f"generated {spec.name}: {bt.num_indices} lookups in {time.perf_counter() - t0:.1f} s")
    tables = tbe.Tables(bt.E, bt.D, bt.B, bt.w_dtype, device=dev, pooling_hint=spec.pooling_hint)
    # the histogram kernels take that table when there are no per-sample weights
    hist_table = tables.c.hist_table if bt.psw is None else -1
    st = batch_stats(bt, hist_table)
    log("batch: " + ", ".join(f"{k} {v}" for k, v in st.items() if k != "per_table"))
    out = torch.empty(bt.B, sum(bt.D), dtype=torch.float32, device=dev)
    weighted = bt.psw is not None
    ws = tbe.workspace(tbe.tbe_backward_workspace_bytes(tables, bt.num_indices, weighted), dev)
    bws = tbe.workspace(tbe.tbe_bounds_check_workspace_bytes(tables), dev)
    counts = torch.zeros(2, dtype=torch.int64, device=dev)
    lr, eps = float(np.float32(spec.lr)), float(np.float32(spec.eps))
    if bt.momentum is None:
        bt.momentum = torch.zeros(sum(bt.E), dtype=torch.float32, device=dev)

    def step(hoist=args.hoist == "on", events=None, one_stream=False):
        # one_stream: the backward on one stream (bwd_streams = 1), so that no kernel shares the GPU
        bcfg = tbe.make_config(pretransposed=1 if hoist else 0, bwd_streams=1 if one_stream else 0)
        if events:
            events[0].record()
        if args.bounds == "standalone":
            tbe.tbe_bounds_check(tables, bt.indices, bt.offsets, counts, bws)
        repair = args.bounds == "fused"
        if hoist:
            tbe.tbe_forward_hoisted(tables, bt.weights, bt.indices, bt.offsets, bt.psw, out,
                                    counts if repair else None, bws if repair else None, ws)
        elif repair:
            tbe.tbe_forward_repair(tables, bt.weights, bt.indices, bt.offsets, bt.psw, out, counts, bws)
        else:
            tbe.tbe_forward(tables, bt.weights, bt.indices, bt.offsets, bt.psw, out)
        if events:
            events[1].record()
        if spec.optimizer == "sgd":
            tbe.tbe_backward_sgd(tables, bt.weights, bt.indices, bt.offsets, bt.psw, bt.grad_out,
                                 lr, ws, bcfg)
        else:
            tbe.tbe_backward_rowwise_adagrad(tables, bt.weights, bt.momentum, bt.indices, bt.offsets,
                                             bt.psw, bt.grad_out, lr, eps, ws, bcfg)
        if events:
            events[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # which kernel dominates: one profiled step per kernel (outside the timed region), with the
    # transpose in the backward call and the backward on one stream, so that no two kernels
    # overlap and each time is its own
    per_kernel, launches_per_step = {}, {}
    for k in ([] if args.dominant else KERNELS):
        tbe.tbe_profile_select(k)
        step(hoist=False, one_stream=True)
        n, ms = tbe.tbe_profile_read()
        if n:
            per_kernel[k] = ms
            launches_per_step[k] = n
    tbe.tbe_profile_select(None)
    dominant = args.dominant or max(per_kernel, key=per_kernel.get)
    log("one step per kernel (ms): " + ", ".join(f"{k} {v:.3f}" for k, v in per_kernel.items()))
    # timed region; the dominant kernel's launches are bracketed by HIP events on its stream
    tbe.tbe_profile_select(dominant)
    # events on the calls' stream split each step into its forward and backward calls
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events=ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    launches, dom_ms = tbe.tbe_profile_read()
    tbe.tbe_profile_select(None)
    ms_per_step = elapsed * 1e3 / args.steps
    fwd_ms = float(np.median([a.elapsed_time(b) for a, b, _ in ev]))
    bwd_ms = float(np.median([b.elapsed_time(c) for _, b, c in ev]))
    N = st["N"]
    # the dense path writes one partial per workgroup; its kernel holds 3 workgroups per CU and
    # launches one round of them over the tables, or one workgroup per CU when it runs beside the
    # short runs (the library's automatic backward when the dense rows are picked before the
    # sort and every table's width falls in one short-run bucket)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    presort, sample_keys = presort_sample(N) if bt.psw is None else (False, 0)
    buckets = len({max(4, 1 << max(0, int(d) - 1).bit_length()) for d in bt.D})
    beside = presort and buckets == 1 and any(p["dense_rows"] for p in st["per_table"])
    dense_P = max(1, min(64, 2048 // bt.T, (bt.B + 63) // 64, cus * (1 if beside else 3) // bt.T))
    ab = algorithmic_bytes(bt, st, args.hoist == "on", dense_P, presort, sample_keys)
    dom_avg_ms = dom_ms / max(launches, 1)
    # the byte models give a radix pass's bytes per launch (the passes' average) and every other
    # kernel's bytes per step (a kernel launched per width bucket covers every table once)
    per_launch_model = ("radix_downsweep", "radix_upsweep")
    nl = lambda k: max(1, launches_per_step.get(k, 1))
    per_launch = lambda m, k: m.get(k, 0) if k in per_launch_model else m.get(k, 0) / nl(k)
    per_step = lambda m, k: m.get(k, 0) * nl(k) if k in per_launch_model else m.get(k, 0)
    dom_bytes = per_launch(ab, dominant)
    side_kernels = ("dense_partial", "dense_apply", "grad_accum", "long_apply")
    achieved = dom_bytes / (dom_avg_ms * 1e-3) / 1e9 if dom_avg_ms > 0 else 0.0
    # every kernel of the step
    step_bytes = sum(per_step(ab, k) for k in launches_per_step)
    comp, step_comp = compulsory_bytes(bt, st, ab, presort)
    dom_comp = per_launch(comp, dominant)
    traffic = measured_traffic(args.workload, dominant, launches_per_step.get(dominant, 1))
    step_traffic = measured_step_traffic(args.workload)
    dom_s = dom_avg_ms * 1e-3
    step_s = ms_per_step * 1e-3
    res = {
        "metric": METRIC,
        "value": N / (ms_per_step * 1e-3),
        "unit": "lookups/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": spec.name, "lookups": N, "unique_rows": st["U"], "hottest_run": st["hottest"],
                   "bags": st["TB"], "weights": str(bt.w_dtype).replace("torch.", ""),
                   "indices": str(bt.indices.dtype).replace("torch.", ""), "optimizer": spec.optimizer,
                   "step": {"fused": "offsets repair + forward with fused id check + backward",
                            "standalone": "bounds check + forward + backward",
                            "off": "forward + backward"}[args.bounds]
                   + ("; transpose hoisted into the forward call, concurrent with the pooling on a "
                      "second stream" if args.hoist == "on" else "")},
        # achieved = the kernel's algorithmic bytes (every lookup's row counted, no credit for
        # cache reuse) over its event-timed average launch; a model, not HBM throughput
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     # FETCH_SIZE + WRITE_SIZE per launch, copy-calibrated (profiles/)
                     "traffic": traffic["copy_calibrated"] if traffic else None,
                     "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_ms": dom_avg_ms,
                     "launches_timed": launches,
                     # what the kernel cannot avoid moving (each input byte read once, each output
                     # byte written once), over the same launch time: the bound with headroom
                     "compulsory_bytes_per_launch": dom_comp,
                     "compulsory_frac": dom_comp / dom_s / (HBM_PEAK_GBS * 1e9) if dom_s > 0 else None,
                     # bytes leaving L2 by request size (32/64/128-byte read requests, 32/64-byte
                     # writes), Infinity-Cache hits included, and the kernel's L2 hit rate
                     "traffic_by_request_size": traffic["by_request_size"] if traffic else None,
                     "traffic_frac": traffic["by_request_size"] / dom_s / (HBM_PEAK_GBS * 1e9)
                     if traffic and dom_s > 0 else None,
                     "l2_hit_rate": traffic["l2_hit_rate"] if traffic else None,
                     # what runs on the second stream while the short runs' first grid runs: the
                     # dense rows (one workgroup per CU), then the long runs, then a second
                     # short-run grid taking the runs the first has not reached from a shared
                     # counter; their bytes and every byte of the span over this launch time
                     "beside": ({"kernels": ["dense_partial", "dense_apply", "grad_accum", "long_apply",
                                             "short_run (second grid)"],
                                 "algorithmic_bytes_per_launch": sum(per_step(ab, k) for k in side_kernels),
                                 "combined_frac": (dom_bytes + sum(per_step(ab, k) for k in side_kernels))
                                 / dom_s / (HBM_PEAK_GBS * 1e9)}
                                if beside and dominant == "short_run" and dom_s > 0 else None),
                     "traffic_note": "bytes leaving L2 towards memory: reads served by the Infinity "
                                     "Cache are included, so they bound HBM bytes from above"},
        "step_algorithmic_GBps": step_bytes / step_s / 1e9 if step_bytes else None,
        # bytes leaving L2 over the whole step (rocprofv3 counters in profiles/, every kernel)
        # over the step time, by request size; Infinity-Cache hits included
        "step_traffic_GBps": step_traffic["by_request_size"] / step_s / 1e9 if step_traffic else None,
        # the whole step's algorithmic bytes at the HBM peak, over the measured step time
        "step_roofline_frac": step_bytes / (HBM_PEAK_GBS * 1e9) / step_s if step_bytes else None,
        # the step's compulsory bytes (ids, offsets, output and gradient once; touched rows read
        # by the forward, read and written by the backward; the sort's own passes) at the peak
        "step_compulsory_GB": step_comp / 1e9,
        "step_compulsory_frac": step_comp / (HBM_PEAK_GBS * 1e9) / step_s,
        # medians over the timed steps, HIP events around each call (the forward call holds the
        # hoisted transpose)
        "forward_call_ms": fwd_ms, "backward_call_ms": bwd_ms,
        "forward_lookups_per_s": N / (fwd_ms * 1e-3), "backward_lookups_per_s": N / (bwd_ms * 1e-3),
        "copy_peak_GBps": copy_peak_gbps(),
        # event-timed per kernel, one step each with nothing overlapping (transpose in the backward,
        # backward on one stream)
        "kernel_ms_one_step": per_kernel,
        # what each of those kernels must move per launch (no credit for cache reuse), GB
        "algorithmic_GB_per_launch": {k: per_launch(ab, k) / 1e9 for k in per_kernel if k in ab},
        # what each cannot avoid moving per step (perfect on-chip reuse), GB
        "compulsory_GB_per_step": {k: per_step(comp, k) / 1e9 for k in per_kernel if k in comp},
        # matrix-core kernels: work as issued over their average launch time (one-step scan),
        # against the dense MFMA peak of their operand type
        "mfma_utilisation": {
            k: {"dtype": dt, "flops_per_launch": fl,
                "achieved_TFLOPs": fl / (per_kernel[k] / launches_per_step[k] * 1e-3) / 1e12,
                "peak_TFLOPs": MFMA_PEAK_TFLOPS[dt],
                "frac": fl / (per_kernel[k] / launches_per_step[k] * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[dt]}
            for k, (fl, dt) in mfma_flops(bt, st).items() if per_kernel.get(k)},
    }
    if not args.no_cpu_baseline:
        del ws, out
        torch.cuda.empty_cache()
        log("timing the CPU oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline(spec, seed)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
