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
    "hist_bwd_partial": ["hist_backward.hip", "tbe_device.h"],
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


def measured_step_traffic():
    """Bytes beyond L2 of one whole step (every kernel, every launch) from the committed
    counters, scaled by the copy calibration; None if any library source changed since."""
    path = os.path.join(ROOT, "profiles", "skewed_large_traffic.json")
    try:
        with open(path) as f:
            st = json.load(f)["step"]
    except (OSError, KeyError, ValueError):
        return None
    return st["traffic_bytes"] if st.get("sources_sha256") == all_sources_hash() else None


def measured_traffic(kernel: str):
    """Bytes beyond L2 per launch from the committed rocprofv3 counters, scaled by the copy
    calibration; None if there are none or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", "skewed_large_traffic.json")
    try:
        with open(path) as f:
            prof = json.load(f)
        k = prof["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if k.get("sources_sha256") != kernel_sources_hash(kernel):
        return None
    c = prof["calibration"]
    return (k["fetch_kib"] * c["fetch_factor"] + k["write_kib"] * c["write_factor"]) * 1024


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def batch_stats(bt: ti.Batch, hist_table: int, threshold=256, chunk=256, dense_min=1024,
                dense_rows=128):
    """Host-side statistics of the drawn batch (from the inputs only), per table.  hist_table
    (or -1): the table whose backward goes through the histogram kernels, not the runs.  The
    dense hot rows are picked as the library does after the sort: per eligible table (no
    per-sample weights, 16 <= D <= 128, D % 16 == 0, not the histogram table), its long runs of
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
        ok = (dmin > 0 and bt.psw is None and 16 <= D <= 128 and D % 16 == 0 and t != hist_table)
        cand = np.flatnonzero(lg & (c >= dmin)) if ok else np.zeros(0, dtype=np.int64)  # key order
        if cand.size > dense_rows:   # the longest; among equal lengths the smaller keys
            cand = np.sort(cand[np.lexsort((cand, -c[cand]))[:dense_rows]])
        dl = c[cand]
        dn = np.zeros(c.size, dtype=bool)
        dn[cand] = True
        gl = lg & ~dn                                                # long runs left to the chunks
        per.append(dict(D=D, N=int(lk.size), U=int(c.size), hottest=int(c.max()) if c.size else 0,
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


def radix_passes(total_rows: int):
    """Radix passes over keys in [0, total_rows] at up to 9 bits a pass."""
    return -(-max(1, int(total_rows).bit_length()) // 9)


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
    passes = radix_passes(sum(bt.E))
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
        # instead), offsets and B x D gradient slice, and its partials (P per table, one row of
        # D floats per dense row each)
        "dense_partial": sum(p["N"] * (2 if presort else s_i) + B * (s_o + p["D"] * 4)
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
        # the dense rows' key set (4 x 128 slots a table, a power of two) and 8 KB filter filled
        slots = 1024
        while slots < 4 * 128 * bt.T:
            slots *= 2
        by["dense_sample"] = sample_keys * (s_i + 8) + passes * sample_keys * 20 + 3 * sample_keys * 4 \
            + slots * 4 + 8192
    for p in hst:
        # per lookup: index; per bag: offset + output (forward) or gradient (backward) row
        by["fwd_hist"] = p["N"] * s_i + B * (s_o + p["D"] * 4) + 64 * p["D"] * s_w
        by["hist_bwd_partial"] = p["N"] * s_i + B * (s_o + p["D"] * 4)
        if hoist:   # + the saved counts, written once and read once
            by["fwd_hist"] += B * 64 * 2
            by["hist_bwd_partial"] = p["tail"] * s_i + B * (s_o + 64 * 2 + p["D"] * 4)
    return by


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
        # bf16 parts of the gradient
        out["dense_partial"] = (sum(((B + 63) // 64) * ((p["dense_rows"] + 15) // 16) * 16 * 64 * 128 * 2 * 3
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
    args = ap.parse_args()
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

    def step(hoist=args.hoist == "on", events=None):
        bcfg = tbe.make_config(pretransposed=1) if hoist else None
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
    # transpose in the backward call so that no two kernels overlap and each time is its own
    per_kernel, launches_per_step = {}, {}
    for k in ([] if args.dominant else KERNELS):
        tbe.tbe_profile_select(k)
        step(hoist=False)
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
    # launches one round of them over the tables
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    dense_P = max(1, min(64, 2048 // bt.T, (bt.B + 63) // 64, cus * 3 // bt.T))
    presort, sample_keys = presort_sample(N) if bt.psw is None else (False, 0)
    ab = algorithmic_bytes(bt, st, args.hoist == "on", dense_P, presort, sample_keys)
    dom_avg_ms = dom_ms / max(launches, 1)
    dom_bytes = ab.get(dominant, 0)
    achieved = dom_bytes / (dom_avg_ms * 1e-3) / 1e9 if dom_avg_ms > 0 else 0.0
    # every kernel of the step, times its launches per step (radix: one per pass)
    step_bytes = sum(ab.get(k, 0) * n for k, n in launches_per_step.items())
    step_traffic = measured_step_traffic() if args.workload == "skewed" else None
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
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(dominant) if args.workload == "skewed" else None,
                     "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_ms": dom_avg_ms,
                     "launches_timed": launches},
        "step_algorithmic_GBps": step_bytes / (ms_per_step * 1e-3) / 1e9 if step_bytes else None,
        # bytes beyond L2 of the whole step (rocprofv3 counters in profiles/, every kernel) over
        # the step time: the achieved rate the counters see (Infinity-Cache hits included)
        "step_traffic_GBps": step_traffic / (ms_per_step * 1e-3) / 1e9 if step_traffic else None,
        # the whole step's algorithmic bytes at the HBM peak, over the measured step time
        "step_roofline_frac": step_bytes / (HBM_PEAK_GBS * 1e9) / (ms_per_step * 1e-3) if step_bytes else None,
        # medians over the timed steps, HIP events around each call (the forward call holds the
        # hoisted transpose)
        "forward_call_ms": fwd_ms, "backward_call_ms": bwd_ms,
        "forward_lookups_per_s": N / (fwd_ms * 1e-3), "backward_lookups_per_s": N / (bwd_ms * 1e-3),
        "copy_peak_GBps": copy_peak_gbps(),
        # event-timed per kernel, one step each with nothing overlapping (transpose in the backward)
        "kernel_ms_one_step": per_kernel,
        # what each of those kernels must move per launch (no credit for cache reuse), GB
        "algorithmic_GB_per_launch": {k: ab[k] / 1e9 for k in per_kernel if k in ab},
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
