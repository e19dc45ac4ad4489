"""Host logic of bench.py: batch statistics, algorithmic and compulsory bytes on a small batch,
and the profile summaries from rocprofv3-shaped CSV files (CPU)."""
import csv
import json
import os

import numpy as np
import torch

import bench
import tbe_inputs as ti


def _spec():
    tables = (ti.TableSpec(64, 128, ("fixed", 100)),
              ti.TableSpec(500, 32, ("poisson", 30.0, None, None), ("zipf", 1.2, None)))
    return ti.BatchSpec("bench host", tables, B=300, w_dtype=torch.float16, w_range=0.05,
                        pooling_hint=(100, 30))


def test_batch_stats_partition_the_lookups():
    bt = ti.make_batch(_spec(), 3, device="cpu")
    st = bench.batch_stats(bt, hist_table=-1, threshold=20, chunk=8)
    idx, off = bt.indices.numpy(), bt.offsets.numpy()
    assert st["N"] == idx.size and st["TB"] == 2 * 300
    assert st["short_lookups"] + st["long_lookups"] == idx.size
    uniq = sum(np.unique(idx[off[t * 300]:off[(t + 1) * 300]]).size for t in range(2))
    assert st["U"] == uniq == st["short_runs"] + st["long_runs"]
    # table 0: 30000 lookups over 64 rows, every row long (>= 20)
    p0 = st["per_table"][0]
    assert p0["long_lookups"] == 30000 and p0["short_runs"] == 0
    # with table 0 on the histogram kernels, the run statistics cover table 1 only
    sh = bench.batch_stats(bt, hist_table=0, threshold=20, chunk=8)
    p1 = sh["per_table"][1]
    assert sh["short_lookups"] + sh["long_lookups"] == p1["N"]


def test_algorithmic_bytes_by_hand():
    bt = ti.make_batch(_spec(), 4, device="cpu")
    st = bench.batch_stats(bt, hist_table=0)
    ab = bench.algorithmic_bytes(bt, st, hoist=False)
    p1 = st["per_table"][1]
    # generic forward: table 1 only; 8-byte ids, 2-byte weights, fp32 output rows of 32
    assert ab["fwd_gather"] == p1["N"] * (8 + 32 * 2) + 300 * (8 + 32 * 4)
    # the histogram table: its ids, one offset and one 128-wide fp32 row per bag, the table once
    assert ab["fwd_hist"] == 30000 * 8 + 300 * (8 + 128 * 4) + 64 * 128 * 2
    assert ab["radix_downsweep"] == p1["N"] * 16
    # hoisted: the forward writes 64 u16 counts a bag, the backward reads them, the gradient
    # rows and offsets, and no ids (no bag is longer than 256)
    assert ab["hist_bwd_partial"] == 30000 * 8 + 300 * (8 + 128 * 4)
    ah = bench.algorithmic_bytes(bt, st, hoist=True)
    assert ah["fwd_hist"] == ab["fwd_hist"] + 300 * 128
    assert ah["hist_bwd_partial"] == 300 * (8 + 128 + 128 * 4)


def test_tail_lookups_past_256():
    tables = (ti.TableSpec(64, 64, ("fixed", 300)), ti.TableSpec(50, 16, ("fixed", 2)))
    bt = ti.make_batch(ti.BatchSpec("tails", tables, B=20, w_dtype=torch.float16, w_range=0.05,
                                    pooling_hint=(300, 2)), 5, device="cpu")
    st = bench.batch_stats(bt, hist_table=0)
    assert st["per_table"][0]["tail"] == 20 * 44 and st["per_table"][1]["tail"] == 0
    ah = bench.algorithmic_bytes(bt, st, hoist=True)
    assert ah["hist_bwd_partial"] == 20 * 44 * 8 + 20 * (8 + 128 + 64 * 4)


def test_dense_rows_statistics():
    """The dense hot rows: per eligible table, long runs of >= dense_min lookups, the 128
    longest when more qualify (equal lengths: the smaller keys); their lookups leave the chunk
    and apply bytes for the dense kernels'."""
    tables = (ti.TableSpec(300, 128, ("fixed", 40)),      # 300 rows x ~133 lookups: all long
              ti.TableSpec(50, 200, ("fixed", 40)),       # D = 200: not eligible
              ti.TableSpec(64, 64, ("fixed", 40)))
    bt = ti.make_batch(ti.BatchSpec("dense stats", tables, B=1000, w_dtype=torch.float16,
                                    w_range=0.05), 6, device="cpu")
    st = bench.batch_stats(bt, hist_table=-1, threshold=64, chunk=64, dense_min=100)
    p0, p1, p2 = st["per_table"]
    idx, off = bt.indices.numpy().astype(np.int64), bt.offsets.numpy().astype(np.int64)
    c0 = np.bincount(idx[off[0]:off[1000]], minlength=300)
    q = np.flatnonzero(c0 >= 100)
    assert q.size > 128
    # brute force: sort the qualifying rows by (lookups descending, row ascending), keep 128
    want = sorted(sorted(q.tolist(), key=lambda r: (-int(c0[r]), r))[:128])
    assert p0["dense_rows"] == len(want) == 128 and p0["dense_lookups"] == int(c0[want].sum())
    assert p0["dense_lookups"] >= int(np.sort(c0[q])[::-1][:128].sum())   # the top 128 counts
    assert p0["gen_long_lookups"] + p0["dense_lookups"] == p0["long_lookups"]
    assert p1["dense_rows"] == 0 and p1["gen_long_lookups"] == p1["long_lookups"]
    assert p2["dense_rows"] == 64                 # every row of the 64-row table
    ab = bench.algorithmic_bytes(bt, st, hoist=False, dense_P=4)
    assert ab["dense_partial"] == sum(p["N"] * 8 + 1000 * (8 + p["D"] * 4) + 4 * p["dense_rows"] * p["D"] * 4
                                      for p in (p0, p2))
    assert ab["dense_apply"] == sum(p["dense_rows"] * (4 * p["D"] * 4 + 2 * p["D"] * 2 + 8) for p in (p0, p2))


def test_mfma_flops():
    bt = ti.make_batch(_spec(), 4, device="cpu")
    st = bench.batch_stats(bt, hist_table=0)
    fl = bench.mfma_flops(bt, st)
    # 300 bags: 19 tiles of 16 bags, counts 16 x 64 times the 64 x 128 table; 5 steps of 64 bags
    assert fl["fwd_hist"] == (19 * 16 * 64 * 128 * 2, "fp16")
    assert fl["hist_bwd_partial"] == (5 * 64 * 64 * 128 * 2, "fp32")
    # the Zipf table's hottest rows take the dense path: per 64-bag step, 16-row tiles x 64 bags
    # x 128 columns, three bf16 parts
    nd = st["per_table"][1]["dense_rows"]
    assert nd >= 1 and fl["dense_partial"] == (5 * ((nd + 15) // 16) * 16 * 64 * 128 * 2 * 3, "bf16")


def test_weighted_batches_take_dense_rows():
    """With per-sample weights the dense rows are picked as without (per-bag sums of the weights
    replace the counts): the same rows, the weights read besides the ids, and nine bf16 part
    products per tile instead of three (no histogram table: it does not take weighted calls)."""
    plain = ti.make_batch(_spec(), 4, device="cpu")
    wtd = ti.make_batch(_spec().replace(weighted=True), 4, device="cpu")
    sp, sw = bench.batch_stats(plain, hist_table=-1), bench.batch_stats(wtd, hist_table=-1)
    assert [p["dense_rows"] for p in sw["per_table"]] == [p["dense_rows"] for p in sp["per_table"]]
    assert sum(p["dense_rows"] for p in sw["per_table"]) > 0
    fp, fw = bench.mfma_flops(plain, sp), bench.mfma_flops(wtd, sw)
    assert fw["dense_partial"][0] == 3 * fp["dense_partial"][0]
    ap = bench.algorithmic_bytes(plain, sp, hoist=False, dense_P=4)
    aw = bench.algorithmic_bytes(wtd, sw, hoist=False, dense_P=4)
    assert aw["dense_partial"] - ap["dense_partial"] == 4 * sum(p["N"] for p in sw["per_table"] if p["dense_rows"])


def test_presort_sample_and_bytes():
    """The pre-sort pick: from 2^26 lookups on, at most 2^20 sampled keys (64 in every power of
    two S); the dense rows' lookups leave the radix passes after the first, and the runs."""
    assert bench.presort_sample(2 ** 26 - 1) == (False, 0)
    on, k = bench.presort_sample(83_897_668)
    assert on and k == 64 * -(-83_897_668 // 8192) and k <= 2 ** 20
    assert bench.radix_passes(64_000_000) == 3 and bench.radix_passes(511) == 1
    # by table: 32 tables of 2M rows (21 bits, three passes either way); 32 tables of 2^17 rows
    # take two passes instead of three once there are 64 sort blocks
    assert bench.radix_passes(64_000_000, [2_000_000] * 32, 84_000_000) == 3
    assert bench.radix_passes(32 << 17, [1 << 17] * 32, 64 * 4096) == 2
    assert bench.radix_passes(32 << 17, [1 << 17] * 32, 63 * 4096) == 3
    tables = (ti.TableSpec(300, 128, ("fixed", 40)), ti.TableSpec(64, 64, ("fixed", 40)))
    bt = ti.make_batch(ti.BatchSpec("presort bytes", tables, B=1000, w_dtype=torch.float16,
                                    w_range=0.05), 7, device="cpu")
    st = bench.batch_stats(bt, hist_table=-1, threshold=64, chunk=64, dense_min=100)
    plain = bench.algorithmic_bytes(bt, st, hoist=False)
    pre = bench.algorithmic_bytes(bt, st, hoist=False, presort=True, sample_keys=4096)
    N = st["N"]
    dl = sum(p["dense_lookups"] for p in st["per_table"])
    kept = N - dl
    assert dl > 0 and plain["radix_downsweep"] == N * 16     # 364 rows: one pass
    assert pre["radix_downsweep"] == N * 8 + kept * 8 and pre["radix_upsweep"] == N * 4
    assert pre["rle"] == 3 * kept * 4 + (st["U"] - 128 - 64) * 8
    assert pre["linearize"] == plain["linearize"] + 2 * N and "dense_sample" in pre
    # the dense kernel reads two slot bytes a lookup instead of its 8-byte id
    assert plain["dense_partial"] - pre["dense_partial"] == N * 6


def test_compulsory_bytes_by_hand():
    """Each touched row once, each bag's gradient slice once per kernel, ids and offsets once."""
    bt = ti.make_batch(_spec(), 8, device="cpu")
    st = bench.batch_stats(bt, hist_table=0, threshold=20, chunk=8, dense_min=0)
    ab = bench.algorithmic_bytes(bt, st, hoist=False)
    comp, step = bench.compulsory_bytes(bt, st, ab)
    p1 = st["per_table"][1]
    idx, off = bt.indices.numpy().astype(np.int64), bt.offsets.numpy().astype(np.int64)
    lk = idx[off[300]:off[600]]
    bag = np.repeat(np.arange(300), np.diff(off[300:601]))
    c = np.bincount(lk, minlength=500)
    short = (c[lk] < 20)
    assert p1["short_bags"] == np.unique(bag[short]).size and p1["long_bags"] == np.unique(bag[~short]).size
    assert comp["fwd_gather"] == p1["N"] * 8 + p1["U"] * 32 * 2 + 300 * (8 + 32 * 4)
    assert comp["short_run"] == (p1["short_lookups"] * 4 + p1["short_runs"] * (16 + 2 * 32 * 2 + 8)
                                 + p1["short_bags"] * 32 * 4)
    assert comp["grad_accum"] == p1["gen_long_lookups"] * 4 + p1["long_bags"] * 32 * 4 + p1["gen_chunks"] * (8 + 32 * 4)
    assert comp["short_run"] < ab["short_run"] and comp["fwd_gather"] < ab["fwd_gather"]
    assert comp["linearize"] == ab["linearize"] and comp["rle"] == ab["rle"]
    # the step: ids, offsets, output and gradient once, rows three times (+ state: SGD has none)
    base = st["N"] * 8 + 601 * 8 + 2 * 300 * 160 * 4 + sum(p["U"] * 3 * p["D"] * 2 for p in st["per_table"])
    assert step > base and step < base + 10 * st["N"] * 20


def test_kernel_groups():
    g = bench.kernel_group
    assert g("void tbe::(anonymous namespace)::short_run_kernel<1, 128, 1, 2, 1, false, 4, 2>(float*)") == "short_run"
    assert g("tbe::(anonymous namespace)::rle_write(unsigned int const*)") == "rle"
    assert g("void tbe::classify_count(int)") == "classify"
    assert g("tbe::(anonymous namespace)::bounds_offsets_reduce<long>(long const*)") == "bounds_offsets"
    assert g("tbe::(anonymous namespace)::radix_downsweep(int)") == "radix_downsweep"
    assert g("tbe::(anonymous namespace)::calibration_copy_kernel(float4 const*)") == "calibration_copy"


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_profile_summaries_from_counter_files(tmp_path):
    """Counter files shaped like rocprofv3's: bytes by request size need no factor (the copy's
    1 GiB of 128-byte reads reads back as 1 GiB), FETCH_SIZE is scaled by the copy's factor,
    per-step figures sum a kernel's dispatches over the counted steps."""
    root = tmp_path / "prof"
    K = "void tbe::(anonymous namespace)::short_run_kernel<1, 128>(float*)"
    C = "tbe::(anonymous namespace)::calibration_copy_kernel(float4 const*)"
    GiB = 1 << 30
    def ctr(kernel, values, n):
        return [{"Kernel_Name": kernel, "Counter_Name": c, "Counter_Value": v}
                for _ in range(n) for c, v in values.items()]
    copy = {"fetch": {"FETCH_SIZE": GiB / 2 / 1024}, "write": {"WRITE_SIZE": GiB / 1024},
            "rd": {"TCC_EA0_RDREQ_sum": GiB / 128, "TCC_EA0_RDREQ_32B_sum": 0, "TCC_EA0_RDREQ_64B_sum": 0,
                   "TCC_EA0_RDREQ_128B_sum": GiB / 128},
            "wr": {"TCC_EA0_WRREQ_sum": GiB / 64, "TCC_EA0_WRREQ_64B_sum": GiB / 64, "TCC_HIT_sum": 0,
                   "TCC_MISS_sum": GiB / 128}}
    kern = {"fetch": {"FETCH_SIZE": 1000.0}, "write": {"WRITE_SIZE": 100.0},
            "rd": {"TCC_EA0_RDREQ_sum": 30.0, "TCC_EA0_RDREQ_32B_sum": 10.0, "TCC_EA0_RDREQ_64B_sum": 10.0,
                   "TCC_EA0_RDREQ_128B_sum": 10.0},
            "wr": {"TCC_EA0_WRREQ_sum": 8.0, "TCC_EA0_WRREQ_64B_sum": 6.0, "TCC_HIT_sum": 75.0,
                   "TCC_MISS_sum": 25.0}}
    for name in ("fetch", "write", "rd", "wr"):
        _write_csv(str(root / f"calib_{name}" / "host" / "1" / "run_counter_collection.csv"), ctr(C, copy[name], 3))
        _write_csv(str(root / f"skewed_{name}" / "host" / "2" / "run_counter_collection.csv"),
                   ctr(K, kern[name], 2 * bench.PROFILE_STEPS))
    _write_csv(str(root / "skewed_trace" / "host" / "3" / "run_kernel_stats.csv"),
               [{"Name": K, "Calls": 30, "TotalDurationNs": 9e7, "AverageNs": 3e6, "Percentage": 35.0}])
    out = tmp_path / "out"
    bench.summarize_profiles(str(root), "skewed", str(out))
    j = json.load(open(out / "skewed_large_traffic.json"))
    cal = j["calibration"]
    assert abs(cal["fetch_factor"] - 2.0) < 1e-12 and abs(cal["write_factor"] - 1.0) < 1e-12
    assert abs(cal["sized_read_over_copy"] - 1.0) < 1e-12 and abs(cal["sized_write_over_copy"] - 1.0) < 1e-12
    k = j["kernels"]["short_run"]
    assert k["dispatches_per_step"] == 2
    assert k["sized_read_bytes_per_step"] == 2 * (32 * 10 + 64 * 10 + 128 * 10)
    assert k["sized_write_bytes_per_step"] == 2 * (32 * 2 + 64 * 6)
    assert k["copy_calibrated_bytes_per_step"] == 2 * (1000 * 2 + 100) * 1024
    assert k["l2_hit_rate"] == 0.75
    assert "short_run" in open(out / "skewed_large_kernel_trace.md").read()
    assert "| `short_run` |" in open(out / "skewed_large_hbm_counters.md").read()


def test_mfma_rows_histogram():
    """Matrix-core utilisation from a trace row: the histogram forward issues one 16x16x16 fp16
    tile product per 16 bags and 16 columns, counts (16 x 64) by table (64 x 128), so
    131072 bags x 64 x 128 x 2 = 2^31 flops; at 50 us that is 42.9 TFLOP/s of 2500."""
    K = "void tbe::(anonymous namespace)::fwd_hist_kernel<long, long, true>(unsigned short const*)"
    rows = [{"Name": K, "Calls": 31, "TotalDurationNs": 31 * 5e4, "AverageNs": 5e4, "Percentage": 9.0},
            {"Name": "void tbe::(anonymous namespace)::short_run_kernel<1>(float*)", "Calls": 31,
             "TotalDurationNs": 31 * 1e5, "AverageNs": 1e5, "Percentage": 12.0}]
    mf = bench.mfma_rows("histogram", rows)
    assert set(mf) == {"fwd_hist"}
    assert mf["fwd_hist"]["flops_per_launch"] == 2 ** 31 and mf["fwd_hist"]["dtype"] == "fp16"
    assert abs(mf["fwd_hist"]["achieved_TFLOPs"] - 2 ** 31 / 5e-5 / 1e12) < 1e-9
    assert abs(mf["fwd_hist"]["frac"] - 2 ** 31 / 5e-5 / 1e12 / 2500.0) < 1e-12
    assert bench.mfma_rows("histogram", rows[1:]) == {}
