"""Transpose and routing parity: sorted keys, payload order, runs and classification are
compared with the oracle bit for bit (compacted lists as sorted sets with exact counts)."""
import numpy as np
import pytest
import torch

import bwd_tbe_fwd_amd as tbe
import oracle
import tbe_inputs as ti
from gpu_util import DevBatch, flush_print, host_arrays
from test_gpu_forward import WORKLOAD_NAMES, mixed_spec, small_spec

pytestmark = pytest.mark.gpu


def gpu_transpose(db: DevBatch, weighted: bool, cfg=None):
    ws = db.workspace(cfg, weighted)
    view = tbe.tbe_transpose(db.tables, db.idx, db.off, weighted, ws, cfg)
    torch.cuda.synchronize()
    N = db.idx.numel()
    cnt = tbe.device_view(view.counters, 16, torch.int32, ws).cpu().numpy()
    runs = int(cnt[tbe.COUNTER_RUNS])
    res = dict(
        counters=cnt,
        keys=tbe.device_view(view.sorted_keys, N, torch.int32, ws).cpu().numpy().view(np.uint32),
        payload=tbe.device_view(view.sorted_payload, N, torch.int32, ws).cpu().numpy().view(np.uint32),
        run_key=tbe.device_view(view.run_key, runs, torch.int32, ws).cpu().numpy().view(np.uint32),
        run_start=tbe.device_view(view.run_start, runs + 1, torch.int32, ws).cpu().numpy().view(np.uint32),
    )
    nl = int(cnt[tbe.COUNTER_LONG])
    nc = int(cnt[tbe.COUNTER_CHUNKS])
    res["long"] = tbe.device_view(view.long_list, 4 * nl, torch.int32, ws).cpu().numpy().view(np.uint32).reshape(nl, 4)
    res["long_table"] = tbe.device_view(view.long_table, nl, torch.int32, ws).cpu().numpy()
    res["chunks"] = tbe.device_view(view.chunk_list, 2 * nc, torch.int32, ws).cpu().numpy().view(np.uint32).reshape(nc, 2)
    res["short"] = {}
    for b in range(tbe.NUM_BUCKETS):
        ns = int(cnt[tbe.COUNTER_SHORT0 + b])
        if view.short_list[b]:
            res["short"][b] = tbe.device_view(view.short_list[b], 4 * ns, torch.int32, ws).cpu().numpy().view(np.uint32).reshape(ns, 4)
        else:
            assert ns == 0
    res["view"] = view
    return res


def check_transpose(bt, weighted, cfg=None, threshold=256, chunk=256, what=""):
    db = DevBatch(bt)
    g = gpu_transpose(db, weighted, cfg)
    a = host_arrays(bt)
    tr = oracle.transpose(a["T"], a["B"], a["E"], a["idx"], a["off"])
    N = a["idx"].size
    assert np.array_equal(g["keys"].astype(np.int64), tr["sorted_key"]), what
    exp_pay = tr["sorted_pos"] if weighted else tr["sorted_bag"]
    assert np.array_equal(g["payload"].astype(np.int64), exp_pay), what
    assert g["counters"][tbe.COUNTER_RUNS] == tr["num_runs"]
    assert np.array_equal(g["run_key"].astype(np.int64), tr["run_key"])
    assert np.array_equal(g["run_start"][:-1].astype(np.int64), tr["run_start"])
    assert int(g["run_start"][-1]) == N
    c = oracle.classify(a["T"], a["E"], a["D"], tr["run_key"], tr["run_len"], threshold, chunk)
    # long runs: same set of (key, start, len), chunk plan consistent
    exp_long = np.stack([tr["run_key"], tr["run_start"], tr["run_len"]], 1)[c["is_long"]]
    got_long = g["long"][:, :3].astype(np.int64)
    assert got_long.shape[0] == exp_long.shape[0]
    assert np.array_equal(got_long[np.lexsort(got_long.T[::-1])], exp_long[np.lexsort(exp_long.T[::-1])])
    assert g["counters"][tbe.COUNTER_CHUNKS] == c["num_chunks"]
    seen = np.zeros(c["num_chunks"], dtype=bool)
    base = np.concatenate([[0], np.cumsum(a["E"])])
    for li, (key, start, ln, cb) in enumerate(g["long"]):
        nch = -(-int(ln) // chunk)
        assert int(g["long_table"][li]) == int(np.searchsorted(base, key, side="right") - 1)
        for k in range(nch):
            assert tuple(g["chunks"][cb + k]) == (li, k)
            seen[cb + k] = True
    assert seen.all()
    # short runs per bucket
    for b in range(tbe.NUM_BUCKETS):
        want = ~c["is_long"] & (c["bucket"] == tbe.BUCKET_D[b])
        exp = np.stack([tr["run_key"], tr["run_start"], tr["run_len"]], 1)[want]
        got = g["short"].get(b, np.zeros((0, 4), np.uint32))[:, :3].astype(np.int64)
        assert got.shape == exp.shape, (what, b, got.shape, exp.shape)
        if exp.size:
            assert np.array_equal(got[np.lexsort(got.T[::-1])], exp[np.lexsort(exp.T[::-1])])
    return g, tr


@pytest.mark.parametrize("n", WORKLOAD_NAMES)
@pytest.mark.parametrize("weighted", [False, True])
def test_transpose_configs_small(n, weighted):
    spec = small_spec(n)
    flush_print(f"transpose {n} weighted={weighted}")
    bt = ti.make_batch(spec)
    check_transpose(bt, weighted, what=n)


@pytest.mark.parametrize("threshold,chunk", [(10 ** 9, 256), (256, 256), (8, 8), (4, 2), (1, 1)])
def test_transpose_routing_sweep(threshold, chunk):
    bt = ti.make_batch(small_spec("skewed"), 15)
    cfg = tbe.make_config(long_threshold=threshold, chunk=chunk)
    check_transpose(bt, False, cfg, threshold, chunk, f"t={threshold} c={chunk}")


def test_transpose_mixed_D_buckets_and_int32():
    bt = ti.make_batch(mixed_spec(torch.float16, torch.int32, torch.int32, False), 5)
    g, _ = check_transpose(bt, False, tbe.make_config(long_threshold=16, chunk=8), 16, 8, "mixed")
    assert len(g["short"]) >= 6


def test_transpose_many_sort_blocks():
    # more radix blocks than tiles per block: exercises block boundaries inside runs
    bt = ti.make_batch(ti.scaled(ti.WORKLOADS["skewed"], B=3000, E_div=400, T=3), 8)
    check_transpose(bt, False, tbe.make_config(sort_blocks=7), what="7 sort blocks")
    check_transpose(bt, True, tbe.make_config(sort_blocks=4096), what="max sort blocks")


def test_transpose_tutorial_batch_statistics():
    """The tutorial's seed-1 batch (regenerated from its prose): the GPU routing reproduces the
    printed short/long/chunk counts of the threshold sweep."""
    from test_oracle_pins import _golden, _tutorial_batch
    gold = _golden("tutorial_stats.json")
    T, E, B, D, ids, off = _tutorial_batch()
    spec = ti.BatchSpec("tutorial", tuple(ti.TableSpec(E, D) for _ in range(T)), B=B,
                        w_dtype=torch.float32, w_range=0.1)
    bt = ti.make_batch(spec, 0)
    bt.indices = torch.from_numpy(ids)
    bt.offsets = torch.from_numpy(off)
    for row in gold["sweep"]:
        cfg = tbe.make_config(long_threshold=min(row["threshold"], 2 ** 31 - 1), chunk=row["chunk"])
        g, tr = check_transpose(bt, False, cfg, row["threshold"], row["chunk"], str(row))
        cnt = g["counters"]
        assert int(cnt[tbe.COUNTER_LONG]) == row["long"]
        assert int(cnt[tbe.COUNTER_SHORT0:tbe.COUNTER_SHORT0 + tbe.NUM_BUCKETS].sum()) == row["short"]
        assert int(cnt[tbe.COUNTER_CHUNKS]) == row["chunks"]
        assert int(cnt[tbe.COUNTER_RUNS]) == gold["unique_rows"]


BY_TABLE_CASES = [("skewed", dict(B=3000, E_div=400, T=8), False),
                  ("skewed", dict(B=3000, E_div=400, T=8), True),
                  ("uniform", dict(B=2000, E_div=100, T=6), False),
                  ("mixed", dict(B=1500, E_div=50), True)]


@pytest.mark.parametrize("name,kw,weighted", BY_TABLE_CASES)
def test_transpose_by_table(name, kw, weighted):
    """Each table's lookups sorted on their own, on the bits of the local row id
    (sort_by_table = 1): the oracle's transpose bit for bit with the automatic, 64 and the
    maximum number of sort blocks (table boundaries inside blocks' ranges, tables of very
    different sizes), and the same as one sort of the linearized ids."""
    bt = ti.make_batch(ti.scaled(ti.WORKLOADS[name], **kw), 21)
    flush_print(f"by table {name} {kw} weighted={weighted} N={bt.num_indices}")
    for blocks in (0, 64, 4096):
        cfg = tbe.make_config(sort_by_table=1, sort_blocks=blocks)
        g, _ = check_transpose(bt, weighted, cfg, what=f"{name} by table, {blocks} blocks")
        assert g["view"].sorted_by_table == 1
    g, _ = check_transpose(bt, weighted, tbe.make_config(sort_by_table=-1), what=f"{name} one sort")
    assert g["view"].sorted_by_table == 0


def test_transpose_by_table_edges():
    """By table with an empty table first and one in the middle, a one-row table and the
    largest table setting the passes (2^21 rows: three 7-bit passes against 22 bits of
    linearized ids).  Out-of-range ids, whose lookups leave the sort, are covered by the whole
    steps in test_gpu_hoisted."""
    tables = (ti.TableSpec(5000, 64, ("fixed", 0)),
              ti.TableSpec(1, 64, ("poisson", 3.0, None, None)),
              ti.TableSpec(1 << 21, 128, ("poisson", 12.0, None, None), ("zipf", 1.05, 20000)),
              ti.TableSpec(700, 64, ("fixed", 0)),
              ti.TableSpec(300_000, 32, ("poisson", 6.0, None, None)),
              ti.TableSpec(9000, 64, ("poisson", 20.0, 1, 60)))
    spec = ti.BatchSpec("by-table edges", tables, B=4000, w_dtype=torch.float16, w_range=0.05,
                        optimizer="sgd", seed=77)
    bt = ti.make_batch(spec)
    flush_print(f"by table edges N={bt.num_indices}")
    for w in (False, True):
        g, _ = check_transpose(bt, w, tbe.make_config(sort_by_table=1), what=f"edges weighted={w}")
        assert g["view"].sorted_by_table == 1 and g["view"].radix_passes == 3
    g, _ = check_transpose(bt, False, tbe.make_config(), what="edges automatic")
    assert g["view"].sorted_by_table == 1


def test_transpose_by_table_many_tables():
    """By table over 600 tables of 300 .. 30000 rows (the table starts of the first pass scanned
    three to a thread, a block's table found among hundreds), with empty tables among them, in
    two passes where the linearized ids need three: the oracle's transpose bit for bit."""
    rng = np.random.default_rng(3)
    tables = []
    for t in range(600):
        E = int(rng.integers(300, 30000))
        L = ("fixed", 0) if t % 97 == 5 else ("poisson", float(rng.integers(4, 30)), None, None)
        idx = ("zipf", 1.05, min(E, 500)) if t % 3 == 0 else ("uniform",)
        tables.append(ti.TableSpec(E, 32, L, idx))
    spec = ti.BatchSpec("600 tables", tuple(tables), B=700, w_dtype=torch.float16, w_range=0.05,
                        optimizer="sgd", seed=41)
    bt = ti.make_batch(spec)
    flush_print(f"600 tables N={bt.num_indices}")
    assert bt.num_indices >= 2 * 600 * 4096
    g, _ = check_transpose(bt, False, tbe.make_config(), what="600 tables")
    # automatic: 15 bits of the largest local row id take 2 passes, 24 bits of linearized ids 3
    assert g["view"].sorted_by_table == 1 and g["view"].radix_passes == 2


@pytest.mark.parametrize("weighted", [False, True])
def test_transpose_without_bags(weighted):
    """B = 0 with lookups present: no bag covers any position, so nothing is sorted and no run
    is found (the linearize launch still has its one workgroup)."""
    t = tbe.Tables([50, 70], [16, 32], 0, torch.float16, device="cuda")
    idx = torch.tensor([3, 1, 4, 1, 5], dtype=torch.int64, device="cuda")
    off = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = tbe.workspace(tbe.tbe_backward_workspace_bytes(t, idx.numel(), weighted))
    view = tbe.tbe_transpose(t, idx, off, weighted, ws)
    torch.cuda.synchronize()
    cnt = tbe.device_view(view.counters, 16, torch.int32, ws).cpu().numpy()
    assert cnt[tbe.COUNTER_RUNS] == 0 and cnt[tbe.COUNTER_LONG] == 0 and cnt[tbe.COUNTER_CHUNKS] == 0
    assert all(cnt[tbe.COUNTER_SHORT0 + b] == 0 for b in range(tbe.NUM_BUCKETS))
