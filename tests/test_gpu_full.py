"""Parity at the full workload sizes, in the launch configuration the benchmark times (id
repair fused into the pooling, the backward's transpose hoisted into the forward call).

Whole tables (test_full_whole_tables): for at least two tables of every workload, including the
one holding the hottest row, everything is compared against the oracle run on that table's own
lookups - tables are independent, so this is the oracle's result for the whole batch
restricted to those tables.

The oracle cannot redo an 84M-lookup batch in seconds, so at these sizes:
  * forward:   sampled bags (random, longest, empty, first/last) are recomputed one by one
               by the oracle from host copies of exactly the rows they touch;
  * backward:  sampled rows (the hottest of each table, random touched rows, short and long
               runs) are recomputed by the oracle from every lookup that touched them; every
               untouched row of every table must be bit-identical after the step;
  * transpose: properties that fix a stable sort uniquely - positions are a permutation,
               each key is the linearized id of its position, (key, position) strictly
               increases - plus exact run / routing counts from a host histogram.
"""
import gc

import numpy as np
import pytest
import torch

import bwd_tbe_fwd_amd as tbe
import oracle
import tbe_inputs as ti
from gpu_util import (ODT, DevBatch, check_forward, check_momentum, check_weights, flush_print,
                      row_g_abs_sq, step_bound)

pytestmark = pytest.mark.gpu

_cache = {}


def full_batch(n):
    if n not in _cache:
        _cache.clear()
        gc.collect()
        torch.cuda.empty_cache()
        spec = ti.WORKLOADS[n]
        flush_print(f"drawing full workload {n}: {spec.name}")
        bt = ti.make_batch(spec, device="cuda")
        db = DevBatch.__new__(DevBatch)
        db.bt, db.device = bt, "cuda"
        db.tables = tbe.Tables(bt.E, bt.D, bt.B, bt.w_dtype, device="cuda", pooling_hint=spec.pooling_hint)
        db.W, db.idx, db.off, db.psw, db.grad, db.mom = (bt.weights, bt.indices, bt.offsets, bt.psw,
                                                          bt.grad_out, bt.momentum)
        host = dict(idx=bt.indices.long().cpu().numpy(), off=bt.offsets.long().cpu().numpy(),
                    psw=None if bt.psw is None else bt.psw.double().cpu().numpy())
        _cache[n] = (db, host)
    return _cache[n]


def table_rows(db, t, rows):
    """Host fp64 copy of rows of table t (W still holds the values before any update)."""
    bt = db.bt
    Wt = db.W[sum(e * d for e, d in zip(bt.E[:t], bt.D[:t])):][:bt.E[t] * bt.D[t]].view(bt.E[t], bt.D[t])
    return Wt[torch.as_tensor(rows, device="cuda", dtype=torch.long)].double().cpu().numpy()


@pytest.mark.parametrize("n", ["uniform", "histogram", "mixed", "skewed"])
def test_full_forward_sampled_bags(n):
    db, h = full_batch(n)
    bt = db.bt
    out = torch.full((bt.B, sum(bt.D)), float("nan"), dtype=torch.float32, device="cuda")
    tbe.tbe_forward(db.tables, db.W, db.idx, db.off, db.psw, out)
    # the benchmark's launch configuration: id repair fused into the pooling and the backward's
    # transpose on the second stream; valid inputs, so nothing is repaired and out is the same
    out_b = torch.full_like(out, float("nan"))
    counts = torch.full((2,), -1, dtype=torch.int64, device="cuda")
    bws = tbe.workspace(tbe.tbe_bounds_check_workspace_bytes(db.tables))
    ws = db.workspace()
    tbe.tbe_forward_hoisted(db.tables, db.W, db.idx, db.off, db.psw, out_b, counts, bws, ws)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0, 0]
    assert torch.equal(out.view(torch.int32), out_b.view(torch.int32))
    del ws, bws, out_b
    rng = np.random.default_rng(len(n))
    off = h["off"]
    lens = np.diff(off)
    picks = set(rng.integers(0, bt.T * bt.B, 300).tolist())
    picks |= set(np.argsort(lens)[-20:].tolist()) | set(np.flatnonzero(lens == 0)[:10].tolist())
    picks |= {0, bt.T * bt.B - 1}
    cols = np.concatenate([[0], np.cumsum(bt.D)])
    for bag in sorted(picks):
        t, b = divmod(bag, bt.B)
        s, e = off[bag], off[bag + 1]
        ids = h["idx"][s:e]
        uniq, local = np.unique(ids, return_inverse=True)
        Wsub = table_rows(db, t, uniq) if uniq.size else np.zeros((0, bt.D[t]))
        psw = None if h["psw"] is None else h["psw"][s:e]
        ref, ref_abs = oracle.forward(1, 1, [max(uniq.size, 1)], [bt.D[t]],
                                      Wsub if uniq.size else np.zeros(bt.D[t]), local, [0, e - s], psw)
        got = out[b, cols[t]:cols[t + 1]].double().cpu().numpy()[None, :]
        check_forward(got, ref, ref_abs, bt.w_dtype == torch.float32, f"{n} bag ({t},{b})")


@pytest.mark.parametrize("n", ["uniform", "histogram", "mixed", "skewed"])
def test_full_transpose_properties(n):
    db, h = full_batch(n)
    bt = db.bt
    N = bt.num_indices
    res = {}
    for weighted in (True, False):
        ws = db.workspace(None, weighted)
        view = tbe.tbe_transpose(db.tables, db.idx, db.off, weighted, ws)
        torch.cuda.synchronize()
        cnt = tbe.device_view(view.counters, 16, torch.int32, ws).cpu().numpy()
        res[weighted] = dict(
            cnt=cnt,
            keys=tbe.device_view(view.sorted_keys, N, torch.int32, ws).cpu().numpy().view(np.uint32),
            pay=tbe.device_view(view.sorted_payload, N, torch.int32, ws).cpu().numpy().view(np.uint32),
            run_key=tbe.device_view(view.run_key, int(cnt[0]), torch.int32, ws).cpu().numpy().view(np.uint32),
            run_start=tbe.device_view(view.run_start, int(cnt[0]) + 1, torch.int32, ws).cpu().numpy().view(np.uint32))
        del ws
    off = h["off"]
    bag_of = np.repeat(np.arange(bt.T * bt.B, dtype=np.int64), np.diff(off))
    rowbase = np.concatenate([[0], np.cumsum(bt.E)])
    key_of = rowbase[bag_of // bt.B] + h["idx"]
    w = res[True]
    pos = w["pay"].astype(np.int64)
    keys = w["keys"].astype(np.int64)
    assert np.all(np.bincount(pos, minlength=N) == 1)                 # a permutation
    assert np.array_equal(keys, key_of[pos])                           # keys follow their lookups
    step = np.diff(keys) * (N + 1) + np.diff(pos)                      # (key, position) increasing
    assert np.all(step > 0)
    u = res[False]
    assert np.array_equal(u["keys"], w["keys"])
    assert np.array_equal(u["pay"].astype(np.int64), bag_of[pos])     # bag payload of each lookup
    heads = np.flatnonzero(np.concatenate([[True], keys[1:] != keys[:-1]]))
    for r in (w, u):
        assert int(r["cnt"][tbe.COUNTER_RUNS]) == heads.size
        assert np.array_equal(r["run_start"][:-1].astype(np.int64), heads)
        assert np.array_equal(r["run_key"].astype(np.int64), keys[heads])
    lens = np.diff(np.concatenate([heads, [N]]))
    is_long = lens >= 256
    assert int(w["cnt"][tbe.COUNTER_LONG]) == int(is_long.sum())
    assert int(w["cnt"][tbe.COUNTER_CHUNKS]) == int(((lens[is_long] + 255) // 256).sum())
    t_of_run = np.searchsorted(rowbase, keys[heads], side="right") - 1
    Dk = np.array(bt.D)[t_of_run]
    for b in range(tbe.NUM_BUCKETS):
        want = int((~is_long & (np.maximum(4, 2 ** np.ceil(np.log2(Dk))) == tbe.BUCKET_D[b])).sum())
        assert int(w["cnt"][tbe.COUNTER_SHORT0 + b]) == want
    flush_print(f"{n}: {N} lookups, {heads.size} runs, {int(is_long.sum())} long, "
                f"max run {int(lens.max())}")


@pytest.mark.parametrize("n", ["uniform", "histogram", "mixed", "skewed"])
def test_full_backward_sampled_rows(n):
    db, h = full_batch(n)
    bt = db.bt
    spec = bt.spec
    rng = np.random.default_rng(100 + len(n))
    off = h["off"]
    samples = []   # (t, row)
    untouched = []
    counts = []
    for t in range(bt.T):
        s, e = off[t * bt.B], off[(t + 1) * bt.B]
        c = np.bincount(h["idx"][s:e], minlength=bt.E[t])
        counts.append(c)
        touched = np.flatnonzero(c)
        hot = touched[np.argsort(c[touched])[-2:]]
        mid = touched[(c[touched] >= 256)][:2]
        rnd = rng.choice(touched, size=min(4, touched.size), replace=False)
        samples += [(t, int(r)) for r in set(hot.tolist() + mid.tolist() + rnd.tolist())]
        free = np.flatnonzero(c == 0)
        if free.size:
            untouched += [(t, int(r)) for r in rng.choice(free, size=min(2, free.size), replace=False)]
    # host copies of the sampled rows, their state and their lookups' gradient rows, before the step
    before = {(t, r): table_rows(db, t, [r])[0] for (t, r) in samples + untouched}
    rowbase = np.concatenate([[0], np.cumsum(bt.E)])
    cols = np.concatenate([[0], np.cumsum(bt.D)])
    mom0 = None if db.mom is None else db.mom.double().cpu().numpy()
    grads = {}
    for (t, r) in samples:
        s, e = off[t * bt.B], off[(t + 1) * bt.B]
        p = s + np.flatnonzero(h["idx"][s:e] == r)
        b = np.searchsorted(off, p, side="right") - 1 - t * bt.B
        g = db.grad[:, cols[t]:cols[t + 1]][torch.as_tensor(b, device="cuda")].double().cpu().numpy()
        grads[(t, r)] = (g, None if h["psw"] is None else h["psw"][p])
    W0 = db.W.clone()
    m0 = None if db.mom is None else db.mom.clone()
    ws = db.workspace()
    lr, eps = oracle.f32_literal(spec.lr), oracle.f32_literal(spec.eps)
    # the benchmark's launch configuration: fused repair, transpose hoisted into the forward
    # call (second stream), backward with pretransposed runs
    out = torch.empty((bt.B, sum(bt.D)), dtype=torch.float32, device="cuda")
    err_counts = torch.full((2,), -1, dtype=torch.int64, device="cuda")
    bws = tbe.workspace(tbe.tbe_bounds_check_workspace_bytes(db.tables))
    tbe.tbe_forward_hoisted(db.tables, db.W, db.idx, db.off, db.psw, out, err_counts, bws, ws)
    cfg = tbe.make_config(pretransposed=1)
    if spec.optimizer == "sgd":
        tbe.tbe_backward_sgd(db.tables, db.W, db.idx, db.off, db.psw, db.grad, lr, ws, cfg)
    else:
        tbe.tbe_backward_rowwise_adagrad(db.tables, db.W, db.mom, db.idx, db.off, db.psw, db.grad,
                                         lr, eps, ws, cfg)
    torch.cuda.synchronize()
    assert err_counts.cpu().tolist() == [0, 0]
    del ws, bws, out
    # every untouched row of every table is bit-identical
    pos = 0
    for t in range(bt.T):
        E, D = bt.E[t], bt.D[t]
        free = torch.from_numpy(counts[t] == 0).cuda()
        a = db.W[pos:pos + E * D].view(E, D)[free]
        b0 = W0[pos:pos + E * D].view(E, D)[free]
        assert torch.equal(a.view(torch.int16) if a.dtype != torch.float32 else a.view(torch.int32),
                           b0.view(torch.int16) if b0.dtype != torch.float32 else b0.view(torch.int32))
        if m0 is not None:
            assert torch.equal(db.mom[rowbase[t]:rowbase[t] + E][free], m0[rowbase[t]:rowbase[t] + E][free])
        pos += E * D
    # sampled rows: one oracle step from every lookup that touched them
    opt = oracle.SGD if spec.optimizer == "sgd" else oracle.ROWWISE_ADAGRAD
    for (t, r) in samples:
        g, psw = grads[(t, r)]
        L, D = g.shape[0], bt.D[t]
        m_in = None if mom0 is None else np.array([mom0[rowbase[t] + r]])
        res = oracle.backward(1, L, [1], [D], ODT[bt.w_dtype], before[(t, r)], np.zeros(L, np.int64),
                              np.arange(L + 1), psw, g, opt, lr, eps, m_in)
        got = table_rows(db, t, [r])[0]
        Wrow = torch.from_numpy(got).to(bt.w_dtype)
        denom = np.sqrt(res["m_new"][0]) + eps if opt == oracle.ROWWISE_ADAGRAD else 1.0
        step_abs = abs(lr) * res["g_abs"] / denom
        check_weights(Wrow, res, bt.w_dtype, step_abs, f"{n} row ({t},{r}) SL={L}")
        if opt == oracle.ROWWISE_ADAGRAD:
            mg = db.mom[rowbase[t] + r:rowbase[t] + r + 1]
            check_momentum(mg, res, np.array([D], float), np.array([(res["g_abs"] ** 2).sum()]),
                           f"{n} state ({t},{r})")
    flush_print(f"{n}: {len(samples)} sampled rows and all untouched rows match")


# tables compared whole at full size: the one holding the batch's hottest row plus fixed picks
# (both tables of the histogram workload; one of each width of the mixed workload)
WHOLE_TABLES = {"uniform": [0, 25], "histogram": [0, 1], "mixed": [0, 5, 10, 15], "skewed": [0, 31]}


def _host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def _u32(ptr, n, ws):
    return tbe.device_view(ptr, n, torch.int32, ws).cpu().numpy().view(np.uint32).astype(np.int64)


@pytest.mark.parametrize("n", ["uniform", "histogram", "mixed", "skewed"])
def test_full_whole_tables(n):
    """Whole tables at the full workload size, in the benchmark's launch configuration (offsets
    repair and id check fused into the pooling, the transpose hoisted into the forward call on
    the second stream with the dense rows picked as the benchmark picks them, the backward
    reusing it).  For every checked table, against the oracle run on that table's own lookups
    (tables are independent): every output column of every bag; every touched row's weights
    and Adagrad state; every untouched row bit for bit; the complete short and long lists (key,
    length, width bucket) and chunk plan as sets, and each run's payloads in the sorted arrays in
    the oracle's stable order."""
    db, h = full_batch(n)
    bt = db.bt
    spec = bt.spec
    T, B, N = bt.T, bt.B, bt.num_indices
    off, idx = h["off"], h["idx"]
    weighted = db.psw is not None
    counts = [np.bincount(idx[off[t * B]:off[(t + 1) * B]], minlength=bt.E[t]) for t in range(T)]
    hot_t = int(np.argmax([c.max() for c in counts]))
    chk = sorted(set(WHOLE_TABLES[n]) | {hot_t})
    rowbase = np.concatenate([[0], np.cumsum(bt.E)]).astype(np.int64)
    wbase = np.concatenate([[0], np.cumsum(np.array(bt.E, np.int64) * np.array(bt.D, np.int64))])
    cols = np.concatenate([[0], np.cumsum(bt.D)])
    W0 = db.W.clone()
    m0 = None if db.mom is None else db.mom.clone()
    lr, eps = oracle.f32_literal(spec.lr), oracle.f32_literal(spec.eps)
    out = torch.full((B, sum(bt.D)), float("nan"), dtype=torch.float32, device="cuda")
    err_counts = torch.full((2,), -1, dtype=torch.int64, device="cuda")
    bws = tbe.workspace(tbe.tbe_bounds_check_workspace_bytes(db.tables))
    ws = db.workspace()
    tbe.tbe_forward_hoisted(db.tables, db.W, db.idx, db.off, db.psw, out, err_counts, bws, ws)
    torch.cuda.synchronize()
    assert err_counts.cpu().tolist() == [0, 0]
    # the routing the hoisted forward left in the workspace, copied out before the backward
    view = tbe.tbe_transpose(db.tables, db.idx, db.off, weighted, ws, tbe.make_config(pretransposed=1))
    cnt = tbe.device_view(view.counters, 16, torch.int32, ws).cpu().numpy()
    kept = int(cnt[13])
    keys = _u32(view.sorted_keys, kept, ws)
    pay = _u32(view.sorted_payload, kept, ws)
    n_long, n_chunk = int(cnt[tbe.COUNTER_LONG]), int(cnt[tbe.COUNTER_CHUNKS])
    long_list = _u32(view.long_list, 4 * n_long, ws).reshape(-1, 4)
    long_table = _u32(view.long_table, n_long, ws)
    chunk_list = _u32(view.chunk_list, 2 * n_chunk, ws).reshape(-1, 2)
    shorts = {b: _u32(view.short_list[b], 4 * int(cnt[tbe.COUNTER_SHORT0 + b]), ws).reshape(-1, 4)
              for b in range(tbe.NUM_BUCKETS) if view.short_list[b]}
    dense_rows = {}
    if view.dense_rows:
        dcnt = tbe.device_view(view.dense_count, T, torch.int32, ws).cpu().numpy()
        drows = tbe.device_view(view.dense_rows, T * 128, torch.int32, ws).cpu().numpy().reshape(T, 128)
        dense_rows = {t: drows[t, :dcnt[t]].astype(np.int64) for t in range(T)}
    cfg = tbe.make_config(pretransposed=1)
    if spec.optimizer == "sgd":
        tbe.tbe_backward_sgd(db.tables, db.W, db.idx, db.off, db.psw, db.grad, lr, ws, cfg)
    else:
        tbe.tbe_backward_rowwise_adagrad(db.tables, db.W, db.mom, db.idx, db.off, db.psw, db.grad,
                                         lr, eps, ws, cfg)
    torch.cuda.synchronize()
    del ws, bws
    hist_t = db.tables.c.hist_table if not weighted else -1
    ada = spec.optimizer == "rowwise_adagrad"
    opt = oracle.ROWWISE_ADAGRAD if ada else oracle.SGD
    for t in chk:
        s, e = int(off[t * B]), int(off[(t + 1) * B])
        E, D = bt.E[t], bt.D[t]
        ids = idx[s:e]
        uniq, local = np.unique(ids, return_inverse=True)
        U = uniq.size
        o_t = off[t * B:(t + 1) * B + 1] - s
        psw = None if h["psw"] is None else h["psw"][s:e]
        rows_dev = torch.as_tensor(uniq, device="cuda")
        Wt0 = W0[wbase[t]:wbase[t + 1]].view(E, D)
        Wt1 = db.W[wbase[t]:wbase[t + 1]].view(E, D)
        W_sub = Wt0[rows_dev].double().cpu().numpy()
        # forward: every bag, every column of the table's slice
        ref, ref_abs = oracle.forward(1, B, [U], [D], W_sub, local, o_t, psw)
        check_forward(out[:, cols[t]:cols[t + 1]].double().cpu().numpy(), ref, ref_abs,
                      bt.w_dtype == torch.float32, f"{n} table {t} forward")
        # backward: every touched row, one oracle step from the table's own lookups
        g_t = db.grad[:, cols[t]:cols[t + 1]].double().cpu().numpy()
        m_in = None if m0 is None else m0[rowbase[t]:rowbase[t + 1]][rows_dev].double().cpu().numpy()
        r = oracle.backward(1, B, [U], [D], ODT[bt.w_dtype], W_sub, local, o_t, psw, g_t, opt, lr, eps, m_in)
        check_weights(Wt1[rows_dev].reshape(-1).cpu(), r, bt.w_dtype, step_bound(r, [U], [D], lr, eps, ada),
                      f"{n} table {t} weights")
        if ada:
            gsq, Dr = row_g_abs_sq(r, [U], [D])
            check_momentum(db.mom[rowbase[t]:rowbase[t + 1]][rows_dev], r, Dr, gsq, f"{n} table {t} state")
        free = torch.from_numpy(counts[t] == 0).cuda()
        bits = (lambda x: x.view(torch.int32) if x.dtype == torch.float32 else x.view(torch.int16))
        assert torch.equal(bits(Wt1[free]), bits(Wt0[free])), f"{n} table {t}: untouched rows changed"
        if m0 is not None:
            assert torch.equal(db.mom[rowbase[t]:rowbase[t + 1]][free], m0[rowbase[t]:rowbase[t + 1]][free])
        # routing: the oracle's runs of this table against the GPU lists
        tr = oracle.transpose(1, B, [U], local, o_t)
        rk = uniq[tr["run_key"]]                # row id of each run
        rl = tr["run_len"]
        lens_all = rl
        if t == hist_t:
            # the histogram table's lookups stay out of the sort: no run of it anywhere
            assert not (long_table == t).any()
            for lst in shorts.values():
                assert not (lst[:, 3] == t).any()
            got_runs = 0
        else:
            dn = dense_rows.get(t, np.zeros(0, np.int64))
            assert np.all(np.isin(dn, rk)), f"{n} table {t}: a dense row with no lookup"
            keep = ~np.isin(rk, dn)
            exp_long = {(int(k), int(l)) for k, l in zip(rk[keep], rl[keep]) if l >= 256}
            exp_short = {(int(k), int(l)) for k, l in zip(rk[keep], rl[keep]) if l < 256}
            sl_t = long_list[long_table == t]
            got_long = {(int(k) - int(rowbase[t]), int(l)) for k, l in zip(sl_t[:, 0], sl_t[:, 2])}
            assert got_long == exp_long, f"{n} table {t}: long runs differ"
            bucket = tbe.BUCKET_D.index(max(4, 1 << (D - 1).bit_length()))
            got_short = set()
            for b, lst in shorts.items():
                mine = lst[lst[:, 3] == t]
                assert b == bucket or mine.shape[0] == 0, f"{n} table {t}: short run in bucket {b}"
                got_short |= {(int(k) - int(rowbase[t]), int(l)) for k, l in zip(mine[:, 0], mine[:, 2])}
            assert got_short == exp_short, f"{n} table {t}: short runs differ"
            # chunk plan of every long run
            for slot in np.flatnonzero(long_table == t):
                k, st0, ln, cb = (int(x) for x in long_list[slot])
                nch = (ln + 255) // 256
                assert np.array_equal(chunk_list[cb:cb + nch], np.stack([np.full(nch, slot), np.arange(nch)], 1))
            # every run's keys and payloads in the sorted arrays: the oracle's stable order
            runs = [long_list[long_table == t][:, :3]] + [lst[lst[:, 3] == t][:, :3] for lst in shorts.values()]
            runs = np.concatenate(runs) if runs else np.zeros((0, 3), np.int64)
            assert np.array_equal(tr["run_key"], np.arange(U))   # one oracle run per touched row
            q = np.searchsorted(uniq, runs[:, 0] - rowbase[t])    # the oracle's run of each GPU run
            ln = runs[:, 2]
            within = np.arange(int(ln.sum())) - np.repeat(np.cumsum(ln) - ln, ln)
            gpu_at = np.repeat(runs[:, 1], ln) + within
            ora_at = np.repeat(tr["run_start"][q], ln) + within
            assert np.array_equal(keys[gpu_at], np.repeat(runs[:, 0], ln)), f"{n} table {t}: keys"
            want = (tr["sorted_pos"] + s) if weighted else (tr["sorted_bag"] + t * B)
            assert np.array_equal(pay[gpu_at], want[ora_at]), f"{n} table {t}: payload order"
            got_runs = runs.shape[0]
        long_share = float(lens_all[lens_all >= 256].sum()) / max(1, ids.size)
        flush_print(f"{n} table {t}: N={ids.size} U={U} max SL={int(lens_all.max()) if U else 0} "
                    f"long-run share={long_share:.3f} runs in lists={got_runs} "
                    f"dense rows={dense_rows.get(t, np.zeros(0)).size}")
    del W0, m0, out


def test_max_total_rows():
    """The largest row space the 32-bit keys allow: 2^31 - 2 rows in all (a 17 GB fp16 table of
    2^31 - 1002 rows next to a 1000-row one), ids spread over the whole range.  Keys up to
    2^31 - 3, four radix passes, the sentinel 2^31 - 2; forward bags, every touched row and a
    sample of untouched rows checked against the oracle."""
    _cache.clear()
    gc.collect()
    torch.cuda.empty_cache()
    E0 = 2 ** 31 - 2 - 1000
    spec = ti.BatchSpec("max rows", (ti.TableSpec(E0, 4, ("poisson", 5.0, None, None)),
                                     ti.TableSpec(1000, 8, ("fixed", 3))),
                        B=2000, w_dtype=torch.float16, w_range=0.5, optimizer="rowwise_adagrad")
    flush_print("drawing the max-rows batch (17 GB of weights)")
    bt = ti.make_batch(spec, 91, device="cuda")
    db = DevBatch.__new__(DevBatch)
    db.bt, db.device = bt, "cuda"
    db.tables = tbe.Tables(bt.E, bt.D, bt.B, bt.w_dtype, device="cuda")
    assert db.tables.c.total_rows == 2 ** 31 - 2
    db.W, db.idx, db.off, db.psw, db.grad, db.mom = (bt.weights, bt.indices, bt.offsets, None,
                                                      bt.grad_out, bt.momentum)
    idx, off = bt.indices.long().cpu().numpy(), bt.offsets.long().cpu().numpy()
    assert idx[:off[bt.B]].max() > 2 ** 30   # high ids are exercised
    # transpose: four passes, keys follow their lookups, (key, position) increasing
    ws = db.workspace(None, True)
    view = tbe.tbe_transpose(db.tables, db.idx, db.off, True, ws)
    torch.cuda.synchronize()
    assert view.radix_passes == 4
    N = bt.num_indices
    keys = tbe.device_view(view.sorted_keys, N, torch.int32, ws).cpu().numpy().view(np.uint32).astype(np.int64)
    pos = tbe.device_view(view.sorted_payload, N, torch.int32, ws).cpu().numpy().view(np.uint32).astype(np.int64)
    del ws
    bag_of = np.repeat(np.arange(bt.T * bt.B, dtype=np.int64), np.diff(off))
    rowbase = np.array([0, E0, E0 + 1000], dtype=np.int64)
    assert np.array_equal(keys, (rowbase[bag_of // bt.B] + idx)[pos])
    assert np.all(np.diff(keys) * (N + 1) + np.diff(pos) > 0)
    # forward, every bag of both tables (few lookups): the oracle on the touched rows
    out = torch.full((bt.B, 12), float("nan"), device="cuda")
    tbe.tbe_forward(db.tables, db.W, db.idx, db.off, None, out)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    cols = [0, 4, 12]
    for t in range(2):
        s, e = off[t * bt.B], off[(t + 1) * bt.B]
        uniq, local = np.unique(idx[s:e], return_inverse=True)
        Wsub = table_rows(db, t, uniq)
        o = off[t * bt.B:(t + 1) * bt.B + 1] - s
        ref, ref_abs = oracle.forward(1, bt.B, [uniq.size], [bt.D[t]], Wsub, local, o)
        check_forward(got[:, cols[t]:cols[t + 1]], ref, ref_abs, False, f"max rows table {t}")
    # backward: every touched row of table 0, against the oracle on its own lookups
    s0, e0 = off[0], off[bt.B]
    uniq, local = np.unique(idx[s0:e0], return_inverse=True)
    W_before = table_rows(db, 0, uniq)
    m_before = db.mom[torch.as_tensor(uniq, device="cuda")].double().cpu().numpy()
    free = np.setdiff1d(np.random.default_rng(0).integers(0, E0, 64), uniq)
    W_free = table_rows(db, 0, free)
    ws = db.workspace()
    lr, eps = oracle.f32_literal(spec.lr), oracle.f32_literal(spec.eps)
    tbe.tbe_backward_rowwise_adagrad(db.tables, db.W, db.mom, db.idx, db.off, None, db.grad, lr, eps, ws)
    torch.cuda.synchronize()
    del ws
    g0 = db.grad[:, 0:4].double().cpu().numpy()
    bag0 = np.repeat(np.arange(bt.B), np.diff(off[:bt.B + 1]))
    # one oracle call over table 0 restricted to its touched rows (renumbered 0..U-1)
    r = oracle.backward(1, bt.B, [uniq.size], [4], oracle.F16, W_before, local,
                        off[:bt.B + 1] - s0, None, g0, oracle.ROWWISE_ADAGRAD, lr, eps, m_before)
    W_after = torch.from_numpy(table_rows(db, 0, uniq).ravel()).to(torch.float16)
    check_weights(W_after, r, torch.float16, step_bound(r, [uniq.size], [4], lr, eps, True), "max rows")
    assert np.array_equal(table_rows(db, 0, free), W_free)
    assert bag0.size == e0 - s0
    del bt, db
    gc.collect()
    torch.cuda.empty_cache()


def test_max_lookups():
    """The largest lookup count the ABI accepts, 2^31 - 4096 (one table of 2^20 rows, 524287
    bags of 4096 int32 ids): sampled bags of the forward, run and chunk counts of the
    transpose, and sampled rows of the summed gradient (SGD, lr = -1, zero fp32 weights)."""
    _cache.clear()
    gc.collect()
    torch.cuda.empty_cache()
    E, L, B = 2 ** 20, 4096, 2 ** 19 - 1
    spec = ti.BatchSpec("max lookups", (ti.TableSpec(E, 4, ("fixed", L)),), B=B,
                        w_dtype=torch.float32, w_range=0.5, itype=torch.int32, otype=torch.int64,
                        optimizer="sgd")
    flush_print("drawing the max-lookups batch (2^31 - 4096 int32 ids)")
    bt = ti.make_batch(spec, 93, device="cuda")
    N = bt.num_indices
    assert N == 2 ** 31 - 4096
    tables = tbe.Tables(bt.E, bt.D, bt.B, bt.w_dtype, device="cuda")
    idx, off = bt.indices, bt.offsets
    # forward: sampled bags against the oracle
    out = torch.full((B, 4), float("nan"), device="cuda")
    tbe.tbe_forward(tables, bt.weights, idx, off, None, out)
    torch.cuda.synchronize()
    W = bt.weights.view(E, 4)
    rng = np.random.default_rng(7)
    for b in [0, B - 1] + rng.integers(0, B, 20).tolist():
        ids = idx[b * L:(b + 1) * L].long().cpu().numpy()
        uniq, local = np.unique(ids, return_inverse=True)
        ref, ref_abs = oracle.forward(1, 1, [uniq.size], [4], W[torch.as_tensor(uniq, device="cuda")].double().cpu().numpy(),
                                      local, [0, L])
        check_forward(out[b:b + 1].double().cpu().numpy(), ref, ref_abs, True, f"max lookups bag {b}")
    del out
    # transpose counters against a histogram of the ids
    counts = torch.bincount(idx.long(), minlength=E)
    ws = tbe.workspace(tbe.tbe_backward_workspace_bytes(tables, N, False))
    view = tbe.tbe_transpose(tables, idx, off, False, ws)
    torch.cuda.synchronize()
    cnt = tbe.device_view(view.counters, 16, torch.int32, ws).cpu().numpy()
    c = counts[counts > 0]
    assert int(cnt[tbe.COUNTER_RUNS]) == c.numel()
    assert int(cnt[tbe.COUNTER_LONG]) == int((c >= 256).sum())
    assert int(cnt[tbe.COUNTER_CHUNKS]) == int(((c[c >= 256] + 255) // 256).sum())
    # backward: sampled rows' summed gradient
    bt.weights.zero_()
    tbe.tbe_backward_sgd(tables, bt.weights, idx, off, None, bt.grad_out, -1.0, ws)
    torch.cuda.synchronize()
    del ws
    for r in rng.integers(0, E, 12).tolist():
        pos = (idx == r).nonzero().flatten()
        g = bt.grad_out[pos // L].double().cpu().numpy()
        res = oracle.backward(1, g.shape[0], [1], [4], oracle.F32, np.zeros(4), np.zeros(g.shape[0], np.int64),
                              np.arange(g.shape[0] + 1), None, g, oracle.SGD, -1.0)
        check_weights(bt.weights.view(E, 4)[r].cpu(), res, torch.float32, res["g_abs"], f"max lookups row {r}")
    del bt, counts, tables
    gc.collect()
    torch.cuda.empty_cache()
