"""Backward parity: one optimizer step per touched row, SGD and exact row-wise Adagrad,
against the oracle; routing invariance; gradient extraction; determinism."""
import numpy as np
import pytest
import torch

import bwd_tbe_fwd_amd as tbe
import oracle
import tbe_inputs as ti
from gpu_util import (DevBatch, check_momentum, check_weights, flush_print, host_arrays,
                      oracle_backward, row_g_abs_sq, step_bound)
from test_gpu_forward import WORKLOAD_NAMES, mixed_spec, small_spec

pytestmark = pytest.mark.gpu


def run_and_check(bt, cfg=None, optimizer=None, lr=None, what=""):
    optimizer = optimizer or bt.spec.optimizer
    db = DevBatch(bt)
    if optimizer == "rowwise_adagrad" and db.mom is None:
        db.mom = torch.zeros(sum(bt.E), dtype=torch.float32, device="cuda")
        bt.momentum = torch.zeros(sum(bt.E), dtype=torch.float32)
    W, mom = db.backward(cfg, optimizer=optimizer, lr=lr)
    torch.cuda.synchronize()
    r = oracle_backward(bt, lr=lr, optimizer=optimizer)
    lr32 = oracle.f32_literal(bt.spec.lr if lr is None else lr)
    ada = optimizer == "rowwise_adagrad"
    sb = step_bound(r, bt.E, bt.D, lr32, oracle.f32_literal(bt.spec.eps), ada)
    check_weights(W, r, bt.w_dtype, sb, what)
    if ada:
        gsq, Dr = row_g_abs_sq(r, bt.E, bt.D)
        check_momentum(mom, r, Dr, gsq, what)
    return db, W, mom, r


@pytest.mark.parametrize("n", WORKLOAD_NAMES)
def test_backward_configs_small(n):
    spec = small_spec(n)
    flush_print(f"backward {n}: {spec.name} ({spec.optimizer})")
    bt = ti.make_batch(spec)
    run_and_check(bt, what=n)


@pytest.mark.parametrize("w_dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("optimizer", ["sgd", "rowwise_adagrad"])
@pytest.mark.parametrize("weighted", [False, True])
def test_backward_dtypes_mixed_D(w_dtype, optimizer, weighted):
    spec = mixed_spec(w_dtype, torch.int64, torch.int32, weighted).replace(optimizer=optimizer)
    bt = ti.make_batch(spec, 19)
    run_and_check(bt, tbe.make_config(long_threshold=32, chunk=16), what=f"{w_dtype} {optimizer} {weighted}")


@pytest.mark.parametrize("optimizer", ["sgd", "rowwise_adagrad"])
@pytest.mark.parametrize("threshold,chunk", [(10 ** 9, 256), (256, 256), (8, 8), (4, 2), (1, 1)])
def test_routing_invariance(optimizer, threshold, chunk):
    """Same batch, every split point: all match the oracle (tutorial section 3's sweep)."""
    bt = ti.make_batch(small_spec("skewed").replace(optimizer=optimizer), 23)
    cfg = tbe.make_config(long_threshold=threshold, chunk=chunk)
    run_and_check(bt, cfg, what=f"{optimizer} t={threshold} c={chunk}")


@pytest.mark.parametrize("weighted", [False, True])
def test_gradient_extraction(weighted):
    """SGD with lr = -1 on all-zero fp32 weights writes the summed gradient itself."""
    spec = small_spec("mixed" if weighted else "skewed").replace(w_dtype=torch.float32, optimizer="sgd")
    bt = ti.make_batch(spec, 29)
    bt.weights = torch.zeros_like(bt.weights)
    db = DevBatch(bt)
    W, _ = db.backward(tbe.make_config(long_threshold=64, chunk=32), lr=-1.0)
    r = oracle_backward(bt, lr=-1.0)
    got = W.double().cpu().numpy()
    err = np.abs(got - r["g"])
    assert np.all(err <= 1e-5 * r["g_abs"]), float((err - 1e-5 * r["g_abs"]).max())


@pytest.mark.parametrize("cfg_kw", [{}, dict(dense_min=64, dense_presort=1)])
def test_backward_deterministic(cfg_kw):
    """Bitwise the same on every run: also when the dense rows are picked before the sort, so
    that two short-run grids on two streams take their runs from a shared counter in whatever
    order they get there."""
    bt = ti.make_batch(small_spec("skewed"), 31)
    cfg = tbe.make_config(long_threshold=16, chunk=16, **cfg_kw)
    outs = []
    for _ in range(2):
        db = DevBatch(bt)
        W, mom = db.backward(cfg)
        outs.append((W.cpu().clone(), mom.cpu().clone()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))


def test_untouched_rows_bit_identical():
    bt = ti.make_batch(small_spec("skewed"), 37)
    db = DevBatch(bt)
    W0 = db.W.clone()
    m0 = db.mom.clone()
    W, mom = db.backward(tbe.make_config(long_threshold=16, chunk=16))
    a = host_arrays(bt)
    tr = oracle.transpose(a["T"], a["B"], a["E"], a["idx"], a["off"])
    touched = np.zeros(sum(bt.E), dtype=bool)
    touched[tr["run_key"]] = True
    D = bt.D[0]
    W2 = W.view(-1, D).cpu()
    W02 = W0.view(-1, D).cpu()
    t = torch.from_numpy(touched)
    assert torch.equal(W2[~t].view(torch.int16), W02[~t].view(torch.int16))
    assert torch.equal(mom.cpu()[~t], m0.cpu()[~t])
    assert (mom.cpu()[t] > m0.cpu()[t]).all()


def test_backward_no_lookups_and_no_bags():
    spec = ti.BatchSpec("empty", (ti.TableSpec(10, 8, ("fixed", 0)),), B=50, w_dtype=torch.float16,
                        w_range=0.5, optimizer="rowwise_adagrad")
    bt = ti.make_batch(spec, 1)
    db = DevBatch(bt)
    W0 = db.W.clone()
    W, mom = db.backward()
    assert torch.equal(W.cpu(), W0.cpu()) and torch.equal(mom.cpu(), torch.zeros_like(mom.cpu()))


def test_backward_out_of_range_ids_dropped():
    spec = ti.BatchSpec("bad ids", (ti.TableSpec(20, 16, ("fixed", 6)), ti.TableSpec(30, 32, ("fixed", 3))),
                        B=40, w_dtype=torch.float32, w_range=0.5, optimizer="sgd")
    bt = ti.make_batch(spec, 2)
    idx = bt.indices.clone()
    bad = torch.zeros(idx.numel(), dtype=torch.bool)
    bad[::7] = True
    idx[bad] = 99999
    bt.indices = idx
    db = DevBatch(bt)
    W, _ = db.backward()
    a = host_arrays(bt)
    keep = (~bad).double().numpy()
    ids = np.where(bad.numpy(), 0, a["idx"])
    r = oracle.backward(a["T"], a["B"], a["E"], a["D"], oracle.F32, a["W"], ids, a["off"], keep,
                        a["grad"], oracle.SGD, oracle.f32_literal(0.01))
    check_weights(W, r, torch.float32, 0.01 * r["g_abs"], "dropped ids")


@pytest.mark.parametrize("optimizer", ["sgd", "rowwise_adagrad"])
@pytest.mark.parametrize("w_dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("threshold,chunk,windows", [(256, 256, 32), (8, 8, 1), (4, 2, 32), (1, 1, 0)])
def test_fused_long_runs(optimizer, w_dtype, threshold, chunk, windows):
    """Long runs in one launch (fence, then countdown; the last chunk applies the update):
    same results as the oracle, and bitwise repeatable."""
    spec = small_spec("skewed").replace(optimizer=optimizer, w_dtype=w_dtype)
    bt = ti.make_batch(spec, 41)
    cfg = tbe.make_config(long_threshold=threshold, chunk=chunk, fused_long=1, bag_windows=windows)
    _, W1, m1, _ = run_and_check(bt, cfg, what=f"fused {optimizer} {w_dtype} t={threshold} c={chunk}")
    _, W2, m2, _ = run_and_check(bt, cfg, what="fused again")
    assert torch.equal(W1.cpu().view(torch.uint8), W2.cpu().view(torch.uint8))


@pytest.mark.parametrize("weighted", [False, True])
def test_fused_long_runs_mixed_D(weighted):
    spec = mixed_spec(torch.bfloat16, torch.int64, torch.int64, weighted).replace(optimizer="rowwise_adagrad")
    bt = ti.make_batch(spec, 43)
    run_and_check(bt, tbe.make_config(long_threshold=16, chunk=8, fused_long=1), what=f"fused mixed {weighted}")


def _hist_spec(E=64, D=128, L=("fixed", 128), B=517, optimizer="rowwise_adagrad", weighted=False,
               itype=torch.int64, otype=torch.int64):
    """Histogram-eligible table 0 (E <= 64, 64 <= D <= 128, fp16, long bags) plus two generic
    companions, one of them hit often enough to form long runs."""
    tables = (ti.TableSpec(E, D, L),
              ti.TableSpec(900, 64, ("poisson", 6.0, None, None), ("zipf", 1.1, None)),
              ti.TableSpec(5000, 128, ("poisson", 4.0, None, None)))
    return ti.BatchSpec(f"hist bwd E={E} D={D} L={L} B={B}", tables, B=B, w_dtype=torch.float16,
                        w_range=0.05, optimizer=optimizer, weighted=weighted, itype=itype, otype=otype,
                        pooling_hint=(128, 6, 4))


@pytest.mark.parametrize("optimizer", ["sgd", "rowwise_adagrad"])
@pytest.mark.parametrize("E,D,L,B", [(64, 128, ("fixed", 128), 517),
                                     (40, 80, ("poisson", 100.0, None, None), 333),   # ragged rows, cols
                                     (64, 64, ("poisson", 300.0, None, None), 130),   # bags > 256
                                     (17, 96, ("fixed", 64), 10),                     # one partial step
                                     (64, 128, ("fixed", 70), 4099)])                 # many steps
def test_hist_backward_matches_oracle(optimizer, E, D, L, B):
    """Counts x gradient on MFMA for the small table, generic runs for the rest: the updated
    weights and Adagrad state equal the oracle's within the stated bounds."""
    bt = ti.make_batch(_hist_spec(E, D, L, B, optimizer), 51)
    db, W, mom, r = run_and_check(bt, what=f"hist {optimizer} E={E} D={D} B={B}")
    assert db.tables.c.hist_table == 0


@pytest.mark.parametrize("itype,otype", [(torch.int32, torch.int32), (torch.int64, torch.int32)])
def test_hist_backward_index_types(itype, otype):
    bt = ti.make_batch(_hist_spec(B=700, itype=itype, otype=otype), 53)
    run_and_check(bt, what=f"hist {itype} {otype}")


def test_hist_backward_exact_with_integer_gradients():
    """Integer gradients in {-1, 0, 1}, zero fp16 weights, SGD with lr = -1: every sum is an
    integer below 2^11, so the histogram path, the generic run path and the oracle agree bit
    for bit."""
    spec = _hist_spec(B=300, optimizer="sgd", L=("poisson", 90.0, None, None))
    bt = ti.make_batch(spec, 57)
    g = torch.Generator().manual_seed(5)
    bt.grad_out = torch.randint(-1, 2, bt.grad_out.shape, generator=g).float()
    bt.weights = torch.zeros_like(bt.weights)
    outs = []
    for hist in (1, 0):
        db = DevBatch(bt)
        W, _ = db.backward(tbe.make_config(hist_enable=hist), lr=-1.0)
        outs.append(W.cpu())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    r = oracle_backward(bt, lr=-1.0)
    E0, D0 = bt.E[0], bt.D[0]
    assert np.array_equal(outs[0][:E0 * D0].double().numpy(), r["g"][:E0 * D0])
    assert np.abs(r["g"][:E0 * D0]).max() > 8  # not trivially zero


def test_hist_backward_deterministic_and_untouched_rows():
    spec = _hist_spec(E=64, D=128, L=("fixed", 1), B=40)   # 40 lookups over 64 rows: some untouched
    bt = ti.make_batch(spec, 59)
    outs = []
    for _ in range(2):
        db = DevBatch(bt)
        W0, m0 = db.W.clone(), db.mom.clone()
        W, mom = db.backward()
        outs.append((W.cpu(), mom.cpu()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])
    ids = bt.indices[bt.offsets[0]:bt.offsets[bt.B]].numpy().astype(np.int64)
    touched = np.zeros(bt.E[0], dtype=bool)
    touched[ids] = True
    assert 0 < touched.sum() < bt.E[0]
    Wt, W0t = outs[0][0][:bt.E[0] * 128].view(-1, 128), W0.cpu()[:bt.E[0] * 128].view(-1, 128)
    t = torch.from_numpy(touched)
    assert torch.equal(Wt[~t].view(torch.int16), W0t[~t].view(torch.int16))
    assert torch.equal(outs[0][1][:bt.E[0]][~t], m0.cpu()[:bt.E[0]][~t])
    assert (outs[0][1][:bt.E[0]][t] > m0.cpu()[:bt.E[0]][t]).all()
    run_and_check(bt, what="hist sparse")


def test_hist_backward_out_of_range_ids_dropped():
    spec = _hist_spec(B=200, optimizer="sgd")
    bt = ti.make_batch(spec, 61)
    idx = bt.indices.clone()
    bad = torch.zeros(idx.numel(), dtype=torch.bool)
    bad[::5] = True
    # one past the last row of the lookup's table, or negative
    t_of = torch.zeros(idx.numel(), dtype=torch.int64)
    for t in range(1, bt.T):
        t_of[int(bt.offsets[t * bt.B]):] = t
    past = torch.tensor(bt.E)[t_of]
    idx[bad] = torch.where(torch.arange(idx.numel())[bad] % 2 == 0, torch.tensor(-2), past[bad]).to(idx.dtype)
    bt.indices = idx
    db = DevBatch(bt)
    W, _ = db.backward()
    a = host_arrays(bt)
    keep = (~bad).double().numpy()
    ids = np.where(bad.numpy(), 0, a["idx"])
    r = oracle.backward(a["T"], a["B"], a["E"], a["D"], oracle.F16, a["W"], ids, a["off"], keep,
                        a["grad"], oracle.SGD, oracle.f32_literal(spec.lr))
    lr32 = oracle.f32_literal(spec.lr)
    check_weights(W, r, torch.float16, step_bound(r, bt.E, bt.D, lr32, 0.0, False), "hist bad ids")


def test_hist_backward_not_used_with_per_sample_weights():
    """With per-sample weights the small table goes through the generic runs (weighted counts
    are not integers); results still match the oracle."""
    bt = ti.make_batch(_hist_spec(B=300, weighted=True), 67)
    run_and_check(bt, what="hist table weighted")


@pytest.mark.parametrize("B", [97, 1000])
def test_hist_backward_middle_table(B):
    """The histogram table between two generic ones: its lookups leave the sorted key space and
    the later tables' positions close up (groups of 64 bags straddle both table boundaries)."""
    tables = (ti.TableSpec(3000, 64, ("poisson", 5.0, None, None), ("zipf", 1.2, None)),
              ti.TableSpec(50, 112, ("poisson", 80.0, None, None)),
              ti.TableSpec(700, 32, ("poisson", 3.0, None, None)))
    spec = ti.BatchSpec(f"hist middle B={B}", tables, B=B, w_dtype=torch.float16, w_range=0.05,
                        optimizer="rowwise_adagrad", pooling_hint=(5, 80, 3))
    bt = ti.make_batch(spec, 71)
    db, _, _, _ = run_and_check(bt, tbe.make_config(long_threshold=32, chunk=16), what=f"hist middle B={B}")
    assert db.tables.c.hist_table == 1


@pytest.mark.parametrize("windows", [8, 32, 64])
@pytest.mark.parametrize("name", ["skewed", "mixed"])
def test_long_chunks_grouped_by_window(name, windows):
    """Long-run chunks grouped by (table, bag window): same result as the ungrouped
    order bit for bit (each chunk writes its own partial; the apply sums them in chunk order),
    and the oracle's within the stated bounds."""
    bt = ti.make_batch(small_spec(name), 47)
    kw = dict(long_threshold=16, chunk=8)
    _, W1, m1, _ = run_and_check(bt, tbe.make_config(bag_windows=windows, **kw), what=f"{name} windows={windows}")
    _, W0, m0, _ = run_and_check(bt, tbe.make_config(bag_windows=1, **kw), what=f"{name} ungrouped")
    assert torch.equal(W1.cpu().view(torch.uint8), W0.cpu().view(torch.uint8))
    if m1 is not None:
        assert torch.equal(m1.cpu(), m0.cpu())


@pytest.mark.parametrize("name", ["skewed", "mixed", "histogram", "tiny"])
@pytest.mark.parametrize("fused", [0, 1])
def test_long_runs_on_second_stream_bitwise_same(name, fused):
    """bwd_streams = 2 runs the long-run chunks and their apply on the library's second
    stream, concurrent with the short runs: the same bits as one stream."""
    bt = ti.make_batch(small_spec(name), 73)
    kw = dict(long_threshold=16, chunk=8, fused_long=fused)
    _, W2, m2, _ = run_and_check(bt, tbe.make_config(bwd_streams=2, **kw), what=f"{name} two streams")
    _, W1, m1, _ = run_and_check(bt, tbe.make_config(bwd_streams=1, **kw), what=f"{name} one stream")
    assert torch.equal(W2.cpu().view(torch.uint8), W1.cpu().view(torch.uint8))
    if m2 is not None:
        assert torch.equal(m2.cpu(), m1.cpu())


def test_more_tables_than_the_lds_table_cache():
    """2100 tables (past the 2048 the classifier keeps in LDS): forward, transpose and a
    row-wise Adagrad step against the oracle, with widths 4 .. 64 and a few long runs."""
    D = (4, 8, 12, 16, 32, 64)
    tables = tuple(ti.TableSpec(40 + (t % 7), D[t % len(D)], ("poisson", 3.0, None, None),
                                ("zipf", 1.3, None) if t % 50 == 0 else ("uniform",))
                   for t in range(2100))
    spec = ti.BatchSpec("2100 tables", tables, B=90, w_dtype=torch.float16, w_range=0.5,
                        optimizer="rowwise_adagrad")
    bt = ti.make_batch(spec, 97)
    db = DevBatch(bt)
    out = db.forward()
    a = host_arrays(bt)
    ref, ref_abs = oracle.forward(a["T"], a["B"], a["E"], a["D"], a["W"], a["idx"], a["off"])
    from gpu_util import check_forward
    check_forward(out.cpu().numpy(), ref, ref_abs, False, "2100 tables forward")
    run_and_check(bt, tbe.make_config(long_threshold=32, chunk=16), what="2100 tables")


@pytest.mark.parametrize("optimizer", ["sgd", "rowwise_adagrad"])
def test_every_lookup_on_one_row(optimizer):
    """Degenerate batch: 200 000 lookups, all of row 3 of a one-row-hot table (and a one-row
    table beside it): one run of 200 000 lookups split into 782 chunks, and a run per table."""
    tables = (ti.TableSpec(10, 64, ("fixed", 200)), ti.TableSpec(1, 16, ("fixed", 2)))
    spec = ti.BatchSpec("one hot row", tables, B=1000, w_dtype=torch.float16, w_range=0.5,
                        optimizer=optimizer)
    bt = ti.make_batch(spec, 99)
    idx = bt.indices.clone()
    idx[:200_000] = 3
    bt.indices = idx
    db, W, mom, r = run_and_check(bt, what=f"one row {optimizer}")
    assert r["num_runs"] == 2
    W0 = bt.weights.view(-1)[:640].view(10, 64)
    got = W.cpu()[:640].view(10, 64)
    untouched = [i for i in range(10) if i != 3]
    assert torch.equal(got[untouched].view(torch.int16), W0[untouched].view(torch.int16))


@pytest.mark.parametrize("B", [10, 70, 200])
def test_hist_backward_table_last(B):
    """The histogram table last among the tables, B not a multiple of the 64-bag workgroup
    step: waves past the last bag stop at the table's end offset."""
    tables = (ti.TableSpec(700, 32, ("poisson", 3.0, None, None)),
              ti.TableSpec(64, 128, ("poisson", 90.0, None, None)))
    spec = ti.BatchSpec(f"hist last B={B}", tables, B=B, w_dtype=torch.float16, w_range=0.05,
                        optimizer="rowwise_adagrad", pooling_hint=(3, 90))
    bt = ti.make_batch(spec, 101)
    db, _, _, _ = run_and_check(bt, what=f"hist last B={B}")
    assert db.tables.c.hist_table == 1


@pytest.mark.parametrize("n", ["uniform", "mixed", "skewed"])
@pytest.mark.parametrize("tiny", [0, 1, 8, 64])
def test_tiny_run_steps(n, tiny):
    """Wave steps whose short runs all have at most tiny_runs lookups serve twice the runs
    with half the lanes each: the oracle's step either way, and with SGD (no cross-lane
    reduction) the same bits as with those steps off."""
    spec = small_spec(n)
    flush_print(f"tiny runs {n} tiny={tiny}")
    bt = ti.make_batch(spec, 61)
    cfg = tbe.make_config(tiny_runs=tiny, long_threshold=32, chunk=16)
    run_and_check(bt, cfg, what=f"tiny {n} {tiny}")
    W = {}
    for t in (0, tiny):
        db = DevBatch(bt)
        W[t], _ = db.backward(tbe.make_config(tiny_runs=t, long_threshold=32, chunk=16), optimizer="sgd")
        torch.cuda.synchronize()
    assert torch.equal(W[0].cpu().view(torch.uint8), W[tiny].cpu().view(torch.uint8))
