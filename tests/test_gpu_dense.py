"""Dense hot rows: per table, the rows of at least dense_min lookups (up to 128, in key order)
are updated from per-bag counts x grad_out on MFMA.  Picked before the sort (dense_presort = 1:
counted on a sample, every lookup up to 2^20 lookups, and left out of the sorted runs) or from
the long runs after it (-1: their chunks skipped).  The step equals the oracle's within the
usual bounds, is bitwise repeatable, and is exact with integer gradients."""
import numpy as np
import pytest
import torch

import bwd_tbe_fwd_amd as tbe
import oracle
import tbe_inputs as ti
from gpu_util import DevBatch, check_weights, flush_print, host_arrays, oracle_backward, step_bound
from test_gpu_backward import run_and_check

pytestmark = pytest.mark.gpu


def _spec(D=(128, 64, 32, 200), E=(300, 1000, 400, 250), B=777, L=(60.0, 40.0, 30.0, 20.0),
          zipf=1.1, w_dtype=torch.float16, optimizer="rowwise_adagrad", itype=torch.int64,
          otype=torch.int64, weighted=False, hint=None):
    """Skewed tables: eligible widths (128, 64, 32) and one that is not (200)."""
    tables = tuple(ti.TableSpec(e, d, ("poisson", l, None, None), ("zipf", zipf, None))
                   for e, d, l in zip(E, D, L))
    return ti.BatchSpec(f"dense D={D} B={B}", tables, B=B, w_dtype=w_dtype, w_range=0.05,
                        optimizer=optimizer, itype=itype, otype=otype, weighted=weighted,
                        pooling_hint=hint)


PRESORT = [1, -1]


def _cfg(dense_min, presort=1, **kw):
    return tbe.make_config(long_threshold=16, chunk=8, dense_min=dense_min, dense_presort=presort, **kw)


def _long_lens(bt, threshold):
    """Per table: lengths of its runs of >= threshold lookups, in key order."""
    idx, off, B = bt.indices.numpy().astype(np.int64), bt.offsets.numpy().astype(np.int64), bt.B
    out = []
    for t in range(bt.T):
        lk = idx[off[t * B]:off[(t + 1) * B]]
        lk = lk[(lk >= 0) & (lk < bt.E[t])]
        c = np.bincount(lk, minlength=bt.E[t])
        out.append(c[c >= threshold])
    return out


@pytest.mark.parametrize("w_dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("optimizer", ["sgd", "rowwise_adagrad"])
@pytest.mark.parametrize("presort", PRESORT)
def test_dense_rows_match_oracle(w_dtype, optimizer, presort):
    spec = _spec(w_dtype=w_dtype, optimizer=optimizer)
    bt = ti.make_batch(spec, 71)
    lens = _long_lens(bt, 48)
    assert sum(int((l >= 48).sum()) for l in lens[:3]) > 20   # the dense path has rows to take
    flush_print(f"dense {w_dtype} {optimizer} presort={presort}")
    run_and_check(bt, _cfg(48, presort), what=f"dense {w_dtype} {optimizer} presort={presort}")


@pytest.mark.parametrize("itype,otype", [(torch.int32, torch.int32), (torch.int64, torch.int32),
                                         (torch.int32, torch.int64)])
def test_dense_rows_index_types(itype, otype):
    bt = ti.make_batch(_spec(itype=itype, otype=otype, B=300), 73)
    run_and_check(bt, _cfg(32), what=f"dense {itype} {otype}")


@pytest.mark.parametrize("presort", PRESORT)
def test_dense_rows_change_the_summation_and_repeat(presort):
    """fp32 weights, Adagrad: the dense path sums the hot rows' gradients in another order than
    the chunks (other low bits, so it did run), and the same bits on every call."""
    bt = ti.make_batch(_spec(w_dtype=torch.float32), 75)
    outs = {}
    for dm in (0, 48, 48):
        db = DevBatch(bt)
        W, mom = db.backward(_cfg(dm, presort))
        torch.cuda.synchronize()
        outs.setdefault(dm, []).append((W.cpu(), mom.cpu()))
    (Wa, ma), (Wb, mb) = outs[48]
    assert torch.equal(Wa.view(torch.int32), Wb.view(torch.int32)) and torch.equal(ma, mb)
    W0, _ = outs[0][0]
    assert not torch.equal(W0.view(torch.int32), Wa.view(torch.int32))


@pytest.mark.parametrize("dense_min", [16, 48])
@pytest.mark.parametrize("presort", PRESORT)
def test_dense_rows_exact_with_integer_gradients(dense_min, presort):
    """Gradients in {-1, 0, 1}, zero weights, SGD with lr = -1: every sum is an exact integer
    in fp32, so the dense path, the chunk path and the oracle agree bit for bit."""
    spec = _spec(w_dtype=torch.float32, optimizer="sgd", B=500)
    bt = ti.make_batch(spec, 77)
    g = torch.Generator().manual_seed(7)
    bt.grad_out = torch.randint(-1, 2, bt.grad_out.shape, generator=g).float()
    bt.weights = torch.zeros_like(bt.weights)
    outs = []
    for dm in (dense_min, 0):
        db = DevBatch(bt)
        W, _ = db.backward(_cfg(dm, presort), lr=-1.0)
        torch.cuda.synchronize()
        outs.append(W.cpu())
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    r = oracle_backward(bt, lr=-1.0)
    assert np.array_equal(outs[0].double().numpy(), r["g"])
    assert np.abs(r["g"]).max() > 20


@pytest.mark.parametrize("presort", PRESORT)
def test_dense_rows_more_than_128_per_table(presort):
    """Every row of a 600-row table is hit about 120 times: the 128 with the most lookups take
    the dense path, the rest their chunks."""
    tables = (ti.TableSpec(600, 128, ("fixed", 100)), ti.TableSpec(3000, 64, ("poisson", 5.0, None, None)))
    spec = ti.BatchSpec("dense cap", tables, B=720, w_dtype=torch.float32, w_range=0.05,
                        optimizer="rowwise_adagrad")
    bt = ti.make_batch(spec, 79)
    assert int((_long_lens(bt, 64)[0] >= 64).sum()) > 300
    run_and_check(bt, _cfg(64, presort), what=f"dense cap presort={presort}")


@pytest.mark.parametrize("presort", PRESORT)
def test_dense_rows_with_histogram_table_and_bad_ids(presort):
    """A histogram-eligible small table (its own MFMA path), dense rows in the others, and ids
    outside their tables (dropped by both paths)."""
    tables = (ti.TableSpec(64, 128, ("fixed", 100)),
              ti.TableSpec(400, 128, ("poisson", 50.0, None, None), ("zipf", 1.2, None)),
              ti.TableSpec(900, 64, ("poisson", 20.0, None, None), ("zipf", 1.1, None)))
    spec = ti.BatchSpec("dense + hist", tables, B=600, w_dtype=torch.float16, w_range=0.05,
                        optimizer="sgd", pooling_hint=(100, 50, 20))
    bt = ti.make_batch(spec, 81)
    idx = bt.indices.clone()
    bad = torch.zeros(idx.numel(), dtype=torch.bool)
    bad[3::11] = True
    idx[bad] = torch.where(torch.arange(idx.numel())[bad] % 2 == 0, torch.tensor(-1),
                           torch.tensor(10 ** 6)).to(idx.dtype)
    bt.indices = idx
    db = DevBatch(bt)
    assert db.tables.c.hist_table == 0
    W, _ = db.backward(_cfg(32, presort))
    torch.cuda.synchronize()
    a = host_arrays(bt)
    keep = (~bad).double().numpy()
    ids = np.where(bad.numpy(), 0, a["idx"])
    lr32 = oracle.f32_literal(spec.lr)
    r = oracle.backward(a["T"], a["B"], a["E"], a["D"], oracle.F16, a["W"], ids, a["off"], keep,
                        a["grad"], oracle.SGD, lr32)
    check_weights(W, r, torch.float16, step_bound(r, bt.E, bt.D, lr32, 0.0, False), "dense + hist")


@pytest.mark.parametrize("B", [1, 63, 64, 65, 4100])
def test_dense_rows_bag_counts(B):
    """Bag counts around the 64-bag step and the partial count."""
    spec = _spec(B=B, L=(90.0, 60.0, 30.0, 10.0))
    bt = ti.make_batch(spec, 83)
    run_and_check(bt, _cfg(16), what=f"dense B={B}")


@pytest.mark.parametrize("w_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("optimizer", ["sgd", "rowwise_adagrad"])
@pytest.mark.parametrize("presort", PRESORT)
def test_dense_rows_with_per_sample_weights(w_dtype, optimizer, presort):
    """Per-sample weights: a dense row takes, per bag, the sum of the weights of the bag's
    lookups of it in place of their count (one lane a bag, in position order), in three exact
    bf16 parts against the gradient's three.  The step matches the oracle and repeats bit for
    bit; with fp32 weights it also differs in its low bits from the chunk path, so the dense
    path ran."""
    bt = ti.make_batch(_spec(w_dtype=w_dtype, optimizer=optimizer, weighted=True, B=400), 85)
    what = f"dense weighted {w_dtype} {optimizer} presort={presort}"
    flush_print(what)
    run_and_check(bt, _cfg(16, presort), what=what)
    outs = []
    for dm in (16, 16, 0):
        db = DevBatch(bt)
        W, mom = db.backward(_cfg(dm, presort))
        torch.cuda.synchronize()
        outs.append((W.cpu(), None if mom is None else mom.cpu()))
    assert torch.equal(outs[0][0].view(torch.uint8), outs[1][0].view(torch.uint8)), what
    if outs[0][1] is not None:
        assert torch.equal(outs[0][1], outs[1][1]), what
    if w_dtype == torch.float32:
        assert not torch.equal(outs[0][0].view(torch.int32), outs[2][0].view(torch.int32)), what


@pytest.mark.parametrize("L", [300, 70000])
@pytest.mark.parametrize("presort", PRESORT)
def test_dense_rows_counts_above_255(L, presort):
    """Bags with hundreds (and tens of thousands) of lookups of one row: the counts go through
    the bf16 product byte by byte and stay exact (integer gradients, so bit for bit)."""
    tables = (ti.TableSpec(2, 64, ("fixed", L)), ti.TableSpec(500, 128, ("poisson", 8.0, None, None)))
    spec = ti.BatchSpec(f"dense big counts L={L}", tables, B=70 if L < 1000 else 3,
                        w_dtype=torch.float32, w_range=0.05, optimizer="sgd")
    bt = ti.make_batch(spec, 87)
    g = torch.Generator().manual_seed(9)
    bt.grad_out = torch.randint(-1, 2, bt.grad_out.shape, generator=g).float()
    bt.weights = torch.zeros_like(bt.weights)
    db = DevBatch(bt)
    W, _ = db.backward(_cfg(16, presort), lr=-1.0)
    torch.cuda.synchronize()
    r = oracle_backward(bt, lr=-1.0)
    assert np.array_equal(W.cpu().double().numpy(), r["g"])
    assert np.abs(r["g"][:128]).max() > 255


@pytest.mark.parametrize("presort", PRESORT)
def test_dense_rows_count_above_2_pow_24(presort):
    """One bag with 3 * 2^23 lookups of one row: an fp32 count would stop at 2^24 (a third
    short); the wave that counts that bag counts in uint32, so the step stays exact (integer
    gradients, zero weights, SGD with lr = -1, so the weights are the oracle's sums bit for
    bit)."""
    L = 3 * 2 ** 23
    tables = (ti.TableSpec(1, 64, ("fixed", L)), ti.TableSpec(500, 128, ("poisson", 8.0, None, None)))
    spec = ti.BatchSpec("dense count 3*2^23", tables, B=1, w_dtype=torch.float32, w_range=0.05,
                        optimizer="sgd", itype=torch.int32, otype=torch.int64)
    bt = ti.make_batch(spec, 88)
    g = torch.Generator().manual_seed(10)
    bt.grad_out = torch.randint(-1, 2, bt.grad_out.shape, generator=g).float()
    bt.grad_out[0, :64] = torch.tensor([1.0, -1.0] * 32)
    bt.weights = torch.zeros_like(bt.weights)
    flush_print(f"dense count above 2^24 presort={presort}: {bt.indices.numel()} lookups")
    db = DevBatch(bt)
    W, _ = db.backward(_cfg(16, presort), lr=-1.0)
    torch.cuda.synchronize()
    r = oracle_backward(bt, lr=-1.0)
    assert np.abs(r["g"][:64]).max() == L
    assert np.array_equal(W.cpu().double().numpy(), r["g"])


@pytest.mark.parametrize("presort", PRESORT)
def test_dense_rows_on_the_second_stream(presort):
    """The dense rows, chunks and applies on the library's second stream, concurrent with the
    short runs: the same bits as on one stream."""
    bt = ti.make_batch(_spec(w_dtype=torch.float32), 89)
    outs = []
    for streams in (1, 2):
        db = DevBatch(bt)
        W, mom = db.backward(_cfg(48, presort, bwd_streams=streams))
        torch.cuda.synchronize()
        outs.append((W.cpu(), mom.cpu()))
    assert torch.equal(outs[0][0].view(torch.int32), outs[1][0].view(torch.int32))
    assert torch.equal(outs[0][1], outs[1][1])


def test_dense_rows_from_a_strided_sample():
    """Over 2^20 lookups the rows are picked from 64 positions in every 128 (rows of about
    dense_min lookups may fall either way): still the oracle's step, the same bits on every
    call, and other low bits than without the dense path (so it did run)."""
    tables = (ti.TableSpec(2000, 128, ("poisson", 40.0, None, None), ("zipf", 1.1, None)),
              ti.TableSpec(5000, 64, ("poisson", 30.0, None, None), ("zipf", 1.05, None)),
              ti.TableSpec(3000, 32, ("poisson", 20.0, None, None)))
    spec = ti.BatchSpec("dense sampled", tables, B=16384, w_dtype=torch.float32, w_range=0.05,
                        optimizer="rowwise_adagrad")
    bt = ti.make_batch(spec, 93)
    assert 2 ** 20 < bt.indices.numel() <= 2 ** 21
    assert int((_long_lens(bt, 512)[0] >= 512).sum()) > 20
    flush_print("dense sampled")
    _, Wa, ma, _ = run_and_check(bt, _cfg(256), what="dense sampled")
    db = DevBatch(bt)
    Wb, mb = db.backward(_cfg(256))
    db0 = DevBatch(bt)
    W0, _ = db0.backward(_cfg(0))
    torch.cuda.synchronize()
    assert torch.equal(Wa.cpu().view(torch.int32), Wb.cpu().view(torch.int32))
    assert torch.equal(ma.cpu(), mb.cpu())
    assert not torch.equal(W0.cpu().view(torch.int32), Wa.cpu().view(torch.int32))


def test_dense_rows_many_tables():
    """40 tables: the dense-row key set (2 x 128 slots a table, rounded up to a power of two)
    outgrows LDS, so linearize filters keys in LDS and probes the set in global memory."""
    tables = tuple(ti.TableSpec(300 + 10 * t, (32, 64, 128)[t % 3], ("poisson", 20.0, None, None),
                                ("zipf", 1.1, None)) for t in range(40))
    spec = ti.BatchSpec("dense 40 tables", tables, B=300, w_dtype=torch.float16, w_range=0.05,
                        optimizer="sgd")
    bt = ti.make_batch(spec, 95)
    assert sum(int((l >= 32).sum()) for l in _long_lens(bt, 32)) > 200
    flush_print("dense 40 tables")
    run_and_check(bt, _cfg(32), what="dense 40 tables")


@pytest.mark.parametrize("presort", PRESORT)
def test_dense_rows_are_the_longest_128(presort):
    """More than 128 rows qualify: the dense path takes the 128 with the most lookups (among
    equal counts the smaller row ids).  fp32 weights: a row the dense path updates ends with
    other low bits than on the chunk path (almost always), so the rows whose bits differ must
    lie in that set, and most of it must show."""
    tables = (ti.TableSpec(600, 64, ("fixed", 100)),)
    spec = ti.BatchSpec("dense top 128", tables, B=720, w_dtype=torch.float32, w_range=0.05,
                        optimizer="sgd")
    bt = ti.make_batch(spec, 97)
    c = np.bincount(bt.indices.numpy().astype(np.int64), minlength=600)
    q = np.flatnonzero(c >= 64)
    assert q.size > 200
    top = set(sorted(q.tolist(), key=lambda r: (-int(c[r]), r))[:128])
    outs = []
    for dm in (64, 0):
        db = DevBatch(bt)
        W, _ = db.backward(_cfg(dm, presort))
        torch.cuda.synchronize()
        outs.append(W.cpu().view(600, 64).view(torch.int32))
    differ = set(torch.nonzero((outs[0] != outs[1]).any(dim=1)).flatten().tolist())
    assert differ <= top and len(differ) >= 100, (len(differ), sorted(differ - top)[:5])


@pytest.mark.parametrize("seed", [1, 2])
def test_dense_rows_random_shapes(seed):
    """Seeded random shapes through both picks: table sizes from 2 rows up, widths in and out
    of the dense path's range, every weight and index type, with and without per-sample
    weights, thresholds and chunk sizes, one or two streams; every step checked against the
    oracle."""
    rng = np.random.default_rng(seed)
    for it in range(30):
        T = int(rng.integers(1, 6))
        tables = tuple(ti.TableSpec(int(rng.choice([2, 17, 64, 300, 1000, 5000])),
                                    int(rng.choice([8, 16, 48, 64, 96, 128, 200])),
                                    ("poisson", float(rng.choice([3, 10, 30, 80])), None, None),
                                    ("zipf", float(rng.choice([0.9, 1.1, 1.3])), None)
                                    if rng.random() < 0.8 else ("uniform",))
                       for _ in range(T))
        spec = ti.BatchSpec(f"dense random {seed}.{it}", tables,
                            B=int(rng.choice([1, 7, 63, 64, 65, 200, 700, 3000])),
                            w_dtype=[torch.float32, torch.float16, torch.bfloat16][int(rng.integers(0, 3))],
                            w_range=0.05, optimizer=["sgd", "rowwise_adagrad"][int(rng.integers(0, 2))],
                            itype=[torch.int32, torch.int64][int(rng.integers(0, 2))],
                            otype=[torch.int32, torch.int64][int(rng.integers(0, 2))])
        cfg = tbe.make_config(long_threshold=int(rng.choice([16, 32, 256])),
                              chunk=int(rng.choice([8, 16, 256])),
                              dense_min=int(rng.choice([16, 24, 40, 100])),
                              dense_presort=int(rng.choice([1, -1])),
                              bwd_streams=int(rng.choice([0, 1, 2])))
        spec = spec.replace(weighted=bool(rng.random() < 0.4))
        bt = ti.make_batch(spec, 1000 * seed + it)
        run_and_check(bt, cfg, what=f"{spec.name} weighted={spec.weighted}: {bt.indices.numel()} lookups")


@pytest.mark.parametrize("seed", [3, 4])
def test_dense_rows_beside_the_short_runs_random_shapes(seed):
    """Seeded random shapes through the automatic backward's side-by-side mode: with the dense
    rows picked before the sort and every table in one short-run bucket, the dense rows (and
    the histogram table, when there is one) run on the second stream beside the short runs,
    whose two grids take their work from one shared counter, the long runs between them on the
    second stream.  Every step is checked against the oracle, the second short-run grid must
    have run, and every third step also goes through the hoisted forward, bit for bit equal to
    the plain calls."""
    from test_gpu_hoisted import _assert_same, _step
    rng = np.random.default_rng(seed)
    for it in range(12):
        bucket = int(rng.choice([64, 128]))
        widths = [d for d in range(16, 129, 16) if bucket // 2 < d <= bucket]
        T = int(rng.integers(1, 5))
        lam = [float(rng.choice([10, 30, 80])) for _ in range(T)]
        tables = [ti.TableSpec(int(rng.choice([40, 300, 1000, 5000])), int(rng.choice(widths)),
                               ("poisson", l, None, None), ("zipf", float(rng.choice([1.05, 1.2, 1.4])), None))
                  for l in lam]
        hint = [max(1, int(l)) for l in lam]
        if bucket == 128 and rng.random() < 0.5:   # a histogram table (at most 64 rows), same bucket
            at = int(rng.integers(0, T + 1))
            L = int(rng.choice([64, 100, 300]))
            tables.insert(at, ti.TableSpec(int(rng.choice([17, 64])), 128, ("fixed", L)))
            hint.insert(at, L)
        spec = ti.BatchSpec(f"beside {seed}.{it}", tuple(tables), B=int(rng.choice([63, 200, 700, 3000])),
                            w_dtype=[torch.float32, torch.float16, torch.bfloat16][int(rng.integers(0, 3))],
                            w_range=0.05, optimizer=["sgd", "rowwise_adagrad"][int(rng.integers(0, 2))],
                            itype=[torch.int32, torch.int64][int(rng.integers(0, 2))],
                            otype=[torch.int32, torch.int64][int(rng.integers(0, 2))],
                            pooling_hint=tuple(hint))
        bt = ti.make_batch(spec, 2000 * seed + it)
        kw = dict(long_threshold=int(rng.choice([16, 32, 256])), chunk=int(rng.choice([8, 16, 256])),
                  dense_min=int(rng.choice([16, 40, 100])), dense_presort=1)
        what = f"{spec.name}: D={bt.D} B={bt.B} {bt.indices.numel()} lookups {kw}"
        flush_print(what)
        tbe.tbe_profile_select("short_run_more")
        db, _, _, _ = run_and_check(bt, tbe.make_config(**kw), what=what)
        n_more, _ = tbe.tbe_profile_read()
        tbe.tbe_profile_select(None)
        assert n_more >= 1, what
        if it % 3 == 0:
            idx, off = bt.indices.numpy(), bt.offsets.numpy()
            repair = bool(rng.integers(0, 2))
            _assert_same(_step(bt, idx, off, hoisted=False, repair=repair, cfg_kw=kw),
                         _step(bt, idx, off, hoisted=True, repair=repair, cfg_kw=kw))
