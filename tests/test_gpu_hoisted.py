"""Transpose hoisted into the forward: tbe_forward_hoisted runs the backward's linearize / sort /
run-length encoding / routing on a second stream while the forward pools; the backward with
pretransposed = 1 then skips its own transpose.  Everything must equal the plain two calls bit
for bit, and the oracle on the (repaired) input within the usual bounds."""
import numpy as np
import pytest
import torch

import bwd_tbe_fwd_amd as tbe
import oracle
import tbe_inputs as ti
from gpu_util import check_momentum, check_weights, flush_print, host_arrays, row_g_abs_sq, step_bound
from test_gpu_forward import small_spec

pytestmark = pytest.mark.gpu


def _inject(bt, seed, bad_offsets):
    """Out-of-range ids (5 %) and, optionally, broken offsets (1 %) on host copies."""
    rng = np.random.default_rng(seed)
    idx = bt.indices.numpy().astype(np.int64).copy()
    off = bt.offsets.numpy().astype(np.int64).copy()
    bad = rng.random(idx.size) < 0.05
    idx[bad] = rng.choice([-1, -50, 10 ** 7], size=int(bad.sum()))
    if bad_offsets:
        ob = rng.random(off.size) < 0.01
        off[ob] = rng.integers(-3, idx.size + 9, size=int(ob.sum()))
        off[-1] = idx.size - 2
    return idx, off


def _step(bt, idx, off, hoisted, repair, cfg_kw=None):
    """forward (+ repair) then backward, on device copies; returns everything observable."""
    cfg_kw = cfg_kw or {}
    spec = bt.spec
    t = tbe.Tables(bt.E, bt.D, bt.B, bt.w_dtype, device="cuda", pooling_hint=spec.pooling_hint)
    W = bt.weights.cuda()
    d_idx = torch.as_tensor(idx).to(bt.indices.dtype).cuda()
    d_off = torch.as_tensor(off).to(bt.offsets.dtype).cuda()
    psw = None if bt.psw is None else bt.psw.cuda()
    grad = bt.grad_out.cuda()
    mom = bt.momentum.cuda() if bt.momentum is not None else None
    out = torch.full((bt.B, sum(bt.D)), float("nan"), device="cuda")
    counts = torch.full((2,), -1, dtype=torch.int64, device="cuda") if repair else None
    bws = tbe.workspace(tbe.tbe_bounds_check_workspace_bytes(t)) if repair else None
    cfg = tbe.make_config(**cfg_kw)
    ws = tbe.workspace(tbe.tbe_backward_workspace_bytes(t, d_idx.numel(), psw is not None, cfg))
    if hoisted:
        tbe.tbe_forward_hoisted(t, W, d_idx, d_off, psw, out, counts, bws, ws, cfg)
        bcfg = tbe.make_config(pretransposed=1, **cfg_kw)
    else:
        if repair:
            tbe.tbe_forward_repair(t, W, d_idx, d_off, psw, out, counts, bws, cfg)
        else:
            tbe.tbe_forward(t, W, d_idx, d_off, psw, out, cfg)
        bcfg = cfg
    lr = oracle.f32_literal(spec.lr)
    if spec.optimizer == "sgd":
        tbe.tbe_backward_sgd(t, W, d_idx, d_off, psw, grad, lr, ws, bcfg)
    else:
        tbe.tbe_backward_rowwise_adagrad(t, W, mom, d_idx, d_off, psw, grad, lr,
                                         oracle.f32_literal(spec.eps), ws, bcfg)
    torch.cuda.synchronize()
    return dict(out=out.cpu(), W=W.cpu(), mom=None if mom is None else mom.cpu(),
                idx=d_idx.cpu(), off=d_off.cpu(), counts=None if counts is None else counts.cpu(),
                hist=t.c.hist_table)


def _assert_same(a, b):
    assert torch.equal(a["out"].view(torch.int32), b["out"].view(torch.int32))
    assert torch.equal(a["W"].view(torch.uint8), b["W"].view(torch.uint8))
    if a["mom"] is not None:
        assert torch.equal(a["mom"].view(torch.int32), b["mom"].view(torch.int32))
    assert torch.equal(a["idx"], b["idx"]) and torch.equal(a["off"], b["off"])
    if a["counts"] is not None:
        assert torch.equal(a["counts"], b["counts"])


@pytest.mark.parametrize("name", ["skewed", "mixed", "histogram", "uniform", "tiny"])
@pytest.mark.parametrize("repair", [False, True])
def test_hoisted_equals_plain(name, repair):
    spec = small_spec(name)
    flush_print(f"hoisted {name} repair={repair}")
    bt = ti.make_batch(spec, 81)
    idx, off = _inject(bt, 3, bad_offsets=repair)
    cfg_kw = dict(long_threshold=32, chunk=16)
    plain = _step(bt, idx, off, hoisted=False, repair=repair, cfg_kw=cfg_kw)
    hoist = _step(bt, idx, off, hoisted=True, repair=repair, cfg_kw=cfg_kw)
    _assert_same(plain, hoist)
    if repair:
        assert hoist["counts"][0] > 0 and hoist["counts"][1] > 0


@pytest.mark.parametrize("repair", [False, True])
@pytest.mark.parametrize("presort", [1, -1])
def test_hoisted_with_dense_rows(repair, presort):
    """The dense hot rows after the hoisted forward (fused repair or not; picked before the
    sort or from the long runs): bitwise the plain two calls, and the dense path really runs
    (fp32 weights: other low bits than the chunks)."""
    spec = small_spec("skewed").replace(w_dtype=torch.float32)
    bt = ti.make_batch(spec, 91)
    idx, off = _inject(bt, 11, bad_offsets=repair)
    kw = dict(long_threshold=32, chunk=16, dense_min=64, dense_presort=presort)
    plain = _step(bt, idx, off, hoisted=False, repair=repair, cfg_kw=kw)
    hoist = _step(bt, idx, off, hoisted=True, repair=repair, cfg_kw=kw)
    _assert_same(plain, hoist)
    chunks = _step(bt, idx, off, hoisted=True, repair=repair, cfg_kw=dict(kw, dense_min=0))
    assert not torch.equal(chunks["W"].view(torch.int32), hoist["W"].view(torch.int32))


@pytest.mark.parametrize("L,B,last", [(("poisson", 300.0, None, None), 130, False),
                                      (("poisson", 300.0, None, None), 77, True),
                                      (("fixed", 256), 33, False),
                                      (("fixed", 257), 48, True),
                                      (("poisson", 40.0, None, None), 1000, False)])
@pytest.mark.parametrize("repair", [False, True])
def test_hoisted_histogram_reuses_forward_counts(L, B, last, repair):
    """After the hoisted forward the histogram backward takes each bag's counts of its first
    256 ids from the forward and reads only the ids past them: bitwise equal to the plain two
    calls (which count every id in the backward), with bags longer than 256, bags of exactly
    256 and 257, a ragged last tile of 16 bags, the table first or last, and out-of-range ids
    dropped (no repair) or repaired to row 0."""
    hist = ti.TableSpec(64, 64, L)
    comp = ti.TableSpec(900, 64, ("poisson", 6.0, None, None), ("zipf", 1.1, None))
    tables, hint = ((comp, hist), (6, 128)) if last else ((hist, comp), (128, 6))
    spec = ti.BatchSpec(f"hoisted hist L={L} B={B} last={last}", tables, B=B, w_dtype=torch.float16,
                        w_range=0.05, optimizer="rowwise_adagrad", pooling_hint=hint)
    flush_print(spec.name, f"repair={repair}")
    bt = ti.make_batch(spec, 87)
    idx, off = _inject(bt, 7, bad_offsets=False)
    cfg_kw = dict(long_threshold=32, chunk=16)
    plain = _step(bt, idx, off, hoisted=False, repair=repair, cfg_kw=cfg_kw)
    hoist = _step(bt, idx, off, hoisted=True, repair=repair, cfg_kw=cfg_kw)
    assert hoist["hist"] == (1 if last else 0)
    _assert_same(plain, hoist)


@pytest.mark.parametrize("name", ["skewed", "histogram"])
def test_hoisted_repaired_matches_oracle(name):
    """The hoisted step on faulty input equals the oracle's step on the repaired input: an
    out-of-range id counts as row 0 of its table in the backward."""
    spec = small_spec(name)
    bt = ti.make_batch(spec, 83)
    idx, off = _inject(bt, 5, bad_offsets=True)
    got = _step(bt, idx, off, hoisted=True, repair=True)
    exp_idx, exp_off, exp_cnt = oracle.bounds_check(bt.T, bt.B, bt.E, idx, off)
    assert np.array_equal(got["idx"].numpy().astype(np.int64), exp_idx)
    assert np.array_equal(got["off"].numpy().astype(np.int64), exp_off)
    a = host_arrays(bt)
    r = oracle.backward(a["T"], a["B"], a["E"], a["D"], oracle.F16, a["W"], exp_idx, exp_off, None,
                        a["grad"], oracle.ROWWISE_ADAGRAD, oracle.f32_literal(spec.lr),
                        oracle.f32_literal(spec.eps), a["mom"])
    lr32, eps32 = oracle.f32_literal(spec.lr), oracle.f32_literal(spec.eps)
    check_weights(got["W"], r, bt.w_dtype, step_bound(r, bt.E, bt.D, lr32, eps32, True), f"hoisted {name}")
    gsq, Dr = row_g_abs_sq(r, bt.E, bt.D)
    check_momentum(got["mom"], r, Dr, gsq, f"hoisted {name}")


def test_hoisted_workspace_holds_latest_batch():
    """Two hoisted forwards into one workspace: the backward uses the second batch's runs."""
    spec = small_spec("skewed")
    bt1, bt2 = ti.make_batch(spec, 85), ti.make_batch(spec, 86)
    t = tbe.Tables(bt1.E, bt1.D, bt1.B, bt1.w_dtype, device="cuda")
    n = max(bt1.num_indices, bt2.num_indices)
    ws = tbe.workspace(tbe.tbe_backward_workspace_bytes(t, n, False))
    out = torch.empty(bt1.B, sum(bt1.D), device="cuda")
    tbe.tbe_forward_hoisted(t, bt1.weights.cuda(), bt1.indices.cuda(), bt1.offsets.cuda(), None, out,
                            None, None, ws)
    i2, o2 = bt2.indices.cuda(), bt2.offsets.cuda()
    tbe.tbe_forward_hoisted(t, bt2.weights.cuda(), i2, o2, None, out, None, None, ws)
    W, mom = bt2.weights.cuda(), bt2.momentum.cuda()
    lr, eps = oracle.f32_literal(spec.lr), oracle.f32_literal(spec.eps)
    tbe.tbe_backward_rowwise_adagrad(t, W, mom, i2, o2, None, bt2.grad_out.cuda(), lr, eps, ws,
                                     tbe.make_config(pretransposed=1))
    ref = _step(bt2, bt2.indices.numpy(), bt2.offsets.numpy(), hoisted=False, repair=False)
    assert torch.equal(W.cpu().view(torch.int16), ref["W"].view(torch.int16))
    assert torch.equal(mom.cpu(), ref["mom"])


@pytest.mark.parametrize("name,kw", [("histogram", dict(B=20000)),
                                     ("skewed", dict(B=3000, E_div=400, T=8)),
                                     ("mixed", dict(B=1500, E_div=50))])
@pytest.mark.parametrize("repair", [False, True])
def test_by_table_sort_same_step(name, kw, repair):
    """A whole step whose sort takes each table on its own (sort_by_table = 1) equals the step
    with one sort of the linearized ids bit for bit, hoisted and plain, with out-of-range ids
    (dropped from the sort, or repaired to row 0 with broken offsets repaired too), the
    histogram table left out of the sort, and dense rows picked before the sort."""
    spec = ti.scaled(ti.WORKLOADS[name], **kw)
    bt = ti.make_batch(spec, 93)
    flush_print(f"by-table step {name} {kw} repair={repair} N={bt.num_indices}")
    idx, off = _inject(bt, 13, bad_offsets=repair)
    base = dict(long_threshold=32, chunk=16, dense_min=64, dense_presort=1)
    one = _step(bt, idx, off, hoisted=False, repair=repair, cfg_kw=dict(base, sort_by_table=-1))
    for hoisted in (False, True):
        by = _step(bt, idx, off, hoisted=hoisted, repair=repair, cfg_kw=dict(base, sort_by_table=1))
        _assert_same(one, by)
