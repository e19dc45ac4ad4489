"""Bounds check and repair: repaired indices, offsets and counts equal the oracle's exactly."""
import json
import os

import numpy as np
import pytest
import torch

import bwd_tbe_fwd_amd as tbe
import oracle
import tbe_inputs as ti

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_bounds(E, D, B, indices, offsets, itype, otype):
    tables = tbe.Tables(E, D, B, torch.float32, device="cuda")
    idx = torch.as_tensor(np.asarray(indices), dtype=itype).cuda()
    off = torch.as_tensor(np.asarray(offsets), dtype=otype).cuda()
    counts = torch.full((2,), -1, dtype=torch.int64, device="cuda")
    ws = tbe.workspace(tbe.tbe_bounds_check_workspace_bytes(tables))
    tbe.tbe_bounds_check(tables, idx, off, counts, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy().astype(np.int64), off.cpu().numpy().astype(np.int64), counts.cpu().numpy()


@pytest.mark.parametrize("itype,otype", [(torch.int64, torch.int64), (torch.int32, torch.int32),
                                         (torch.int32, torch.int64)])
def test_bounds_golden_example(itype, otype):
    with open(os.path.join(GOLDEN, "bounds_example.json")) as f:
        g = json.load(f)
    idx, off, cnt = gpu_bounds(g["E"], [4] * g["T"], g["B"], g["indices"], g["offsets"], itype, otype)
    assert idx.tolist() == g["expected_indices"]
    assert off.tolist() == g["expected_offsets"]
    assert cnt.tolist() == g["expected_counts"]


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("itype", [torch.int32, torch.int64])
def test_bounds_injected_faults(seed, itype):
    spec = ti.BatchSpec("faults", (ti.TableSpec(1000, 8, ("poisson", 6.0, None, None)),
                                   ti.TableSpec(50, 8, ("poisson", 2.0, None, None)),
                                   ti.TableSpec(7, 8, ("fixed", 3))),
                        B=2999, w_dtype=torch.float32, w_range=0.5)
    bt = ti.make_batch(spec, seed, with_grad=False)
    rng = np.random.default_rng(seed)
    idx = bt.indices.numpy().astype(np.int64)
    off = bt.offsets.numpy().astype(np.int64)
    N = idx.size
    bad = rng.random(N) < 0.05
    idx[bad] = rng.choice([-1, -1000, 7, 50, 1000, 2 ** 30], size=int(bad.sum()))
    ob = rng.random(off.size) < 0.01
    off[ob] = rng.integers(-5, N + 50, size=int(ob.sum()))
    off[0] = rng.integers(-3, 3)
    off[-1] = N - rng.integers(0, 5)
    exp_idx, exp_off, exp_cnt = oracle.bounds_check(3, spec.B, bt.E, idx, off)
    assert exp_cnt[0] > 0 and exp_cnt[1] > 0
    got_idx, got_off, got_cnt = gpu_bounds(bt.E, bt.D, spec.B, idx, off, itype, torch.int64)
    assert np.array_equal(got_off, exp_off)
    assert np.array_equal(got_idx, exp_idx)
    assert got_cnt.tolist() == exp_cnt.tolist()


def test_bounds_valid_input_unchanged():
    bt = ti.make_batch(ti.scaled(ti.WORKLOADS["skewed"], B=4000, E_div=100, T=3), 5, with_grad=False)
    got_idx, got_off, cnt = gpu_bounds(bt.E, bt.D, bt.B, bt.indices.numpy(), bt.offsets.numpy(),
                                       torch.int64, torch.int64)
    assert cnt.tolist() == [0, 0]
    assert np.array_equal(got_idx, bt.indices.numpy())
    assert np.array_equal(got_off, bt.offsets.numpy())


def _faulty_batch(spec, seed):
    bt = ti.make_batch(spec, seed, with_grad=False)
    rng = np.random.default_rng(seed)
    idx = bt.indices.numpy().astype(np.int64)
    off = bt.offsets.numpy().astype(np.int64)
    N = idx.size
    bad = rng.random(N) < 0.05
    idx[bad] = rng.choice([-1, -77, 10 ** 6, 2 ** 31 - 1], size=int(bad.sum()))
    ob = rng.random(off.size) < 0.01
    off[ob] = rng.integers(-5, N + 50, size=int(ob.sum()))
    off[-1] = N - 3
    return bt, idx, off


@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("hist", [False, True])
@pytest.mark.parametrize("itype", [torch.int32, torch.int64])
def test_fused_bounds_forward_equals_check_then_forward(weighted, hist, itype):
    """tbe_forward_repair == tbe_bounds_check + tbe_forward: repaired arrays and counts exact,
    pooled output within the forward tolerance of the oracle on the repaired input."""
    from gpu_util import check_forward
    tables = (ti.TableSpec(64, 128, ("poisson", 70.0, None, None)),
              ti.TableSpec(500, 32, ("poisson", 5.0, None, None), ("zipf", 1.1, None)),
              ti.TableSpec(3000, 128, ("poisson", 12.0, None, None)))
    spec = ti.BatchSpec("fused bounds", tables, B=1111, w_dtype=torch.float16, w_range=0.05,
                        weighted=weighted, itype=itype, pooling_hint=(70, 5, 12) if hist else None)
    bt, idx, off = _faulty_batch(spec, 3)
    exp_idx, exp_off, exp_cnt = oracle.bounds_check(spec.T, spec.B, bt.E, idx, off)
    t = tbe.Tables(bt.E, bt.D, bt.B, bt.w_dtype, device="cuda", pooling_hint=spec.pooling_hint)
    assert (t.c.hist_table == 0) == hist  # used only without per-sample weights
    W = bt.weights.cuda()
    d_idx = torch.as_tensor(idx).to(itype).cuda()
    d_off = torch.as_tensor(off).cuda()
    psw = None if bt.psw is None else bt.psw.cuda()
    out = torch.full((bt.B, sum(bt.D)), float("nan"), device="cuda")
    counts = torch.full((2,), -1, dtype=torch.int64, device="cuda")
    ws = tbe.workspace(tbe.tbe_bounds_check_workspace_bytes(t))
    tbe.tbe_forward_repair(t, W, d_idx, d_off, psw, out, counts, ws)
    torch.cuda.synchronize()
    assert np.array_equal(d_off.cpu().numpy(), exp_off)
    assert np.array_equal(d_idx.cpu().numpy().astype(np.int64), exp_idx)
    assert counts.cpu().tolist() == exp_cnt.tolist()
    ref, ref_abs = oracle.forward(spec.T, spec.B, bt.E, bt.D, bt.weights.double().numpy(), exp_idx,
                                  exp_off, None if bt.psw is None else bt.psw.double().numpy())
    check_forward(out.cpu().numpy(), ref, ref_abs, False, "fused bounds forward")


@pytest.mark.parametrize("weighted", [False, True])
def test_fused_bounds_forward_unroll_is_bitwise_neutral(weighted):
    """The fused id check pools with 4 or 8 row loads in flight per lane group: the same
    output bits, repaired arrays and counts either way."""
    tables = (ti.TableSpec(500, 32, ("poisson", 5.0, None, None), ("zipf", 1.1, None)),
              ti.TableSpec(3000, 128, ("poisson", 40.0, None, None)),
              ti.TableSpec(200, 256, ("poisson", 3.0, None, None)))
    spec = ti.BatchSpec("fused unroll", tables, B=777, w_dtype=torch.bfloat16, w_range=0.05,
                        weighted=weighted)
    bt, idx, off = _faulty_batch(spec, 5)
    t = tbe.Tables(bt.E, bt.D, bt.B, bt.w_dtype, device="cuda")
    res = []
    for u in (4, 8):
        d_idx, d_off = torch.as_tensor(idx).cuda(), torch.as_tensor(off).cuda()
        out = torch.full((bt.B, sum(bt.D)), float("nan"), device="cuda")
        counts = torch.full((2,), -1, dtype=torch.int64, device="cuda")
        ws = tbe.workspace(tbe.tbe_bounds_check_workspace_bytes(t))
        psw = None if bt.psw is None else bt.psw.cuda()
        tbe.tbe_forward_repair(t, bt.weights.cuda(), d_idx, d_off, psw, out, counts, ws,
                               tbe.make_config(fwd_unroll=u))
        torch.cuda.synchronize()
        res.append((out.cpu(), d_idx.cpu(), d_off.cpu(), counts.cpu()))
    assert torch.equal(res[0][0].view(torch.int32), res[1][0].view(torch.int32))
    for a, b in zip(res[0][1:], res[1][1:]):
        assert torch.equal(a, b)
    assert res[0][3][0] > 0
