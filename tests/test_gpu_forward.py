"""Forward parity: the HIP gather / histogram kernels against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import bwd_tbe_fwd_amd as tbe
import oracle
import tbe_inputs as ti
from gpu_util import DevBatch, check_forward, flush_print, host_arrays

pytestmark = pytest.mark.gpu


def small_spec(name: str) -> ti.BatchSpec:
    """A workload's recipe at a size the oracle finishes in about a second; ragged B and N."""
    W = ti.WORKLOADS
    if name == "tiny":
        return W["tiny"]
    if name == "uniform":
        return ti.scaled(W["uniform"], B=1500, E_div=500, T=5)
    if name == "histogram":
        h = W["histogram"]
        return h.replace(name="hist+companion small",
                         tables=(h.tables[0], ti.TableSpec(1000, 128, ("poisson", 10.0, None, None))),
                         B=700)
    if name == "mixed":
        return ti.scaled(W["mixed"], B=700, E_div=200, T=8)
    return ti.scaled(W["skewed"], B=1500, E_div=200, T=4)


WORKLOAD_NAMES = ["tiny", "uniform", "histogram", "mixed", "skewed"]


def mixed_spec(w_dtype, itype, otype, weighted, B=333):
    tables = (ti.TableSpec(50, 4, ("poisson", 3.0, None, None), ("zipf", 1.2, None)),
              ti.TableSpec(700, 12, ("poisson", 9.0, None, None)),
              ti.TableSpec(300, 36, ("poisson", 1.0, None, None)),   # many empty bags
              ti.TableSpec(2000, 128, ("poisson", 70.0, None, None), ("zipf", 1.05, None)),
              ti.TableSpec(90, 200, ("fixed", 5)),
              ti.TableSpec(40, 512, ("poisson", 4.0, None, None)),
              ti.TableSpec(30, 1024, ("poisson", 2.0, None, None)))
    return ti.BatchSpec("mixed D", tables, B=B, w_dtype=w_dtype, w_range=0.5, itype=itype,
                        otype=otype, weighted=weighted, optimizer="sgd")


def _oracle_forward(bt):
    a = host_arrays(bt)
    return oracle.forward(a["T"], a["B"], a["E"], a["D"], a["W"], a["idx"], a["off"], a["psw"])


@pytest.mark.parametrize("n", WORKLOAD_NAMES)
def test_forward_configs_small(n):
    spec = small_spec(n)
    flush_print(f"forward {n}: {spec.name}")
    bt = ti.make_batch(spec)
    db = DevBatch(bt)
    out = db.forward()
    torch.cuda.synchronize()
    ref, ref_abs = _oracle_forward(bt)
    check_forward(out.cpu().numpy(), ref, ref_abs, bt.w_dtype == torch.float32, n)


@pytest.mark.parametrize("w_dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("itype,otype", [(torch.int32, torch.int32), (torch.int32, torch.int64),
                                         (torch.int64, torch.int32), (torch.int64, torch.int64)])
@pytest.mark.parametrize("weighted", [False, True])
def test_forward_dtypes_mixed_D(w_dtype, itype, otype, weighted):
    spec = mixed_spec(w_dtype, itype, otype, weighted)
    bt = ti.make_batch(spec, 77)
    db = DevBatch(bt)
    out = db.forward()
    torch.cuda.synchronize()
    ref, ref_abs = _oracle_forward(bt)
    check_forward(out.cpu().numpy(), ref, ref_abs, w_dtype == torch.float32,
                  f"{w_dtype} {itype} {otype} psw={weighted}")


def test_forward_D_not_multiple_of_8():
    # fp16 tables with D % 8 != 0 use 8-byte vectors
    tables = (ti.TableSpec(100, 4), ti.TableSpec(100, 20, ("poisson", 5.0, None, None)),
              ti.TableSpec(100, 44))
    spec = ti.BatchSpec("D%8", tables, B=130, w_dtype=torch.float16, w_range=0.5)
    bt = ti.make_batch(spec, 5)
    db = DevBatch(bt)
    assert db.tables.c.all_D_mult8 == 0
    out = db.forward()
    ref, ref_abs = _oracle_forward(bt)
    check_forward(out.cpu().numpy(), ref, ref_abs, False, "D%8")


def test_forward_unroll_knob_is_bitwise_neutral():
    bt = ti.make_batch(small_spec("skewed"), 9)
    db = DevBatch(bt)
    outs = [db.forward(tbe.make_config(fwd_unroll=u)).cpu() for u in (2, 4, 8)]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


@pytest.mark.parametrize("name", ["skewed", "mixed"])
def test_forward_bags_per_wave_knob_is_bitwise_neutral(name):
    """Each bag is pooled by one wave in the same order whatever the number of bags a wave
    takes per step (ragged: B is not a multiple of any of them)."""
    bt = ti.make_batch(small_spec(name), 10)
    db = DevBatch(bt)
    outs = [db.forward(tbe.make_config(bags_per_wave=g)).cpu() for g in (64, 1, 7, 16, 33)]
    for o in outs[1:]:
        assert torch.equal(outs[0], o)
    ref, ref_abs = _oracle_forward(bt)
    check_forward(outs[0].numpy(), ref, ref_abs, bt.w_dtype == torch.float32, name)


def _integer_weights(bt, lo=-8, hi=8, seed=0):
    g = torch.Generator().manual_seed(seed)
    bt.weights = torch.randint(lo, hi + 1, bt.weights.shape, generator=g).to(bt.w_dtype)
    return bt


@pytest.mark.parametrize("L", [("fixed", 128), ("poisson", 200.0, None, None)])
def test_histogram_path_exact(L):
    """Small-table histogram + MFMA path: with integer-valued weights every sum is exact, so
    the path must equal both the generic gather and the oracle bit for bit (bags longer than
    256 exercise the gathered tail)."""
    spec = ti.BatchSpec("hist", (ti.TableSpec(64, 128, L), ti.TableSpec(500, 64, ("poisson", 3.0, None, None)),
                                 ti.TableSpec(37, 96, ("poisson", 90.0, None, None))),
                        B=517, w_dtype=torch.float16, w_range=0.05, pooling_hint=(128, 3, 90))
    bt = _integer_weights(ti.make_batch(spec, 3))
    db = DevBatch(bt)
    assert db.tables.c.hist_table == 0
    on = db.forward(tbe.make_config(hist_enable=1)).cpu()
    off = db.forward(tbe.make_config(hist_enable=0)).cpu()
    ref, _ = _oracle_forward(bt)
    assert torch.equal(on, off)
    assert np.array_equal(on.double().numpy(), ref)


def test_histogram_path_matches_oracle_histogram_recipe():
    bt = ti.make_batch(small_spec("histogram"))
    db = DevBatch(bt)
    assert db.tables.c.hist_table == 0
    out = db.forward()
    ref, ref_abs = _oracle_forward(bt)
    check_forward(out.cpu().numpy(), ref, ref_abs, False, "histogram workload")


def test_histogram_not_used_with_per_sample_weights():
    spec = ti.BatchSpec("hist psw", (ti.TableSpec(64, 128, ("fixed", 70)),), B=100,
                        w_dtype=torch.float16, w_range=0.05, weighted=True, pooling_hint=(70,))
    bt = ti.make_batch(spec, 4)
    db = DevBatch(bt)
    out = db.forward()
    ref, ref_abs = _oracle_forward(bt)
    check_forward(out.cpu().numpy(), ref, ref_abs, False, "hist table with psw")


def test_forward_edge_cases():
    # B = 1 and T = 1; all bags empty; no lookups at all
    spec = ti.BatchSpec("one bag", (ti.TableSpec(10, 8, ("fixed", 4)),), B=1, w_dtype=torch.float32,
                        w_range=0.5)
    bt = ti.make_batch(spec, 1)
    db = DevBatch(bt)
    ref, ref_abs = _oracle_forward(bt)
    check_forward(db.forward().cpu().numpy(), ref, ref_abs, True, "B=1")
    spec0 = ti.BatchSpec("empty", (ti.TableSpec(10, 8, ("fixed", 0)), ti.TableSpec(5, 16, ("fixed", 0))),
                         B=70, w_dtype=torch.float16, w_range=0.5)
    bt0 = ti.make_batch(spec0, 1)
    assert bt0.num_indices == 0
    out = DevBatch(bt0).forward()
    assert torch.equal(out.cpu(), torch.zeros_like(out.cpu()))


def test_forward_out_of_range_ids_contribute_nothing():
    spec = ti.BatchSpec("bad ids", (ti.TableSpec(20, 16, ("fixed", 6)), ti.TableSpec(30, 32, ("fixed", 3))),
                        B=40, w_dtype=torch.float32, w_range=0.5)
    bt = ti.make_batch(spec, 2)
    idx = bt.indices.clone()
    g = torch.Generator().manual_seed(0)
    bad = torch.rand(idx.numel(), generator=g) < 0.2
    idx[bad] = torch.where(torch.rand(idx.numel(), generator=g)[bad] < 0.5,
                           torch.tensor(-3), torch.tensor(1000))
    bt.indices = idx
    db = DevBatch(bt)
    out = db.forward()
    a = host_arrays(bt)
    keep = (~bad).double().numpy()
    ids = np.where(bad.numpy(), 0, a["idx"])
    ref, ref_abs = oracle.forward(a["T"], a["B"], a["E"], a["D"], a["W"], ids, a["off"], keep)
    check_forward(out.cpu().numpy(), ref, ref_abs, True, "out-of-range ids")
