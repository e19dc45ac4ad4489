"""The forward with the fused bounds check that allocates nothing (tbe_forward_repair_noalloc):
the same repaired indices and offsets, error counts and pooled output, bit for bit, as
tbe_forward_repair with a caller workspace.  Two calls in a row, the second on a smaller batch
(its offsets repair reads fewer block partials from the shared scratch, which still holds the
first call's), then the first batch again."""
import pytest
import torch

import bwd_tbe_fwd_amd as tbe
import tbe_inputs as ti
from gpu_util import flush_print

pytestmark = pytest.mark.gpu


def _batch(name, tables, B, w_dtype, seed, itype, otype, weighted, hint=None):
    spec = ti.BatchSpec(name, tables, B=B, w_dtype=w_dtype, w_range=0.05, itype=itype, otype=otype,
                        weighted=weighted, optimizer="sgd", pooling_hint=hint)
    bt = ti.make_batch(spec, seed, with_grad=False)
    idx, off = bt.indices.clone(), bt.offsets.clone()
    # ids outside their tables, offsets that are neither clamped nor monotone
    idx[5::97] = -3
    idx[11::89] = 2 ** 30
    nb = off.numel() - 1
    off[7] = off[9] + 5
    off[nb // 2] = -4
    off[nb // 3] = 10 ** 9
    return bt, idx, off


def _forward(fn, bt, idx, off):
    tables = tbe.Tables(bt.E, bt.D, bt.B, bt.w_dtype, pooling_hint=bt.spec.pooling_hint)
    W = bt.weights.cuda()
    psw = None if bt.psw is None else bt.psw.cuda()
    i, o = idx.cuda(), off.cuda()
    out = torch.full((bt.B, sum(bt.D)), float("nan"), device="cuda")
    cnt = torch.full((2,), -1, dtype=torch.int64, device="cuda")
    if fn == "noalloc":
        tbe.tbe_forward_repair_noalloc(tables, W, i, o, psw, out, cnt)
    else:
        ws = tbe.workspace(tbe.tbe_bounds_check_workspace_bytes(tables))
        tbe.tbe_forward_repair(tables, W, i, o, psw, out, cnt, ws)
    torch.cuda.synchronize()
    return out.cpu(), i.cpu(), o.cpu(), cnt.cpu()


def test_noalloc_forward_repair_equals_workspace_entry_point():
    big = _batch("noalloc big: 300000 bags", (ti.TableSpec(5000, 64, ("poisson", 3.0, None, None)),
                                              ti.TableSpec(64, 128, ("fixed", 70)),
                                              ti.TableSpec(200000, 32, ("poisson", 2.0, None, None),
                                                           ("zipf", 1.1, None))),
                 100_000, torch.float16, 41, torch.int64, torch.int64, False, hint=(3, 70, 2))
    small = _batch("noalloc small: 2000 bags", (ti.TableSpec(300, 128, ("poisson", 5.0, None, None)),
                                                ti.TableSpec(70, 48, ("poisson", 9.0, None, None))),
                   1000, torch.float32, 43, torch.int32, torch.int32, True)
    for bt, idx, off in (big, small, big):
        flush_print(f"noalloc: {bt.spec.name}, {idx.numel()} lookups")
        a = _forward("workspace", bt, idx, off)
        b = _forward("noalloc", bt, idx, off)
        assert a[3].tolist() == b[3].tolist() and a[3][0] > 0 and a[3][1] > 0, (a[3], b[3])
        assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
        assert torch.equal(a[0].view(torch.int32), b[0].view(torch.int32))
        assert not torch.isnan(b[0]).any()
