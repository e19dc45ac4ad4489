"""The seeded input generator: reproducible, counter-based, and shaped like the workloads."""
import numpy as np
import torch

import tbe_inputs as ti


def test_splitmix64_reference_value():
    # SplitMix64 seeded with 0: the first output is 0xE220A8397B1DCDAF (Steele, Lea, Flood 2014)
    got = ti.draw_bits(0, 0, 1, "cpu").item() & ((1 << 64) - 1)
    assert got == 0xE220A8397B1DCDAF


def test_slices_are_independent_of_what_precedes_them():
    base = ti.stream_base(7, "weights", 3)
    full = ti.draw_bits(base, 0, 1000, "cpu")
    part = ti.draw_bits(base, 600, 400, "cpu")
    assert torch.equal(full[600:], part)


def test_batch_is_reproducible_and_values_exact_in_dtype():
    sp = ti.scaled(ti.WORKLOADS["mixed"], B=64, E_div=1000, T=4)
    a = ti.make_batch(sp, 5)
    b = ti.make_batch(sp, 5)
    for x, y in [(a.weights, b.weights), (a.indices, b.indices), (a.offsets, b.offsets),
                 (a.psw, b.psw), (a.grad_out, b.grad_out)]:
        assert torch.equal(x, y)
    s, K = ti.dyadic_grid(0.05, torch.bfloat16)
    k = a.weights.double() * 2.0 ** s
    assert torch.equal(k, torch.round(k)) and k.abs().max() <= K
    assert a.psw.min() >= 0 and a.psw.max() < 1


def test_skewed_config_statistics_at_reduced_size():
    # C5 recipe with 1/16 of the bags and 4 tables: Poisson(20) bag sizes, Zipf-skewed rows
    sp = ti.scaled(ti.WORKLOADS["skewed"], B=8192, T=4)
    bt = ti.make_batch(sp, ti.WORKLOADS["skewed"].seed, with_grad=False, with_weights=False)
    L = np.diff(bt.offsets.numpy())
    assert abs(L.mean() - 20.0) < 0.2
    idx = bt.indices.numpy()
    off = bt.offsets.numpy()
    counts = np.bincount(idx[off[0]:off[sp.B]], minlength=sp.tables[0].E)
    assert counts.max() > 100 * max(1.0, counts[counts > 0].mean())   # a hot row exists
    assert (counts > 0).sum() <= 95_000                               # truncated support
