"""Seeded random shapes through every path at once: tables of 1 row up, widths from 4 to 520,
fixed and Poisson bag lengths, Zipf and uniform ids, every weight and index type, per-sample
weights, histogram-eligible tables, the dense rows (either pick) and the fused long-run kernel.
The backward is checked against the oracle, and the hoisted forward + backward against the
plain two calls bit for bit, with out-of-range ids (and, with repair, broken offsets)."""
import numpy as np
import pytest
import torch

import bwd_tbe_fwd_amd as tbe
import tbe_inputs as ti
from gpu_util import flush_print
from test_gpu_backward import run_and_check
from test_gpu_hoisted import _assert_same, _inject, _step

pytestmark = pytest.mark.gpu


def _random_case(rng, it, seed):
    T = int(rng.integers(1, 6))
    tables, hint = [], []
    for _ in range(T):
        E = int(rng.choice([1, 2, 64, 300, 5000, 100000]))
        D = int(rng.choice([4, 8, 16, 32, 64, 100, 128, 256, 520]))
        L = float(rng.choice([1, 5, 20, 60, 150]))
        idx = ("zipf", float(rng.choice([0.9, 1.1, 1.3])), None) if rng.random() < 0.6 else ("uniform",)
        bags = ("fixed", int(L)) if rng.random() < 0.2 else ("poisson", L, None, None)
        tables.append(ti.TableSpec(E, D, bags, idx))
        hint.append(int(L))
    spec = ti.BatchSpec(f"random {seed}.{it}", tuple(tables), B=int(rng.choice([1, 5, 64, 300, 2000])),
                        w_dtype=[torch.float32, torch.float16, torch.bfloat16][int(rng.integers(0, 3))],
                        w_range=0.05, optimizer=["sgd", "rowwise_adagrad"][int(rng.integers(0, 2))],
                        itype=[torch.int32, torch.int64][int(rng.integers(0, 2))],
                        otype=[torch.int32, torch.int64][int(rng.integers(0, 2))],
                        weighted=bool(rng.random() < 0.3),
                        pooling_hint=tuple(hint) if rng.random() < 0.5 else None)
    kw = dict(long_threshold=int(rng.choice([8, 32, 256])), chunk=int(rng.choice([8, 64, 256])),
              dense_min=int(rng.choice([0, 16, 64, 1024])), dense_presort=int(rng.choice([0, 1, -1])),
              bwd_streams=int(rng.choice([0, 1, 2])), fused_long=int(rng.random() < 0.2))
    return spec, kw, bool(rng.random() < 0.5)


@pytest.mark.parametrize("seed", [3, 4])
def test_random_shapes_every_path(seed):
    rng = np.random.default_rng(seed)
    for it in range(25):
        spec, kw, repair = _random_case(rng, it, seed)
        bt = ti.make_batch(spec, 100 * seed + it)
        what = f"{spec.name}: {bt.indices.numel()} lookups, {kw}, repair={repair}"
        flush_print(what)
        run_and_check(bt, tbe.make_config(**kw), what=what)
        idx, off = _inject(bt, it, bad_offsets=repair)
        _assert_same(_step(bt, idx, off, hoisted=False, repair=repair, cfg_kw=kw),
                     _step(bt, idx, off, hoisted=True, repair=repair, cfg_kw=kw))

