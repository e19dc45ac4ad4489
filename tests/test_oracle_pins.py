"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each test checks the oracle against something it cannot agree with by
construction: numbers the pages print, hand-worked examples, closed forms,
dense brute force with a library matmul, library routines (numpy's stable
argsort, torch's embedding_bag, numpy's float16 conversion) and invariants.
No GPU is needed.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import tbe_inputs as ti

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _np_batch(bt):
    """Host float64 / int64 views of a tbe_inputs batch (exact widening)."""
    return dict(T=bt.T, B=bt.B, E=np.array(bt.E), D=np.array(bt.D),
                W=bt.weights.double().numpy(), idx=bt.indices.long().numpy(),
                off=bt.offsets.long().numpy(),
                psw=None if bt.psw is None else bt.psw.double().numpy(),
                grad=bt.grad_out.double().numpy())


def _dense_counts(T, B, E, idx, off, psw):
    """A[t*B+b, rowbase_t + r] = sum of psw over lookups of bag (t, b) hitting row r."""
    rows = int(np.sum(E))
    A = np.zeros((T * B, rows))
    base = np.concatenate([[0], np.cumsum(E)])
    for bag in range(T * B):
        t = bag // B
        for j in range(off[bag], off[bag + 1]):
            A[bag, base[t] + idx[j]] += 1.0 if psw is None else psw[j]
    return A


def _small_spec(weighted=False, dtype=torch.float32, optimizer="sgd", B=9):
    tables = (ti.TableSpec(7, 4, ("poisson", 3.0, None, None), ("zipf", 1.2, None)),
              ti.TableSpec(5, 8, ("poisson", 2.0, None, None)),
              ti.TableSpec(11, 4, ("fixed", 3), ("zipf", 1.5, None)))
    return ti.BatchSpec("pin", tables, B=B, w_dtype=dtype, w_range=0.5, weighted=weighted,
                        optimizer=optimizer)


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

def test_worked_example_exact():
    g = _golden("worked_example.json")
    W = np.array(g["W"], dtype=np.float64)
    bags = g["bags"]
    off = np.concatenate([[0], np.cumsum([len(b) for b in bags])])
    idx = np.array([i for b in bags for i in b], dtype=np.int64)
    out, _ = oracle.forward(1, len(bags), [g["E"]], [g["D"]], W, idx, off)
    assert np.array_equal(out, np.array(g["expected"], dtype=np.float64))


@pytest.mark.parametrize("weighted", [False, True])
def test_forward_dense_brute_force(weighted):
    bt = ti.make_batch(_small_spec(weighted), seed=11)
    a = _np_batch(bt)
    out, oabs = oracle.forward(a["T"], a["B"], a["E"], a["D"], a["W"], a["idx"], a["off"], a["psw"])
    A = _dense_counts(a["T"], a["B"], a["E"], a["idx"], a["off"], a["psw"])
    # block-diagonal weight matrix: table t's rows map to output columns of table t
    rows, width = int(a["E"].sum()), int(a["D"].sum())
    Wd = np.zeros((rows, width))
    rb, cb, wb = 0, 0, 0
    for t in range(a["T"]):
        E, D = a["E"][t], a["D"][t]
        Wd[rb:rb + E, cb:cb + D] = a["W"][wb:wb + E * D].reshape(E, D)
        rb, cb, wb = rb + E, cb + D, wb + E * D
    ref = np.zeros((a["B"], width))
    for t in range(a["T"]):
        ref += A[t * a["B"]:(t + 1) * a["B"]] @ Wd
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)
    assert np.all(oabs >= np.abs(out) - 1e-15)


@pytest.mark.parametrize("weighted", [False, True])
def test_forward_matches_torch_embedding_bag(weighted):
    bt = ti.make_batch(_small_spec(weighted), seed=12)
    a = _np_batch(bt)
    out, _ = oracle.forward(a["T"], a["B"], a["E"], a["D"], a["W"], a["idx"], a["off"], a["psw"])
    cols, wb = 0, 0
    for t in range(a["T"]):
        E, D, B = a["E"][t], a["D"][t], a["B"]
        Wt = torch.from_numpy(a["W"][wb:wb + E * D].reshape(E, D))
        o = a["off"][t * B:(t + 1) * B + 1]
        ids = torch.from_numpy(a["idx"][o[0]:o[-1]])
        pw = None if a["psw"] is None else torch.from_numpy(a["psw"][o[0]:o[-1]])
        ref = torch.nn.functional.embedding_bag(ids, Wt, torch.from_numpy(o[:-1] - o[0]),
                                                mode="sum", per_sample_weights=pw,
                                                include_last_offset=False)
        np.testing.assert_allclose(out[:, cols:cols + D], ref.numpy(), rtol=0, atol=1e-13)
        cols, wb = cols + D, wb + E * D


def test_forward_special_cases():
    # one row repeated L times gives L * row exactly (fp16 values, L <= 2048)
    bt = ti.make_batch(ti.BatchSpec("rep", (ti.TableSpec(3, 8),), B=1, w_dtype=torch.float16,
                                    w_range=0.05), seed=3)
    W = bt.weights.double().numpy()
    L = 2000
    out, _ = oracle.forward(1, 2, [3], [8], W, np.full(L, 2), [0, L, L])
    assert np.array_equal(out[0], L * W[16:24])
    assert np.array_equal(out[1], np.zeros(8))          # empty bag
    # per-sample weights of exactly 1 reproduce the unweighted sum bit for bit
    b2 = ti.make_batch(_small_spec(False), seed=5)
    a = _np_batch(b2)
    o1, _ = oracle.forward(a["T"], a["B"], a["E"], a["D"], a["W"], a["idx"], a["off"])
    o2, _ = oracle.forward(a["T"], a["B"], a["E"], a["D"], a["W"], a["idx"], a["off"],
                           np.ones(a["idx"].size))
    assert np.array_equal(o1, o2)


def test_forward_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.forward(1, 1, [3], [2], np.zeros(6), [3], [0, 1])


# ---------------------------------------------------------------------------
# transpose and routing
# ---------------------------------------------------------------------------

def _tutorial_batch():
    """Regenerates the tutorial's seed-1 batch from its section-2 prose (see golden file)."""
    g = torch.Generator().manual_seed(1)
    T, E, B, D, L = 3, 50, 16, 24, 12
    torch.randn(T * E, D, generator=g)                      # weights are drawn first
    lengths = torch.randint(0, L + 1, (T * B,), generator=g)
    off = np.concatenate([[0], np.cumsum(lengths.numpy())])
    u = torch.rand(int(off[-1]), generator=g).double()
    ids = np.minimum(np.floor(-np.log1p(-u.numpy()) / 0.15), E - 1).astype(np.int64)
    return T, E, B, D, ids, off


def test_tutorial_printed_statistics():
    gold = _golden("tutorial_stats.json")
    T, E, B, D, ids, off = _tutorial_batch()
    tr = oracle.transpose(T, B, [E] * T, ids, off)
    assert ids.size == gold["lookups"]
    assert tr["num_runs"] == gold["unique_rows"]
    assert int(tr["run_len"].max()) == gold["max_run"]
    for row in gold["sweep"]:
        c = oracle.classify(T, [E] * T, [D] * T, tr["run_key"], tr["run_len"],
                            row["threshold"], row["chunk"])
        assert int((~c["is_long"]).sum()) == row["short"]
        assert int(c["is_long"].sum()) == row["long"]
        assert c["num_chunks"] == row["chunks"]


def test_transpose_matches_numpy_stable_sort():
    bt = ti.make_batch(ti.scaled(ti.WORKLOADS["skewed"], B=300, E_div=20000, T=3), seed=21)
    a = _np_batch(bt)
    tr = oracle.transpose(a["T"], a["B"], a["E"], a["idx"], a["off"])
    base = np.concatenate([[0], np.cumsum(a["E"])])
    bag = np.repeat(np.arange(a["T"] * a["B"]), np.diff(a["off"]))
    key = base[bag // a["B"]] + a["idx"]
    perm = np.argsort(key, kind="stable")
    assert np.array_equal(tr["sorted_pos"], perm)
    assert np.array_equal(tr["sorted_key"], key[perm])
    assert np.array_equal(tr["sorted_bag"], bag[perm])
    uk, ucnt = np.unique(key, return_counts=True)
    assert np.array_equal(tr["run_key"], uk)
    assert np.array_equal(tr["run_len"], ucnt)
    assert np.array_equal(tr["run_start"], np.concatenate([[0], np.cumsum(ucnt)[:-1]]))
    assert tr["run_len"].max() > 30                      # the Zipf batch really is skewed


def test_classify_buckets_and_chunks():
    # two tables of widths 24 and 64: buckets 32 and 64; runs of lengths 1, 7, 8, 17
    T, E, D = 2, [4, 4], [24, 64]
    run_key = np.array([0, 3, 4, 6])
    run_len = np.array([1, 7, 8, 17])
    c = oracle.classify(T, E, D, run_key, run_len, threshold=8, chunk=4)
    assert c["is_long"].tolist() == [False, False, True, True]
    assert c["bucket"].tolist() == [32, 32, 0, 0]
    assert c["nchunks"].tolist() == [0, 0, 2, 5]
    assert c["num_chunks"] == 7


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def _hand_batch():
    """T=1, E=3, D=4, B=3: bag0 = {row 1}, bag1 = {row 1}, bag2 = {row 2, row 2}; row 0 untouched."""
    return dict(T=1, B=3, E=[3], D=[4], idx=np.array([1, 1, 2, 2]), off=np.array([0, 1, 2, 4]),
                grad=np.array([[1.0, 2.0, 0.0, 0.0], [2.0, 2.0, 0.0, 0.0], [0.5, -1.0, 0.25, 2.0]]))


def test_sgd_hand_example():
    h = _hand_batch()
    W = np.arange(12, dtype=np.float64)
    r = oracle.backward(h["T"], h["B"], h["E"], h["D"], oracle.F32, W, h["idx"], h["off"], None,
                        h["grad"], oracle.SGD, lr=0.5)
    # row 1: g = [3, 4, 0, 0]; row 2 (hit twice by bag 2): g = [1, -2, 0.5, 4]
    exp = np.arange(12, dtype=np.float64)
    exp[4:8] -= 0.5 * np.array([3.0, 4.0, 0.0, 0.0])
    exp[8:12] -= 0.5 * np.array([1.0, -2.0, 0.5, 4.0])
    assert np.array_equal(r["w_new"], exp)
    assert r["touched"].tolist() == [False, True, True]


def test_rowwise_adagrad_hand_example():
    h = _hand_batch()
    W = np.ones(12)
    mom = np.array([5.0, 9.75, 0.0])
    r = oracle.backward(h["T"], h["B"], h["E"], h["D"], oracle.F32, W, h["idx"], h["off"], None,
                        h["grad"], oracle.ROWWISE_ADAGRAD, lr=0.5, eps=0.0, momentum=mom)
    # row 1: g = [3,4,0,0], mean(g^2) = 25/4, m' = 9.75 + 6.25 = 16, sqrt = 4 -> step 0.5*g/4
    # row 2: g = [1,-2,0.5,4], mean(g^2) = 21.25/4 = 5.3125, m' = 5.3125
    assert r["m_new"].tolist() == [5.0, 16.0, 5.3125]
    assert np.array_equal(r["w_new"][4:8], np.array([1 - 0.375, 1 - 0.5, 1.0, 1.0]))
    s = math.sqrt(5.3125)
    np.testing.assert_allclose(r["w_new"][8:12], 1 - 0.5 * np.array([1, -2, 0.5, 4]) / s,
                               rtol=1e-15)
    assert np.array_equal(r["w_new"][0:4], np.ones(4))   # untouched row and state unchanged


def test_adagrad_trap_is_caught():
    """One step on the summed gradient differs from one step per lookup (tutorial section 5);
    for SGD the two agree to rounding.  A per-lookup oracle would fail the hand example above."""
    h = _hand_batch()
    W = np.ones(12)
    one = oracle.backward(1, 3, [3], [4], oracle.F32, W, h["idx"], h["off"], None, h["grad"],
                          oracle.ROWWISE_ADAGRAD, lr=0.5, eps=0.0, momentum=np.zeros(3))
    w, m = W.copy(), np.zeros(3)
    for bag in range(3):                     # planted mistake: optimizer applied per bag
        off = np.array([0, h["off"][bag + 1] - h["off"][bag]])
        ids = h["idx"][h["off"][bag]:h["off"][bag + 1]]
        r = oracle.backward(1, 1, [3], [4], oracle.F32, w, ids, off, None, h["grad"][bag:bag + 1],
                            oracle.ROWWISE_ADAGRAD, lr=0.5, eps=0.0, momentum=m)
        w, m = r["w_new"], r["m_new"]
    assert np.abs(w - one["w_new"]).max() > 0.05
    one_sgd = oracle.backward(1, 3, [3], [4], oracle.F32, W, h["idx"], h["off"], None, h["grad"],
                              oracle.SGD, lr=0.5)
    w = W.copy()
    for bag in range(3):
        off = np.array([0, h["off"][bag + 1] - h["off"][bag]])
        ids = h["idx"][h["off"][bag]:h["off"][bag + 1]]
        w = oracle.backward(1, 1, [3], [4], oracle.F32, w, ids, off, None, h["grad"][bag:bag + 1],
                            oracle.SGD, lr=0.5)["w_new"]
    np.testing.assert_allclose(w, one_sgd["w_new"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("weighted", [False, True])
def test_backward_gradient_dense_brute_force(weighted):
    bt = ti.make_batch(_small_spec(weighted), seed=31)
    a = _np_batch(bt)
    A = _dense_counts(a["T"], a["B"], a["E"], a["idx"], a["off"], a["psw"])
    # SGD with lr = -1 on all-zero weights returns the gradient itself
    r = oracle.backward(a["T"], a["B"], a["E"], a["D"], oracle.F32, np.zeros_like(a["W"]),
                        a["idx"], a["off"], a["psw"], a["grad"], oracle.SGD, lr=-1.0)
    rb, cb, wb = 0, 0, 0
    for t in range(a["T"]):
        E, D, B = a["E"][t], a["D"][t], a["B"]
        gt = A[t * B:(t + 1) * B, rb:rb + E].T @ a["grad"][:, cb:cb + D]
        np.testing.assert_allclose(r["w_new"][wb:wb + E * D].reshape(E, D), gt, rtol=0, atol=1e-13)
        np.testing.assert_allclose(r["g"][wb:wb + E * D].reshape(E, D), gt, rtol=0, atol=1e-13)
        rb, cb, wb = rb + E, cb + D, wb + E * D


def test_backward_column_sum_invariant():
    """Per table and column: sum over rows of g = sum over bags of (sum of psw in bag) * grad."""
    bt = ti.make_batch(_small_spec(True), seed=41)
    a = _np_batch(bt)
    r = oracle.backward(a["T"], a["B"], a["E"], a["D"], oracle.F32, a["W"], a["idx"], a["off"],
                        a["psw"], a["grad"], oracle.SGD, lr=0.1)
    cb, wb = 0, 0
    for t in range(a["T"]):
        E, D, B = a["E"][t], a["D"][t], a["B"]
        bag_w = np.array([a["psw"][a["off"][t * B + b]:a["off"][t * B + b + 1]].sum()
                          for b in range(B)])
        lhs = r["g"][wb:wb + E * D].reshape(E, D).sum(axis=0)
        rhs = (bag_w[:, None] * a["grad"][:, cb:cb + D]).sum(axis=0)
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
        cb, wb = cb + D, wb + E * D


def test_backward_one_update_per_row():
    bt = ti.make_batch(_small_spec(False, torch.float16, "rowwise_adagrad"), seed=51)
    a = _np_batch(bt)
    m0 = np.linspace(0.0, 1.0, int(a["E"].sum()))
    r = oracle.backward(a["T"], a["B"], a["E"], a["D"], oracle.F16, a["W"], a["idx"], a["off"],
                        None, a["grad"], oracle.ROWWISE_ADAGRAD, lr=0.01, eps=1e-8, momentum=m0)
    tr = oracle.transpose(a["T"], a["B"], a["E"], a["idx"], a["off"])
    touched = np.zeros(m0.size, dtype=bool)
    touched[tr["run_key"]] = True
    assert np.array_equal(r["touched"], touched)
    assert np.array_equal(r["m_new"][~touched], m0[~touched])
    # a touched row's state grows by exactly one step's mean(g^2)
    rb = np.concatenate([[0], np.cumsum(a["E"])])
    wb = np.concatenate([[0], np.cumsum(a["E"] * a["D"])])
    for key in tr["run_key"]:
        t = int(np.searchsorted(rb, key, side="right") - 1)
        D = a["D"][t]
        row = key - rb[t]
        g = r["g"][wb[t] + row * D: wb[t] + (row + 1) * D]
        np.testing.assert_allclose(r["m_new"][key], m0[key] + np.sum(g * g) / D, rtol=1e-14)
    # untouched weights are unchanged bit for bit
    for t in range(a["T"]):
        E, D = a["E"][t], a["D"][t]
        tt = touched[rb[t]:rb[t] + E]
        wn = r["w_bits"][wb[t]:wb[t] + E * D].reshape(E, D)[~tt]
        w0 = bt.weights.numpy()[wb[t]:wb[t] + E * D].view(np.uint16).reshape(E, D)[~tt]
        assert np.array_equal(wn, w0.astype(np.uint32))


# ---------------------------------------------------------------------------
# rounding to storage formats
# ---------------------------------------------------------------------------

def test_round_f16_matches_numpy():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
                        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, 2 ** -24, 2 ** -25,
                         3 * 2 ** -25, 2 ** -14, 1 + 2 ** -11, 1 + 3 * 2 ** -11]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.round_bits(oracle.F16, x), ref.astype(np.uint32))


def _bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def test_round_bf16_nearest_even():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-30, 30, 5000),
                        [1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -40, -(1 + 2 ** -8),
                         2 ** -130, 3 * 2 ** -134, 0.0]])
    got = oracle.round_bits(oracle.BF16, x)
    # brute force: the two bf16 neighbours of x, pick the nearer, ties to the even code
    for xi, gi in zip(x, got):
        lo = int(torch.tensor([abs(xi)], dtype=torch.float64).float().view(torch.int32).item()) >> 16
        cands = [c for c in (lo - 1, lo, lo + 1, lo + 2) if 0 <= c < 0x7f80]
        vals = _bf16_to_f64(cands)
        d = np.abs(vals - abs(xi))
        best = min(range(len(cands)), key=lambda i: (d[i], cands[i] & 1))
        exp = cands[best] | (0x8000 if math.copysign(1.0, xi) < 0 else 0)
        assert gi == exp, (xi, hex(gi), hex(exp))
    # and agreement with torch's fp32 -> bf16 for values exact in fp32
    f = torch.from_numpy(rng.standard_normal(20000).astype(np.float32))
    ref = f.to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16).astype(np.uint32)
    assert np.array_equal(oracle.round_bits(oracle.BF16, f.double().numpy()), ref)


def test_round_f32_matches_numpy():
    x = np.random.default_rng(2).standard_normal(10000) * 1e3
    assert np.array_equal(oracle.round_bits(oracle.F32, x), x.astype(np.float32).view(np.uint32))


# ---------------------------------------------------------------------------
# bounds check
# ---------------------------------------------------------------------------

def test_bounds_check_hand_example():
    g = _golden("bounds_example.json")
    idx, off, counts = oracle.bounds_check(g["T"], g["B"], g["E"], g["indices"], g["offsets"])
    assert idx.tolist() == g["expected_indices"]
    assert off.tolist() == g["expected_offsets"]
    assert counts.tolist() == g["expected_counts"]


def test_bounds_check_valid_input_unchanged():
    bt = ti.make_batch(_small_spec(False), seed=61)
    a = _np_batch(bt)
    idx, off, counts = oracle.bounds_check(a["T"], a["B"], a["E"], a["idx"], a["off"])
    assert counts.tolist() == [0, 0]
    assert np.array_equal(idx, a["idx"]) and np.array_equal(off, a["off"])
