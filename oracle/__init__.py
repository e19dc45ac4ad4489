"""ctypes wrapper of the plain C oracle (``tbe_oracle.c``).

TEST INFRASTRUCTURE ONLY: only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the GPU library and never imports it.

Every function takes and returns numpy arrays; floating-point inputs are
widened to float64 (exact for fp32 / fp16 / bf16 values) before the C code
sees them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tbe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_tbe.so")

F32, F16, BF16 = 0, 1, 2
SGD, ROWWISE_ADAGRAD = 0, 1


def build(force: bool = True) -> str:
    """Compiles the oracle with the host C compiler (plain -O2, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.oracle_forward.argtypes = [i64, i64, p, p, p, p, p, p, p, p]
        L.oracle_forward.restype = ctypes.c_int
        L.oracle_transpose.argtypes = [i64, i64, p, p, p, p, p, p, p, p, p]
        L.oracle_transpose.restype = i64
        L.oracle_classify.argtypes = [i64, p, p, i64, p, p, i64, i64, p, p, p]
        L.oracle_classify.restype = i64
        L.oracle_backward.argtypes = [i64, i64, p, p, ctypes.c_int, p, p, p, p, p, ctypes.c_int,
                                      ctypes.c_double, ctypes.c_double, p, p, p, p, p, p, p, p]
        L.oracle_backward.restype = i64
        L.oracle_bounds_check.argtypes = [i64, i64, p, p, i64, p, p]
        L.oracle_bounds_check.restype = None
        L.oracle_round_array.argtypes = [ctypes.c_int, p, i64, p]
        L.oracle_round_array.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.int64)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def round_bits(dtype: int, x) -> np.ndarray:
    """Bits of float64 values rounded (nearest, ties even) to fp32/fp16/bf16, as uint32."""
    x = _f64(x).ravel()
    out = np.empty(x.size, dtype=np.uint32)
    lib().oracle_round_array(dtype, _p(x), x.size, _p(out))
    return out


def forward(T, B, E, D, W, indices, offsets, psw=None):
    """Pooled sums (float64, B x sum D) and the sums of |terms| beside them."""
    E, D = _i64(E), _i64(D)
    W, idx, off = _f64(W).ravel(), _i64(indices), _i64(offsets)
    pw = None if psw is None else _f64(psw)
    width = int(D.sum())
    out = np.empty((B, width), dtype=np.float64)
    oab = np.empty((B, width), dtype=np.float64)
    rc = lib().oracle_forward(T, B, _p(E), _p(D), _p(W), _p(idx), _p(off), _p(pw), _p(out), _p(oab))
    if rc != 0:
        raise ValueError(f"oracle_forward: invalid input ({rc})")
    return out, oab


def transpose(T, B, E, indices, offsets):
    """Stable sort of lookups by linearized key and its runs (all int64 arrays)."""
    E, idx, off = _i64(E), _i64(indices), _i64(offsets)
    N = idx.size
    a = {k: np.empty(N, dtype=np.int64) for k in
         ("sorted_key", "sorted_pos", "sorted_bag", "run_key", "run_start", "run_len")}
    n = lib().oracle_transpose(T, B, _p(E), _p(idx), _p(off), _p(a["sorted_key"]),
                               _p(a["sorted_pos"]), _p(a["sorted_bag"]), _p(a["run_key"]),
                               _p(a["run_start"]), _p(a["run_len"]))
    if n < 0:
        raise ValueError(f"oracle_transpose: invalid input ({n})")
    for k in ("run_key", "run_start", "run_len"):
        a[k] = a[k][:n]
    a["num_runs"] = int(n)
    return a


def classify(T, E, D, run_key, run_len, threshold=256, chunk=256):
    """Long/short routing, D-bucket of each short run and chunks of each long run."""
    E, D, rk, rl = _i64(E), _i64(D), _i64(run_key), _i64(run_len)
    n = rk.size
    is_long = np.empty(n, dtype=np.int8)
    bucket = np.empty(n, dtype=np.int64)
    nch = np.empty(n, dtype=np.int64)
    total = lib().oracle_classify(T, _p(E), _p(D), n, _p(rk), _p(rl), threshold, chunk,
                                  _p(is_long), _p(bucket), _p(nch))
    return dict(is_long=is_long.astype(bool), bucket=bucket, nchunks=nch, num_chunks=int(total))


def backward(T, B, E, D, w_dtype, W, indices, offsets, psw, grad_out, optimizer, lr, eps=0.0,
             momentum=None):
    """Summed row gradients and one optimizer step per touched row (float64)."""
    E, D = _i64(E), _i64(D)
    W, idx, off = _f64(W).ravel(), _i64(indices), _i64(offsets)
    pw = None if psw is None else _f64(psw)
    go = _f64(grad_out).ravel()
    mom = None if momentum is None else _f64(momentum)
    elems = int((E * D).sum())
    rows = int(E.sum())
    out = dict(g=np.empty(elems), g_abs=np.empty(elems), w_new=np.empty(elems),
               w_bits=np.empty(elems, dtype=np.uint32), m_new=np.empty(rows),
               m_f32=np.empty(rows, dtype=np.float32), touched=np.empty(rows, dtype=np.int8))
    n = lib().oracle_backward(T, B, _p(E), _p(D), w_dtype, _p(W), _p(idx), _p(off), _p(pw),
                              _p(go), optimizer, float(lr), float(eps), _p(mom),
                              _p(out["g"]), _p(out["g_abs"]), _p(out["w_new"]), _p(out["w_bits"]),
                              _p(out["m_new"]), _p(out["m_f32"]), _p(out["touched"]))
    if n < 0:
        raise ValueError(f"oracle_backward: invalid input ({n})")
    out["touched"] = out["touched"].astype(bool)
    out["num_runs"] = int(n)
    return out


def bounds_check(T, B, E, indices, offsets):
    """Repaired copies of (indices, offsets) and counts [bad indices, changed offsets]."""
    E = _i64(E)
    idx, off = _i64(indices).copy(), _i64(offsets).copy()
    counts = np.zeros(2, dtype=np.int64)
    lib().oracle_bounds_check(T, B, _p(E), _p(idx), idx.size, _p(off), _p(counts))
    return idx, off, counts


def f32_literal(x: float) -> float:
    """The exact value of an fp32 literal, as a Python float (lr, eps)."""
    return float(np.float32(x))
