"""Seeded synthetic inputs for the table-batched embedding (TBE) path.

This module only *draws* inputs: table sizes, weights, bag lengths, indices,
per-sample weights and upstream gradients.  It holds none of the pooling,
transpose or optimizer arithmetic, so the CPU oracle and the GPU library can
both be fed from it without sharing any of the method's code.

Layout of a batch (the pages' notation: T tables, table t has E_t rows of
width D_t, B bags per table, L lookups per bag):
  * ``weights``  one flat buffer, tables concatenated in table order, each
    table row-major E_t x D_t;
  * ``offsets``  table-major, length T*B+1, bag (t, b) is entry t*B+b;
  * ``indices``  row ids local to their table, in bag order;
  * ``psw``      one fp32 weight per lookup (weighted batches only);
  * ``grad_out`` upstream gradient of the pooled output, B x sum_t D_t fp32.

Random numbers come from a counter-based SplitMix64 stream (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014): the
i-th draw of a stream is mix64(base + (i+1)*0x9E3779B97F4A7C15), so any slice
of any tensor can be drawn on any device without drawing what precedes it.
Integer arithmetic wraps modulo 2^64 on int64 tensors, so CPU and GPU draws
are bit-identical.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_CHUNK = 1 << 24  # elements drawn per step on the host, bounds temporaries
_CHUNK_GPU = 1 << 27  # on a GPU (fewer, larger launches)


def _chunk(device) -> int:
    return _CHUNK_GPU if torch.device(device).type == "cuda" else _CHUNK


def _s64(x: int) -> int:
    """Python int holding an unsigned 64-bit value -> signed int64 value."""
    x &= (1 << 64) - 1
    return x - (1 << 64) if x >= (1 << 63) else x


def _lsr(z: torch.Tensor, k: int) -> torch.Tensor:
    """Logical shift right of int64 lanes (torch's >> is arithmetic)."""
    return (z >> k) & ((1 << (64 - k)) - 1)


def _mix64(z: torch.Tensor) -> torch.Tensor:
    z = z ^ _lsr(z, 30)
    z = z * _s64(_M1)
    z = z ^ _lsr(z, 27)
    z = z * _s64(_M2)
    return z ^ _lsr(z, 31)


def _mix64_int(z: int) -> int:
    m = (1 << 64) - 1
    z &= m
    z ^= z >> 30
    z = (z * _M1) & m
    z ^= z >> 27
    z = (z * _M2) & m
    return z ^ (z >> 31)


_TAGS = {"weights": 1, "lengths": 2, "indices": 3, "psw": 4, "grad": 5,
         "scatter": 6, "sample": 7}


def stream_base(seed: int, tensor: str, table: int = 0) -> int:
    """Base state of the sub-stream for (seed, tensor kind, table)."""
    z = _mix64_int(seed * _GOLDEN + 0x5EED)
    z = _mix64_int(z ^ (_TAGS[tensor] * 0xD1B54A32D192ED03))
    return _mix64_int(z ^ ((table + 1) * 0x8CB92BA72F3D8DD7))


def draw_bits(base: int, start: int, n: int, device) -> torch.Tensor:
    """Draws start .. start+n-1 of the stream with base state ``base`` (int64)."""
    ctr = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    return _mix64(ctr * _s64(_GOLDEN) + _s64(base))


def u01(bits: torch.Tensor) -> torch.Tensor:
    """Top 53 bits as a float64 in [0, 1) (exact)."""
    return _lsr(bits, 11).to(torch.float64) * (2.0 ** -53)


def below(bits: torch.Tensor, n: int) -> torch.Tensor:
    """Integer in [0, n) from the top 32 bits (n < 2^31): floor(hi32 * n / 2^32)."""
    assert 0 < n < (1 << 31)
    return (_lsr(bits, 32) * n) >> 32


# ----------------------------------------------------------------------------
# distributions
# ----------------------------------------------------------------------------

_SIG_BITS = {torch.float32: 24, torch.float16: 11, torch.bfloat16: 8}


def dyadic_grid(a: float, dtype: torch.dtype):
    """Step 2^-s and half-width K so that k*2^-s, |k| <= K, is exact in dtype.

    U(-a, a) is drawn on the finest such grid: s is the largest integer with
    floor(a * 2^s) < 2^p (p = significand bits of dtype).
    """
    p = _SIG_BITS[dtype]
    s = 0
    while math.floor(a * 2.0 ** (s + 1)) < (1 << p):
        s += 1
    while math.floor(a * 2.0 ** s) >= (1 << p):
        s -= 1
    return s, int(math.floor(a * 2.0 ** s))


def uniform_sym(bits: torch.Tensor, a: float, dtype: torch.dtype) -> torch.Tensor:
    """U(-a, a) on the dyadic grid of ``dyadic_grid``; every value exact in dtype."""
    s, K = dyadic_grid(a, dtype)
    k = below(bits, 2 * K + 1) - K
    return (k.to(torch.float64) * (2.0 ** -s)).to(torch.float32).to(dtype)


def uniform01_f32(bits: torch.Tensor) -> torch.Tensor:
    """U(0, 1) on the grid 2^-24 (exact in fp32)."""
    return (_lsr(bits, 40).to(torch.float64) * (2.0 ** -24)).to(torch.float32)


def normal_f32(bits: torch.Tensor) -> torch.Tensor:
    """N(0, 1) by Box-Muller from one 64-bit draw (two 32-bit uniforms), in float64."""
    u1 = (_lsr(bits, 32).to(torch.float64) + 1.0) * (2.0 ** -32)   # (0, 1]
    u2 = (bits & 0xFFFFFFFF).to(torch.float64) * (2.0 ** -32)     # [0, 1)
    z = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)
    return z.to(torch.float32)


def poisson_cdf(lam: float) -> np.ndarray:
    """CDF of Poisson(lam) at k = 0, 1, ... until the tail is below 2^-60."""
    pmf = math.exp(-lam)
    cdf, acc, k = [], 0.0, 0
    while True:
        acc += pmf
        cdf.append(acc)
        k += 1
        pmf *= lam / k
        if k > lam and (1.0 - acc) < 2.0 ** -60 or k > 10 * lam + 100:
            break
    return np.asarray(cdf, dtype=np.float64)


def zipf_cdf(alpha: float, S: int) -> np.ndarray:
    """CDF over ranks 1..S of p_k proportional to k^-alpha (float64)."""
    k = np.arange(1, S + 1, dtype=np.float64)
    p = k ** (-alpha)
    c = np.cumsum(p)
    return c / c[-1]


def inverse_cdf(cdf: torch.Tensor, u: torch.Tensor) -> torch.Tensor:
    """Smallest k with cdf[k] > u (exact comparisons, device independent)."""
    k = torch.searchsorted(cdf, u, right=True)
    return torch.clamp(k, max=cdf.numel() - 1)


# ----------------------------------------------------------------------------
# batch specification
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class TableSpec:
    E: int                       # rows
    D: int                       # width
    L: tuple = ("fixed", 8)      # ("fixed", L) | ("poisson", lam, lo, hi)  (lo/hi None = no clip)
    idx: tuple = ("uniform",)    # ("uniform",) | ("zipf", alpha, S)  (S None = E)


@dataclasses.dataclass(frozen=True)
class BatchSpec:
    name: str
    tables: tuple                # of TableSpec
    B: int
    w_dtype: torch.dtype
    w_range: float               # weights ~ U(-w_range, w_range)
    itype: torch.dtype = torch.int64
    otype: torch.dtype = torch.int64
    weighted: bool = False       # per-sample weights ~ U(0, 1)
    optimizer: str = "sgd"       # "sgd" | "rowwise_adagrad"
    lr: float = 0.01
    eps: float = 1e-8
    pooling_hint: Optional[tuple] = None  # per-table expected L (plan-time hint)
    seed: int = 0                # default seed of make_batch

    @property
    def T(self) -> int:
        return len(self.tables)

    def replace(self, **kw) -> "BatchSpec":
        return dataclasses.replace(self, **kw)


def _c4_tables():
    out = []
    for t in range(16):
        E = int(round(1e5 * 40.0 ** (t / 15.0)))
        out.append(TableSpec(E=E, D=(32, 64, 128, 256)[t % 4], L=("poisson", 30.0, None, None),
                             idx=("zipf", 1.1, None)))
    return tuple(out)


WORKLOADS = {
    "tiny": BatchSpec("tiny: T=4 E=1000 D=64 fp32, B=256, L=8, SGD",
                 tuple(TableSpec(1000, 64, ("fixed", 8)) for _ in range(4)),
                 B=256, w_dtype=torch.float32, w_range=0.1, optimizer="sgd", seed=1001),
    "uniform": BatchSpec("uniform mid-size: T=26 E=1M D=128 fp16, B=65536, L~Poisson(20) in [1,100], int32",
                 tuple(TableSpec(1_000_000, 128, ("poisson", 20.0, 1, 100)) for _ in range(26)),
                 B=65536, w_dtype=torch.float16, w_range=0.05, itype=torch.int32,
                 otype=torch.int32, optimizer="rowwise_adagrad", seed=1002),
    "histogram": BatchSpec("histogram + companion: E=64 L=128 and E=100K L~Poisson(10), D=128 fp16, B=131072",
                 (TableSpec(64, 128, ("fixed", 128)),
                  TableSpec(100_000, 128, ("poisson", 10.0, None, None))),
                 B=131072, w_dtype=torch.float16, w_range=0.05, optimizer="rowwise_adagrad",
                 pooling_hint=(128, 10), seed=1003),
    "mixed": BatchSpec("mixed-width weighted: T=16 D in {32,64,128,256}, E 1e5..4e6, bf16, Zipf(1.1), B=32768",
                 _c4_tables(), B=32768, w_dtype=torch.bfloat16, w_range=0.05, weighted=True,
                 optimizer="sgd", seed=1004),
    "skewed": BatchSpec("skewed large: T=32 E=2M D=128 fp16, B=131072, L~Poisson(20), Zipf(0.91, 95000)",
                 tuple(TableSpec(2_000_000, 128, ("poisson", 20.0, None, None),
                                 ("zipf", 0.91, 95_000)) for _ in range(32)),
                 B=131072, w_dtype=torch.float16, w_range=0.05, optimizer="rowwise_adagrad",
                 seed=1005),
}


# ----------------------------------------------------------------------------
# drawing a batch
# ----------------------------------------------------------------------------

class Batch:
    """Tensors of one synthetic batch (all on one device)."""

    def __init__(self, spec: BatchSpec, seed: int):
        self.spec = spec
        self.seed = seed
        self.T = spec.T
        self.B = spec.B
        self.E: List[int] = [t.E for t in spec.tables]
        self.D: List[int] = [t.D for t in spec.tables]
        self.w_dtype = spec.w_dtype
        self.weights: torch.Tensor = None
        self.offsets: torch.Tensor = None
        self.indices: torch.Tensor = None
        self.psw: Optional[torch.Tensor] = None
        self.grad_out: torch.Tensor = None
        self.momentum: Optional[torch.Tensor] = None

    @property
    def num_indices(self) -> int:
        return int(self.indices.numel())

    def table_weights(self, t: int) -> torch.Tensor:
        """View of table t as E_t x D_t."""
        start = sum(e * d for e, d in zip(self.E[:t], self.D[:t]))
        return self.weights[start:start + self.E[t] * self.D[t]].view(self.E[t], self.D[t])


def _draw_lengths(ts: TableSpec, base: int, B: int, device) -> torch.Tensor:
    kind = ts.L[0]
    if kind == "fixed":
        return torch.full((B,), int(ts.L[1]), dtype=torch.int64, device=device)
    if kind == "poisson":
        lam, lo, hi = ts.L[1], ts.L[2], ts.L[3]
        cdf = torch.from_numpy(poisson_cdf(lam)).to(device)
        k = inverse_cdf(cdf, u01(draw_bits(base, 0, B, device)))
        if lo is not None or hi is not None:
            k = torch.clamp(k, min=lo, max=hi)
        return k
    raise ValueError(kind)


def _scatter_params(seed: int, t: int, E: int):
    """Seeded bijection rank -> row: row = (a*(k-1) + c) mod E with gcd(a, E) = 1."""
    base = stream_base(seed, "scatter", t)
    i = 0
    while True:
        a = 1 + _mix64_int(base + (i + 1) * _GOLDEN) % max(E - 1, 1)
        i += 1
        if math.gcd(a, E) == 1:
            break
    c = _mix64_int(base + (i + 1) * _GOLDEN) % E
    return a, c


def _draw_indices(ts: TableSpec, seed: int, t: int, n: int, device) -> torch.Tensor:
    base = stream_base(seed, "indices", t)
    out = torch.empty(n, dtype=torch.int64, device=device)
    kind = ts.idx[0]
    if kind == "zipf":
        alpha, S = ts.idx[1], ts.idx[2] or ts.E
        cdf = torch.from_numpy(zipf_cdf(alpha, S)).to(device)
        a, c = _scatter_params(seed, t, ts.E)
    ch = _chunk(device)
    for s in range(0, n, ch):
        m = min(ch, n - s)
        bits = draw_bits(base, s, m, device)
        if kind == "uniform":
            out[s:s + m] = below(bits, ts.E)
        elif kind == "zipf":
            k = inverse_cdf(cdf, u01(bits))          # rank - 1, in [0, S)
            out[s:s + m] = (a * k + c) % ts.E
        else:
            raise ValueError(kind)
    return out


def _fill_weights(w: torch.Tensor, base: int, a: float, dtype, device):
    n = w.numel()
    ch = _chunk(device)
    for s in range(0, n, ch):
        m = min(ch, n - s)
        w[s:s + m] = uniform_sym(draw_bits(base, s, m, device), a, dtype)


def make_batch(spec: BatchSpec, seed: Optional[int] = None, device="cpu", with_grad=True,
               with_weights=True) -> Batch:
    """Draws every tensor of ``spec`` with ``seed`` (default: the spec's own) on ``device``."""
    if seed is None:
        seed = spec.seed
    dev = torch.device(device)
    bt = Batch(spec, seed)
    T, B = spec.T, spec.B
    # weights: table t draws from its own stream, counter = element index in the table
    total = sum(ts.E * ts.D for ts in spec.tables)
    bt.weights = torch.empty(total if with_weights else 0, dtype=spec.w_dtype, device=dev)
    pos = 0
    for t, ts in enumerate(spec.tables if with_weights else ()):
        _fill_weights(bt.weights[pos:pos + ts.E * ts.D], stream_base(seed, "weights", t),
                      spec.w_range, spec.w_dtype, dev)
        pos += ts.E * ts.D
    # bag lengths, table-major
    lengths = torch.cat([_draw_lengths(ts, stream_base(seed, "lengths", t), B, dev)
                         for t, ts in enumerate(spec.tables)]) if T > 0 else \
        torch.zeros(0, dtype=torch.int64, device=dev)
    offsets = torch.zeros(T * B + 1, dtype=torch.int64, device=dev)
    if T * B:
        offsets[1:] = torch.cumsum(lengths, 0)
    N = int(offsets[-1].item())
    idx = torch.empty(N, dtype=torch.int64, device=dev)
    for t, ts in enumerate(spec.tables):
        s, e = int(offsets[t * B].item()), int(offsets[(t + 1) * B].item())
        idx[s:e] = _draw_indices(ts, seed, t, e - s, dev)
    bt.indices = idx.to(spec.itype)
    bt.offsets = offsets.to(spec.otype)
    if spec.weighted:
        bt.psw = torch.empty(N, dtype=torch.float32, device=dev)
        base = stream_base(seed, "psw")
        for s in range(0, N, _chunk(dev)):
            m = min(_chunk(dev), N - s)
            bt.psw[s:s + m] = uniform01_f32(draw_bits(base, s, m, dev))
    if with_grad:
        W = sum(spec_t.D for spec_t in spec.tables)
        g = torch.empty(B * W, dtype=torch.float32, device=dev)
        base = stream_base(seed, "grad")
        for s in range(0, B * W, _chunk(dev)):
            m = min(_chunk(dev), B * W - s)
            g[s:s + m] = normal_f32(draw_bits(base, s, m, dev))
        bt.grad_out = g.view(B, W)
    if spec.optimizer == "rowwise_adagrad":
        bt.momentum = torch.zeros(sum(ts.E for ts in spec.tables), dtype=torch.float32, device=dev)
    return bt


def scaled(spec: BatchSpec, B: int = None, E_div: int = 1, T: int = None,
           name_suffix: str = " (scaled)") -> BatchSpec:
    """Same recipe at a smaller size: fewer bags, fewer tables, E (and Zipf support) / E_div."""
    tables = spec.tables if T is None else tuple(spec.tables[i % spec.T] for i in range(T))
    new = []
    for ts in tables:
        E = max(1, ts.E // E_div)
        idx = ts.idx
        if idx[0] == "zipf" and idx[2] is not None:
            idx = ("zipf", idx[1], max(1, min(E, idx[2] // E_div)))
        new.append(TableSpec(E, ts.D, ts.L, idx))
    hint = spec.pooling_hint
    if hint is not None and T is not None:
        hint = tuple(hint[i % len(hint)] for i in range(T))
    return spec.replace(name=spec.name + name_suffix, tables=tuple(new),
                        B=spec.B if B is None else B, pooling_hint=hint)
