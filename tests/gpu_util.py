"""Helpers shared by the GPU parity tests: device copies of seeded batches, calls
through the C ABI (the binding), oracle calls on host copies, and the tolerances.

Tolerances, from the arithmetic (fp32 unit roundoff 6e-8 times a summation depth
well under 160 stays below 1e-5 of the sum of |terms|; fp64 accumulation ends in one
rounding to fp32):
  * fp16/bf16 tables, fp32 accumulation:  |gpu - oracle| <= 1e-5 * sum|terms|
  * fp32 tables, fp64 accumulation:       |gpu - oracle| <= 1e-12 * sum|terms| + 0.5 ulp_fp32
  * updated fp16/bf16 weights:            within 1 ulp of the oracle's rounded value; only
                                          where the gradient's own bound carried through the
                                          step, 1e-5 * sum|step terms|, exceeds one ulp of the
                                          exact result (a step that cancels the weight), the
                                          weight may instead lie within that bound + 1 ulp of
                                          the exact result
  * updated fp32 weights:                 |gpu - oracle| <= 1e-5 * (|w| + |step terms|)
  * row-wise Adagrad state:               |gpu - oracle| <= 1e-5 * (m + sum_d g_abs_d^2 / D)
"""
from __future__ import annotations

import numpy as np
import torch

import bwd_tbe_fwd_amd as tbe
import oracle
import tbe_inputs as ti

ODT = {torch.float32: oracle.F32, torch.float16: oracle.F16, torch.bfloat16: oracle.BF16}


def flush_print(*a):
    print(*a, flush=True)


class DevBatch:
    """Device copies of a batch plus its tbe tables."""

    def __init__(self, bt: ti.Batch, device="cuda", pooling_hint=None):
        self.bt = bt
        hint = pooling_hint if pooling_hint is not None else bt.spec.pooling_hint
        self.tables = tbe.Tables(bt.E, bt.D, bt.B, bt.w_dtype, device=device, pooling_hint=hint)
        self.W = bt.weights.to(device)
        self.idx = bt.indices.to(device)
        self.off = bt.offsets.to(device)
        self.psw = None if bt.psw is None else bt.psw.to(device)
        self.grad = None if bt.grad_out is None else bt.grad_out.to(device)
        self.mom = None if bt.momentum is None else bt.momentum.to(device)
        self.device = device

    def forward(self, cfg=None, psw="batch"):
        bt = self.bt
        out = torch.full((bt.B, sum(bt.D)), float("nan"), dtype=torch.float32, device=self.device)
        tbe.tbe_forward(self.tables, self.W, self.idx, self.off, self.psw if psw == "batch" else psw,
                        out, cfg)
        return out

    def workspace(self, cfg=None, weighted=None):
        w = (self.psw is not None) if weighted is None else weighted
        return tbe.workspace(tbe.tbe_backward_workspace_bytes(self.tables, self.idx.numel(), w, cfg),
                             self.device)

    def backward(self, cfg=None, W=None, mom=None, lr=None, optimizer=None):
        bt = self.bt
        W = self.W if W is None else W
        optimizer = optimizer or bt.spec.optimizer
        lr = oracle.f32_literal(bt.spec.lr if lr is None else lr)
        ws = self.workspace(cfg)
        if optimizer == "sgd":
            tbe.tbe_backward_sgd(self.tables, W, self.idx, self.off, self.psw, self.grad, lr, ws, cfg)
        else:
            mom = self.mom if mom is None else mom
            tbe.tbe_backward_rowwise_adagrad(self.tables, W, mom, self.idx, self.off, self.psw,
                                             self.grad, lr, oracle.f32_literal(bt.spec.eps), ws, cfg)
        return W, mom


def host_arrays(bt: ti.Batch):
    return dict(T=bt.T, B=bt.B, E=np.array(bt.E), D=np.array(bt.D),
                W=bt.weights.double().cpu().numpy(), idx=bt.indices.long().cpu().numpy(),
                off=bt.offsets.long().cpu().numpy(),
                psw=None if bt.psw is None else bt.psw.double().cpu().numpy(),
                grad=None if bt.grad_out is None else bt.grad_out.double().cpu().numpy(),
                mom=None if bt.momentum is None else bt.momentum.double().cpu().numpy())


def ulp_f32(x):
    x = np.abs(np.asarray(x, dtype=np.float64)).astype(np.float32)
    return np.spacing(x).astype(np.float64)


def check_forward(got: np.ndarray, ref: np.ndarray, ref_abs: np.ndarray, fp64_acc: bool, what=""):
    got = np.asarray(got, dtype=np.float64)
    if fp64_acc:
        tol = 1e-12 * ref_abs + 0.5 * np.maximum(ulp_f32(ref), ulp_f32(got))
    else:
        tol = 1e-5 * ref_abs
    err = np.abs(got - ref)
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} forward elements off; first at {tuple(i)}: "
                             f"gpu {got[tuple(i)]!r} oracle {ref[tuple(i)]!r} tol {tol[tuple(i)]!r}")


def ordered16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64) & 0xFFFF
    return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)


def ordered32(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64) & 0xFFFFFFFF
    return np.where(b & 0x80000000, 0x80000000 - (b & 0x7FFFFFFF), 0x80000000 + b)


def weight_bits(W: torch.Tensor) -> np.ndarray:
    if W.dtype == torch.float32:
        return W.cpu().view(torch.int32).numpy().astype(np.int64) & 0xFFFFFFFF
    return W.cpu().view(torch.int16).numpy().astype(np.int64) & 0xFFFF


def step_bound(r: dict, E, D, lr: float, eps: float, adagrad: bool) -> np.ndarray:
    """Per weight element: sum of |terms| of its optimizer step (scale of the step's error)."""
    if not adagrad:
        return abs(lr) * r["g_abs"]
    out, pos, rpos = [], 0, 0
    for e, d in zip(E, D):
        denom = np.sqrt(r["m_new"][rpos:rpos + e]) + eps
        ga = r["g_abs"][pos:pos + e * d].reshape(e, d)
        out.append((abs(lr) * ga / np.where(denom > 0, denom, 1.0)[:, None]).ravel())
        pos += e * d
        rpos += e
    return np.concatenate(out)


def bf_or_h_ulp(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Spacing of the fp16 / bf16 grid at |x| (subnormal spacing near 0)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    if dtype == torch.float16:
        e = np.floor(np.log2(np.maximum(ax, 2.0 ** -14)))
        return 2.0 ** (e - 10)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


# fp16/bf16 weights checked so far in this process: how many, how many lay beyond 1 ulp of the
# oracle's rounded value (each of those passed only under the composed bound), and the largest
# distance in ulp
ULP_STATS = {"weights": 0, "beyond_1ulp": 0, "max_ulp": 0}


def check_weights(W_gpu: torch.Tensor, r: dict, dtype: torch.dtype, step_abs=None, what=""):
    """fp16/bf16: within 1 ulp of the oracle's rounded value, except under the one condition in
    the module docstring; fp32: 1e-5 * (|w| + |step terms|).  Prints, for fp16/bf16, how many
    weights lay beyond 1 ulp and the largest distance."""
    bits = weight_bits(W_gpu)
    if dtype == torch.float32:
        got = W_gpu.double().cpu().numpy()
        exp = r["w_new"]
        tol = 1e-5 * (np.abs(exp) + (0 if step_abs is None else step_abs))
        tol = np.maximum(tol, 0.5 * ulp_f32(exp))
        bad = ~(np.abs(got - exp) <= tol)
    else:
        d = np.abs(ordered16(bits) - ordered16(r["w_bits"]))
        bad = d > 1
        beyond = int(bad.sum())
        if beyond and step_abs is not None:
            # the composed bound: the gradient may be off by 1e-5 of its |terms| (fp32
            # accumulation), which the step carries into the weight as 1e-5 * step_abs; where
            # that exceeds one ulp of the exact result, a correctly rounded fp32 step can land
            # more than 1 ulp from the oracle's rounded value
            got = W_gpu.double().cpu().numpy()
            exp = r["w_new"]
            one_ulp = np.abs(bf_or_h_ulp(exp, dtype))
            sa = np.broadcast_to(np.asarray(step_abs, dtype=np.float64), exp.shape)
            composed = 1e-5 * sa > one_ulp
            bad &= ~(composed & (np.abs(got - exp) <= one_ulp + 1e-5 * sa))
        mx = int(d.max()) if d.size else 0
        ULP_STATS["weights"] += int(d.size)
        ULP_STATS["beyond_1ulp"] += beyond
        ULP_STATS["max_ulp"] = max(ULP_STATS["max_ulp"], mx)
        flush_print(f"{what}: {d.size} {'fp16' if dtype == torch.float16 else 'bf16'} weights, "
                    f"{beyond} beyond 1 ulp (max {mx} ulp)")
    if bad.any():
        i = int(np.argwhere(bad)[0][0])
        raise AssertionError(f"{what}: {int(bad.sum())} weights off; first at {i}: gpu bits "
                             f"{bits[i]:#x} oracle bits {int(r['w_bits'][i]):#x} "
                             f"(oracle value {r['w_new'][i]!r})")


def check_momentum(m_gpu: torch.Tensor, r: dict, D_of_row: np.ndarray, g_abs_rows: np.ndarray,
                   what=""):
    got = m_gpu.double().cpu().numpy()
    exp = r["m_new"]
    tol = 1e-5 * (np.abs(exp) + g_abs_rows / D_of_row)
    bad = ~(np.abs(got - exp) <= tol)
    if bad.any():
        i = int(np.argwhere(bad)[0][0])
        raise AssertionError(f"{what}: {int(bad.sum())} momentum entries off; first {i}: "
                             f"gpu {got[i]!r} oracle {exp[i]!r}")


def row_g_abs_sq(r: dict, E, D) -> (np.ndarray, np.ndarray):
    """Per row: sum_d g_abs_d^2 and D (for the momentum tolerance)."""
    out, dd = [], []
    pos = 0
    for e, d in zip(E, D):
        ga = r["g_abs"][pos:pos + e * d].reshape(e, d)
        out.append((ga * ga).sum(axis=1))
        dd.append(np.full(e, d, dtype=np.float64))
        pos += e * d
    return np.concatenate(out), np.concatenate(dd)


def oracle_backward(bt: ti.Batch, W=None, lr=None, optimizer=None):
    a = host_arrays(bt)
    optimizer = optimizer or bt.spec.optimizer
    lr = oracle.f32_literal(bt.spec.lr if lr is None else lr)
    opt = oracle.SGD if optimizer == "sgd" else oracle.ROWWISE_ADAGRAD
    Wd = a["W"] if W is None else W
    r = oracle.backward(a["T"], a["B"], a["E"], a["D"], ODT[bt.w_dtype], Wd, a["idx"], a["off"],
                        a["psw"], a["grad"], opt, lr, oracle.f32_literal(bt.spec.eps),
                        a["mom"] if opt == oracle.ROWWISE_ADAGRAD else None)
    r["w_old"] = Wd
    return r
