"""Python binding of libtbe.so, the MI355X (gfx950) table-batched embedding library.

Argument marshalling only: every function here turns torch tensors into device
pointers and calls the C entry point of the same name declared in
``include/tbe.h``; all computation happens in the library's HIP kernels.
PyTorch provides device memory and the current stream.  There is no fallback:
if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtbe.so")

TBE_F32, TBE_F16, TBE_BF16 = 0, 1, 2
TBE_I32, TBE_I64 = 0, 1
NUM_BUCKETS = 9
BUCKET_D = [4 << b for b in range(NUM_BUCKETS)]  # short-run bucket widths next_pow2(D)
COUNTER_RUNS, COUNTER_LONG, COUNTER_CHUNKS, COUNTER_SHORT0 = 0, 1, 2, 3

_W_DTYPE = {torch.float32: TBE_F32, torch.float16: TBE_F16, torch.bfloat16: TBE_BF16}
_I_DTYPE = {torch.int32: TBE_I32, torch.int64: TBE_I64}


class TbeError(RuntimeError):
    """A libtbe call returned an error status."""


class tbe_tables(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("B", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
                ("max_D", ctypes.c_int32), ("out_width", ctypes.c_int32),
                ("all_D_mult8", ctypes.c_int32), ("hist_table", ctypes.c_int32),
                ("hist_E", ctypes.c_int32), ("hist_D", ctypes.c_int32), ("hist_col", ctypes.c_int32),
                ("row_bits", ctypes.c_int32), ("hist_w_base", ctypes.c_int64),
                ("total_rows", ctypes.c_int64), ("total_elems", ctypes.c_int64),
                ("bucket_rows", ctypes.c_int64 * NUM_BUCKETS), ("meta", ctypes.c_void_p)]


class tbe_config(ctypes.Structure):
    _fields_ = [("long_threshold", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("hist_enable", ctypes.c_int32), ("fwd_unroll", ctypes.c_int32),
                ("bwd_unroll", ctypes.c_int32), ("sort_blocks", ctypes.c_int32),
                ("bag_windows", ctypes.c_int32), ("fused_long", ctypes.c_int32),
                ("pretransposed", ctypes.c_int32), ("bags_per_wave", ctypes.c_int32),
                ("bwd_streams", ctypes.c_int32), ("tiny_runs", ctypes.c_int32),
                ("dense_min", ctypes.c_int32), ("dense_presort", ctypes.c_int32),
                ("sort_by_table", ctypes.c_int32)]


class tbe_runs_view(ctypes.Structure):
    _fields_ = [("sorted_keys", ctypes.c_void_p), ("sorted_payload", ctypes.c_void_p),
                ("run_key", ctypes.c_void_p), ("run_start", ctypes.c_void_p),
                ("counters", ctypes.c_void_p), ("long_list", ctypes.c_void_p),
                ("long_table", ctypes.c_void_p), ("chunk_list", ctypes.c_void_p),
                ("short_list", ctypes.c_void_p * NUM_BUCKETS),
                ("long_capacity", ctypes.c_int64), ("chunk_capacity", ctypes.c_int64),
                ("short_capacity", ctypes.c_int64 * NUM_BUCKETS),
                ("payload_is_position", ctypes.c_int32), ("radix_passes", ctypes.c_int32),
                ("dense_rows", ctypes.c_void_p), ("dense_count", ctypes.c_void_p),
                ("sorted_by_table", ctypes.c_int32), ("reserved", ctypes.c_int32)]


# every symbol the headers in include/ declare, with its ctypes signature
_P = ctypes.c_void_p
_SIGS = {
    "tbe_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "tbe_last_error": ([], ctypes.c_char_p),
    "tbe_config_default": ([_P], None),
    "tbe_meta_entries": ([ctypes.c_int32], ctypes.c_int64),
    "tbe_tables_derive": ([ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P],
                          ctypes.c_int),
    "tbe_bounds_check_workspace_bytes": ([_P], ctypes.c_size_t),
    "tbe_bounds_check": ([_P, _P, ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int64, _P, _P,
                          ctypes.c_size_t, _P], ctypes.c_int),
    "tbe_forward": ([_P, _P, _P, ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int64, _P, _P, _P, _P],
                    ctypes.c_int),
    "tbe_forward_repair": ([_P, _P, _P, ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int64, _P, _P,
                            _P, _P, ctypes.c_size_t, _P, _P], ctypes.c_int),
    "tbe_forward_repair_noalloc": ([_P, _P, _P, ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int64,
                                    _P, _P, _P, _P, _P], ctypes.c_int),
    "tbe_forward_hoisted": ([_P, _P, _P, ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int64, _P, _P,
                             _P, _P, ctypes.c_size_t, _P, ctypes.c_size_t, _P, _P], ctypes.c_int),
    "tbe_backward_workspace_bytes": ([_P, ctypes.c_int64, ctypes.c_int32, _P], ctypes.c_size_t),
    "tbe_backward_sgd": ([_P, _P, _P, ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int64, _P, _P,
                          ctypes.c_float, _P, ctypes.c_size_t, _P, _P], ctypes.c_int),
    "tbe_backward_rowwise_adagrad": ([_P, _P, _P, _P, ctypes.c_int32, _P, ctypes.c_int32,
                                      ctypes.c_int64, _P, _P, ctypes.c_float, ctypes.c_float, _P,
                                      ctypes.c_size_t, _P, _P], ctypes.c_int),
    "tbe_transpose": ([_P, _P, ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                       _P, ctypes.c_size_t, _P, _P, _P], ctypes.c_int),
    # measurement hooks (include/tbe_measure.h)
    "tbe_profile_select": ([ctypes.c_char_p], ctypes.c_int),
    "tbe_profile_read": ([_P, _P], ctypes.c_int),
    "tbe_calibration_copy": ([_P, _P, ctypes.c_int64, _P], ctypes.c_int),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise TbeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        L = lib()
        raise TbeError(f"{what}: {L.tbe_status_string(status).decode()} "
                       f"({L.tbe_last_error().decode()})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def tbe_config_default() -> tbe_config:
    c = tbe_config()
    lib().tbe_config_default(ctypes.byref(c))
    return c


def make_config(**kw) -> tbe_config:
    """Defaults with some fields replaced, e.g. make_config(long_threshold=8, chunk=8)."""
    c = tbe_config_default()
    for k, v in kw.items():
        setattr(c, k, int(v))
    return c


class Tables:
    """tbe_tables plus the device copy of its metadata (kept alive here)."""

    def __init__(self, E: Sequence[int], D: Sequence[int], B: int, w_dtype: torch.dtype,
                 device="cuda", pooling_hint: Optional[Sequence[int]] = None):
        T = len(E)
        self.c = tbe_tables()
        n = lib().tbe_meta_entries(T)
        meta = (ctypes.c_int64 * n)()
        E_arr = (ctypes.c_int64 * T)(*[int(e) for e in E])
        D_arr = (ctypes.c_int32 * T)(*[int(d) for d in D])
        H_arr = None if pooling_hint is None else (ctypes.c_int32 * T)(*[int(h) for h in pooling_hint])
        st = lib().tbe_tables_derive(T, int(B), _W_DTYPE[w_dtype], E_arr, D_arr, H_arr, meta,
                                     ctypes.byref(self.c))
        _check(st, "tbe_tables_derive")
        self.meta_host = torch.tensor(list(meta), dtype=torch.int64)
        self.meta_dev = self.meta_host.to(device) if device is not None else None
        self.c.meta = self.meta_dev.data_ptr() if self.meta_dev is not None else None
        self.w_dtype = w_dtype
        self.E, self.D, self.B = list(E), list(D), int(B)

    @property
    def ref(self):
        return ctypes.byref(self.c)


def tbe_bounds_check_workspace_bytes(tables: Tables) -> int:
    return int(lib().tbe_bounds_check_workspace_bytes(tables.ref))


def tbe_bounds_check(tables: Tables, indices: torch.Tensor, offsets: torch.Tensor,
                     error_counts: torch.Tensor, workspace: torch.Tensor, stream=None):
    st = lib().tbe_bounds_check(tables.ref, _ptr(indices), _I_DTYPE[indices.dtype], _ptr(offsets),
                                _I_DTYPE[offsets.dtype], indices.numel(), _ptr(error_counts),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    _check(st, "tbe_bounds_check")


def tbe_forward(tables: Tables, weights: torch.Tensor, indices: torch.Tensor, offsets: torch.Tensor,
                per_sample_weights: Optional[torch.Tensor], out: torch.Tensor,
                config: Optional[tbe_config] = None, stream=None):
    st = lib().tbe_forward(tables.ref, _ptr(weights), _ptr(indices), _I_DTYPE[indices.dtype],
                           _ptr(offsets), _I_DTYPE[offsets.dtype], indices.numel(),
                           _ptr(per_sample_weights), _ptr(out),
                           None if config is None else ctypes.byref(config), _stream(stream))
    _check(st, "tbe_forward")


def tbe_forward_repair(tables: Tables, weights: torch.Tensor, indices: torch.Tensor,
                       offsets: torch.Tensor, per_sample_weights: Optional[torch.Tensor],
                       out: torch.Tensor, error_counts: torch.Tensor, workspace: torch.Tensor,
                       config: Optional[tbe_config] = None, stream=None):
    st = lib().tbe_forward_repair(tables.ref, _ptr(weights), _ptr(indices), _I_DTYPE[indices.dtype],
                                  _ptr(offsets), _I_DTYPE[offsets.dtype], indices.numel(),
                                  _ptr(per_sample_weights), _ptr(out), _ptr(error_counts),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  None if config is None else ctypes.byref(config), _stream(stream))
    _check(st, "tbe_forward_repair")


def tbe_forward_repair_noalloc(tables: Tables, weights: torch.Tensor, indices: torch.Tensor,
                               offsets: torch.Tensor, per_sample_weights: Optional[torch.Tensor],
                               out: torch.Tensor, error_counts: torch.Tensor,
                               config: Optional[tbe_config] = None, stream=None):
    st = lib().tbe_forward_repair_noalloc(tables.ref, _ptr(weights), _ptr(indices),
                                          _I_DTYPE[indices.dtype], _ptr(offsets),
                                          _I_DTYPE[offsets.dtype], indices.numel(),
                                          _ptr(per_sample_weights), _ptr(out), _ptr(error_counts),
                                          None if config is None else ctypes.byref(config),
                                          _stream(stream))
    _check(st, "tbe_forward_repair_noalloc")


def tbe_forward_hoisted(tables: Tables, weights: torch.Tensor, indices: torch.Tensor,
                        offsets: torch.Tensor, per_sample_weights: Optional[torch.Tensor],
                        out: torch.Tensor, error_counts: Optional[torch.Tensor],
                        bounds_workspace: Optional[torch.Tensor], bwd_workspace: torch.Tensor,
                        config: Optional[tbe_config] = None, stream=None):
    bws = 0 if bounds_workspace is None else bounds_workspace.numel() * bounds_workspace.element_size()
    st = lib().tbe_forward_hoisted(tables.ref, _ptr(weights), _ptr(indices), _I_DTYPE[indices.dtype],
                                   _ptr(offsets), _I_DTYPE[offsets.dtype], indices.numel(),
                                   _ptr(per_sample_weights), _ptr(out), _ptr(error_counts),
                                   _ptr(bounds_workspace), bws, _ptr(bwd_workspace),
                                   bwd_workspace.numel() * bwd_workspace.element_size(),
                                   None if config is None else ctypes.byref(config), _stream(stream))
    _check(st, "tbe_forward_hoisted")


def tbe_backward_workspace_bytes(tables: Tables, num_indices: int, weighted: bool,
                                 config: Optional[tbe_config] = None) -> int:
    return int(lib().tbe_backward_workspace_bytes(tables.ref, int(num_indices), int(bool(weighted)),
                                                  None if config is None else ctypes.byref(config)))


def tbe_backward_sgd(tables: Tables, weights: torch.Tensor, indices: torch.Tensor,
                     offsets: torch.Tensor, per_sample_weights: Optional[torch.Tensor],
                     grad_out: torch.Tensor, lr: float, workspace: torch.Tensor,
                     config: Optional[tbe_config] = None, stream=None):
    st = lib().tbe_backward_sgd(tables.ref, _ptr(weights), _ptr(indices), _I_DTYPE[indices.dtype],
                                _ptr(offsets), _I_DTYPE[offsets.dtype], indices.numel(),
                                _ptr(per_sample_weights), _ptr(grad_out), float(lr), _ptr(workspace),
                                workspace.numel() * workspace.element_size(),
                                None if config is None else ctypes.byref(config), _stream(stream))
    _check(st, "tbe_backward_sgd")


def tbe_backward_rowwise_adagrad(tables: Tables, weights: torch.Tensor, momentum: torch.Tensor,
                                 indices: torch.Tensor, offsets: torch.Tensor,
                                 per_sample_weights: Optional[torch.Tensor], grad_out: torch.Tensor,
                                 lr: float, eps: float, workspace: torch.Tensor,
                                 config: Optional[tbe_config] = None, stream=None):
    st = lib().tbe_backward_rowwise_adagrad(
        tables.ref, _ptr(weights), _ptr(momentum), _ptr(indices), _I_DTYPE[indices.dtype],
        _ptr(offsets), _I_DTYPE[offsets.dtype], indices.numel(), _ptr(per_sample_weights),
        _ptr(grad_out), float(lr), float(eps), _ptr(workspace),
        workspace.numel() * workspace.element_size(),
        None if config is None else ctypes.byref(config), _stream(stream))
    _check(st, "tbe_backward_rowwise_adagrad")


def tbe_transpose(tables: Tables, indices: torch.Tensor, offsets: torch.Tensor, weighted: bool,
                  workspace: torch.Tensor, config: Optional[tbe_config] = None,
                  stream=None) -> tbe_runs_view:
    view = tbe_runs_view()
    st = lib().tbe_transpose(tables.ref, _ptr(indices), _I_DTYPE[indices.dtype], _ptr(offsets),
                             _I_DTYPE[offsets.dtype], indices.numel(), int(bool(weighted)),
                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                             None if config is None else ctypes.byref(config), ctypes.byref(view),
                             _stream(stream))
    _check(st, "tbe_transpose")
    return view


def tbe_profile_select(kernel_name: Optional[str]):
    _check(lib().tbe_profile_select(None if kernel_name is None else kernel_name.encode()),
           "tbe_profile_select")


def tbe_profile_read():
    """(launches, total milliseconds) of the selected kernel since the last read."""
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _check(lib().tbe_profile_read(ctypes.byref(n), ctypes.byref(ms)), "tbe_profile_read")
    return int(n.value), float(ms.value)


def tbe_calibration_copy(src: torch.Tensor, dst: torch.Tensor, nbytes: int, stream=None):
    _check(lib().tbe_calibration_copy(_ptr(src), _ptr(dst), int(nbytes), _stream(stream)),
           "tbe_calibration_copy")


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A 256-byte aligned uint8 device buffer of at least nbytes (torch allocations are)."""
    t = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


def device_view(ptr: int, n: int, dtype: torch.dtype, like: torch.Tensor) -> torch.Tensor:
    """Copies n elements at a device address inside `like`'s allocation into a new tensor."""
    esize = torch.empty(0, dtype=dtype).element_size()
    base = like.data_ptr()
    off = int(ptr) - base
    if n == 0:
        return torch.empty(0, dtype=dtype, device=like.device)
    assert 0 <= off and off + n * esize <= like.numel() * like.element_size() and off % esize == 0
    flat = like.view(torch.uint8)[off:off + n * esize]
    return flat.view(dtype).clone()
