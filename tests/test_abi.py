"""The C-ABI library loads, exports every symbol the headers in include/ declare (tbe.h, the
computation; tbe_measure.h, the measurement hooks), its structs have the layout the binding
assumes, and host-side validation works - no GPU needed (no kernel runs)."""
import glob
import ctypes
import os
import re
import subprocess

import pytest
import torch

import bwd_tbe_fwd_amd as tbe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tbe.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions(headers=None):
    names = set()
    for h in headers or HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(tbe_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = tbe.lib()
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(tbe._SIGS), set(names) ^ set(tbe._SIGS)
    # the product header holds the computation, the measurement hooks live apart
    measure = set(declared_functions([os.path.join(ROOT, "include", "tbe_measure.h")]))
    assert measure == {"tbe_profile_select", "tbe_profile_read", "tbe_calibration_copy"}
    assert not measure & set(declared_functions([HEADER]))


def test_headers_compile_as_c(tmp_path):
    src = tmp_path / "inc.c"
    src.write_text("".join(f'#include "{h}"\n' for h in HEADERS) + "int main(void) { return 0; }\n")
    subprocess.check_call(["gcc", "-std=c11", "-Wall", "-Werror", "-o", str(tmp_path / "inc"), str(src)])


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(f"""
#include <stdio.h>
#include <stddef.h>
#include "{HEADER}"
int main(void) {{
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(tbe_tables), offsetof(tbe_tables, hist_w_base),
         offsetof(tbe_tables, bucket_rows), offsetof(tbe_tables, meta), sizeof(tbe_config),
         sizeof(tbe_runs_view), offsetof(tbe_runs_view, short_capacity),
         offsetof(tbe_runs_view, dense_count), offsetof(tbe_runs_view, sorted_by_table),
         offsetof(tbe_config, sort_by_table), offsetof(tbe_tables, row_bits));
  return 0;
}}
""")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-o", str(exe), str(src)])
    got = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    exp = [ctypes.sizeof(tbe.tbe_tables), tbe.tbe_tables.hist_w_base.offset,
           tbe.tbe_tables.bucket_rows.offset, tbe.tbe_tables.meta.offset, ctypes.sizeof(tbe.tbe_config),
           ctypes.sizeof(tbe.tbe_runs_view), tbe.tbe_runs_view.short_capacity.offset,
           tbe.tbe_runs_view.dense_count.offset, tbe.tbe_runs_view.sorted_by_table.offset,
           tbe.tbe_config.sort_by_table.offset, tbe.tbe_tables.row_bits.offset]
    assert got == exp


def test_tables_derive_host_logic():
    t = tbe.Tables([100, 64, 4_000_000, 7], [32, 128, 256, 1024], 512, torch.float16, device=None,
                   pooling_hint=[10, 128, 30, 100])
    c = t.c
    assert (c.T, c.B, c.max_D, c.out_width) == (4, 512, 1024, 32 + 128 + 256 + 1024)
    assert c.row_bits == 22  # the largest local row id, 3999999, takes 22 bits
    assert c.total_rows == 100 + 64 + 4_000_000 + 7
    assert c.total_elems == 100 * 32 + 64 * 128 + 4_000_000 * 256 + 7 * 1024
    assert c.hist_table == 1 and c.hist_E == 64 and c.hist_D == 128 and c.hist_col == 32
    assert c.hist_w_base == 100 * 32
    assert list(c.bucket_rows) == [0, 0, 0, 100, 0, 64, 4_000_000, 0, 7]
    meta = t.meta_host.view(-1, 4).tolist()
    assert meta[1] == [100, 3200, 32, 128] and meta[4] == [c.total_rows, c.total_elems, c.out_width, 0]
    # no histogram path without a pooling hint, for bf16, or with E > 64
    assert tbe.Tables([64], [128], 8, torch.float16, device=None).c.hist_table == -1
    assert tbe.Tables([64], [128], 8, torch.bfloat16, device=None, pooling_hint=[100]).c.hist_table == -1
    assert tbe.Tables([65], [128], 8, torch.float16, device=None, pooling_hint=[100]).c.hist_table == -1


def test_derive_rejects_bad_geometry():
    for E, D in [([10], [3]), ([10], [1028]), ([0], [8]), ([2 ** 31], [8])]:
        with pytest.raises(tbe.TbeError):
            tbe.Tables(E, D, 4, torch.float32, device=None)


def test_calls_validate_before_launching():
    t = tbe.Tables([10], [8], 4, torch.float32, device=None)
    L = tbe.lib()
    # meta not uploaded -> argument error, nothing launched
    st = L.tbe_forward(t.ref, None, None, 1, None, 1, 0, None, None, None, None)
    assert st == 1 and b"meta" in L.tbe_last_error()
    t.c.meta = 256  # any non-null address: the following calls must fail on the host first
    st = L.tbe_forward(t.ref, None, None, 1, ctypes.c_void_p(4096), 1, 4, None, None, None, None)
    assert st == 1 and b"indices" in L.tbe_last_error()
    st = L.tbe_backward_sgd(t.ref, ctypes.c_void_p(4096), ctypes.c_void_p(4096), 1,
                            ctypes.c_void_p(4096), 1, 4, None, ctypes.c_void_p(4096), 0.1,
                            ctypes.c_void_p(4096), 16, None, None)
    assert st == 3  # workspace too small
    assert L.tbe_status_string(3) == b"workspace missing, misaligned or too small"
    st = L.tbe_forward(t.ref, None, None, 7, ctypes.c_void_p(4096), 1, 4, None, None, None, None)
    assert st == 1 and b"index type" in L.tbe_last_error()


def test_workspace_bound_from_index_count():
    t = tbe.Tables([2_000_000] * 32, [128] * 32, 131072, torch.float16, device=None)
    n = 83_897_668
    b = tbe.tbe_backward_workspace_bytes(t, n, False)
    # sort ping-pong 16 + runs 8 + short descriptors 16 + chunk partials 4 (N/128 rows of 128
    # floats) + long lists: about 45 bytes per lookup, 3.8 GB of the 288 GB
    assert 40 * n < b < 48 * n
    assert tbe.tbe_backward_workspace_bytes(t, n, True) > b


def test_config_defaults():
    c = tbe.make_config()
    # the pages' long/short split and chunk size; histogram paths on; the optional paths off
    assert (c.long_threshold, c.chunk, c.hist_enable) == (256, 256, 1)
    assert c.bag_windows <= 1 and c.fused_long == 0 and c.sort_blocks == 0
    assert c.pretransposed == 0 and c.bags_per_wave == 0  # 0: chosen from the batch shape
    assert c.bwd_streams == 0  # 0: chosen from the tables' widths
    assert c.tiny_runs == 8    # short runs of <= 8 lookups: half the lanes per run
    assert c.dense_min == 1024  # rows of >= 1024 lookups (the 128 longest): dense counts x gradient
    assert c.dense_presort == 0  # 0: picked before the sort from 2^26 lookups on


def test_workspace_histogram_table_partials():
    """A histogram-eligible table adds its per-workgroup partials (512 x 64 x 128 floats and
    512 x 64 counts) and the forward's saved counts (B rounded up to 16, x 64 u16) to the
    unweighted workspace only."""
    E, D, B, n = [64, 1000], [128, 64], 4096, 600_000
    plain = tbe.Tables(E, D, B, torch.float16, device=None)
    hist = tbe.Tables(E, D, B, torch.float16, device=None, pooling_hint=[128, 5])
    assert plain.c.hist_table == -1 and hist.c.hist_table == 0
    extra = 512 * 64 * 128 * 4 + 512 * 64 * 4 + 4096 * 64 * 2
    d = tbe.tbe_backward_workspace_bytes(hist, n, False) - tbe.tbe_backward_workspace_bytes(plain, n, False)
    assert extra <= d < extra + 1024
    assert tbe.tbe_backward_workspace_bytes(hist, n, True) == tbe.tbe_backward_workspace_bytes(plain, n, True)


def test_lookup_count_limit():
    """At most 2^31 - 4096 lookups (32-bit positions with room for a step past the end)."""
    t = tbe.Tables([10], [8], 4, torch.float32, device=None)
    t.c.meta = 256
    L = tbe.lib()
    top = 2 ** 31 - 4096
    for n in (top + 1, 2 ** 31, -1):
        st = L.tbe_forward(t.ref, None, ctypes.c_void_p(4096), 1, ctypes.c_void_p(4096), 1, n, None,
                           None, None, None)
        assert st == 2 and b"num_indices" in L.tbe_last_error(), n
    # at the limit the same call gets past the count check (and stops at the missing weights)
    st = L.tbe_forward(t.ref, None, ctypes.c_void_p(4096), 1, ctypes.c_void_p(4096), 1, top, None,
                       None, None, None)
    assert b"num_indices" not in L.tbe_last_error()
