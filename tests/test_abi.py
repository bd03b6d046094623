"""The C-ABI boundary, checked without a GPU.

libdet.so must load and export every function include/det.h declares; the workspace-size
functions and argument validation are host-only code and are exercised here (every call
below returns before anything is enqueued).  The spec constants the library reports must be
the ones the oracle is written for.
"""
import ctypes
import os
import re

import pytest

import oracle
from scan_fixed_order_amd import det

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "det.h")

E_INVALID, E_UNSUPPORTED, E_TOO_LARGE, E_WORKSPACE = 1, 2, 3, 4
NULL = None
FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: every call here fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(det_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert {"det_sum", "det_scan", "det_scatter_add"} <= set(names)
    lib = det.lib()
    for name in names:
        assert hasattr(lib, name), name


def test_spec_constants_match_oracle():
    V, L, A, A2 = det.det_spec_constants()
    assert V == oracle.SPEC_V and L == oracle.SPEC_W * oracle.SPEC_NW and A == oracle.SPEC_A
    assert A2 == oracle.SPEC_A2
    assert det.det_spec_version() == 1
    assert det.det_status_string(0) == "DET_SUCCESS"
    assert det.det_status_string(4) == "DET_ERROR_WORKSPACE"


def test_workspace_sizes():
    lib = det.lib()
    assert lib.det_sum_workspace_size(0, 0) >= 256
    assert lib.det_sum_workspace_size(-1, 0) == 0
    assert lib.det_sum_workspace_size(1, 7) == 0
    assert lib.det_sum_workspace_size(1 << 28, 0) >= (1 << 14) * 4
    s32 = lib.det_scan_workspace_size(1 << 28, 0, 0, 0)
    s64 = lib.det_scan_workspace_size(1 << 28, 1, 0, 0)
    assert s64 > s32 > (1 << 28) // 8192 * 8
    assert lib.det_scan_workspace_size(10, 0, 4, 0) == 0          # unknown flag bit
    w = lib.det_scatter_add_workspace_size(1 << 24, 65536, 1, 0)
    assert w >= (1 << 24) * 16                                     # two key + two value buffers
    assert lib.det_scatter_add_workspace_size(10, 10, 0, 0) == 0   # row_len < 1


def test_validation_errors_enqueue_nothing():
    lib = det.lib()
    ws = FAKE
    # sum
    assert lib.det_sum(FAKE, -1, 0, FAKE, ws, 1 << 20, NULL) == E_INVALID
    assert lib.det_sum(FAKE, 10, 9, FAKE, ws, 1 << 20, NULL) == E_UNSUPPORTED
    assert lib.det_sum(FAKE, 1 << 31, 0, FAKE, ws, 1 << 40, NULL) == E_TOO_LARGE
    assert lib.det_sum(NULL, 10, 0, FAKE, ws, 1 << 20, NULL) == E_INVALID
    assert lib.det_sum(FAKE, 10, 0, NULL, ws, 1 << 20, NULL) == E_INVALID
    assert lib.det_sum(FAKE, 1 << 20, 0, FAKE, NULL, 1 << 20, NULL) == E_WORKSPACE
    assert lib.det_sum(FAKE, 1 << 24, 0, FAKE, ws, 16, NULL) == E_WORKSPACE
    # scan
    assert lib.det_scan(FAKE, FAKE, 10, 0, 8, NULL, 0, ws, 1 << 20, NULL) == E_INVALID
    x = ctypes.c_void_p(0x100000)
    y_overlap = ctypes.c_void_p(0x100000 + 4)
    assert lib.det_scan(x, y_overlap, 10, 0, 0, NULL, 0, ws, 1 << 20, NULL) == E_INVALID
    assert lib.det_scan(x, x, 10, 0, 1, NULL, 0, ws, 1 << 20, NULL) == E_INVALID  # excl in place
    assert lib.det_scan(FAKE, ctypes.c_void_p(0x900000), 10, 0, 0, FAKE, 0, ws, 1 << 20,
                        NULL) == E_INVALID                                          # S = 0, n > 0
    assert lib.det_scan(FAKE, ctypes.c_void_p(0x900000), 1 << 20, 0, 0, NULL, 0, ws, 8,
                        NULL) == E_WORKSPACE
    assert lib.det_scan(FAKE, FAKE, 10, 3, 0, NULL, 0, ws, 1 << 20, NULL) == E_UNSUPPORTED
    # int32 is a scan type only
    assert lib.det_scan_workspace_size(1 << 20, 2, 1, 0) > 0
    assert lib.det_sum(FAKE, 10, 2, FAKE, ws, 1 << 20, NULL) == E_UNSUPPORTED
    assert lib.det_sum_workspace_size(10, 2) == 0
    assert lib.det_scatter_add_workspace_size(10, 10, 1, 2) == 0
    assert lib.det_scan_error(NULL, FAKE, NULL) == E_INVALID
    assert lib.det_scan_error(FAKE, NULL, NULL) == E_INVALID
    # scatter
    sa = lib.det_scatter_add
    assert sa(FAKE, FAKE, 10, 0, 0, ctypes.c_void_p(0x900000), 4, NULL, NULL, ws, 1 << 30,
              NULL) == E_INVALID                                                    # row_len 0
    assert sa(FAKE, FAKE, -5, 1, 0, ctypes.c_void_p(0x900000), 4, NULL, NULL, ws, 1 << 30,
              NULL) == E_INVALID
    assert sa(x, FAKE, 10, 1, 0, ctypes.c_void_p(0x100000 + 8), 4, NULL, NULL, ws, 1 << 30,
              NULL) == E_INVALID                                                    # values alias out
    assert sa(FAKE, FAKE, 1 << 31, 1, 0, ctypes.c_void_p(0x900000), 4, NULL, NULL, ws, 1 << 40,
              NULL) == E_TOO_LARGE
    assert sa(FAKE, FAKE, 1000, 1, 0, ctypes.c_void_p(0x900000), 4, NULL, NULL, ws, 64,
              NULL) == E_WORKSPACE
    assert sa(FAKE, FAKE, 10, 1, 5, ctypes.c_void_p(0x900000), 4, NULL, NULL, ws, 1 << 30,
              NULL) == E_UNSUPPORTED


def test_running_scatter_validation():
    lib = det.lib()
    ra = lib.det_scatter_add_running
    o = ctypes.c_void_p(0x900000)
    big = 1 << 30
    # the running prev needs the scatter's sort plus the grouped values and their scan
    assert lib.det_scatter_add_running_workspace_size(1 << 20, 1000, 1, 0) > \
        lib.det_scatter_add_workspace_size(1 << 20, 1000, 1, 0)
    assert lib.det_scatter_add_running_workspace_size(1 << 20, 1000, 1, 0) > (1 << 20) * (16 + 8)
    assert lib.det_scatter_add_running_workspace_size(10, 10, 0, 0) == 0
    assert lib.det_scatter_add_running_workspace_size(10, 10, 65535 * 32 + 1, 0) == 0
    assert ra(FAKE, FAKE, 10, 1, 0, o, 4, NULL, NULL, FAKE, big, NULL) == E_INVALID  # no prev
    assert ra(FAKE, FAKE, 10, 1, 0, o, 4, ctypes.c_void_p(0x900000 + 4), NULL, FAKE, big,
              NULL) == E_INVALID                                                  # prev aliases out
    assert ra(FAKE, FAKE, 10, 1, 0, o, 4, ctypes.c_void_p(0x10000 + 8), NULL, FAKE, big,
              NULL) == E_INVALID                                                  # prev aliases values
    assert ra(FAKE, FAKE, 10, 65535 * 32 + 1, 0, o, 4, ctypes.c_void_p(0xA00000), NULL, FAKE,
              big, NULL) == E_TOO_LARGE
    assert ra(FAKE, FAKE, 10, 1, 2, o, 4, ctypes.c_void_p(0xA00000), NULL, FAKE, big,
              NULL) == E_UNSUPPORTED                                              # int32
    assert ra(FAKE, FAKE, 1000, 1, 0, o, 4, ctypes.c_void_p(0xA00000), NULL, FAKE, 64,
              NULL) == E_WORKSPACE


def test_alignment_is_checked():
    lib = det.lib()
    ws_odd = ctypes.c_void_p(0x10000 + 128)        # 128-byte aligned only
    assert lib.det_sum(FAKE, 10, 0, FAKE, ws_odd, 1 << 20, NULL) == E_WORKSPACE
    assert lib.det_scan(FAKE, ctypes.c_void_p(0x900000), 10, 0, 0, NULL, 0, ws_odd, 1 << 20,
                        NULL) == E_WORKSPACE
    assert lib.det_scatter_add(FAKE, FAKE, 10, 1, 0, ctypes.c_void_p(0x900000), 4, NULL, NULL,
                               ws_odd, 1 << 30, NULL) == E_WORKSPACE
    odd = ctypes.c_void_p(0x100002)                 # not 4-byte aligned
    assert lib.det_sum(odd, 10, 0, FAKE, FAKE, 1 << 20, NULL) == E_INVALID
    assert lib.det_sum(ctypes.c_void_p(0x100004), 10, 1, FAKE, FAKE, 1 << 20, NULL) == E_INVALID
    assert lib.det_scan(odd, ctypes.c_void_p(0x900000), 10, 0, 0, NULL, 0, FAKE, 1 << 20,
                        NULL) == E_INVALID
    assert lib.det_scan(FAKE, ctypes.c_void_p(0x900000), 10, 0, 0, ctypes.c_void_p(0x200004), 1,
                        FAKE, 1 << 20, NULL) == E_INVALID                        # offsets int64
    assert lib.det_scatter_add(FAKE, odd, 10, 1, 0, ctypes.c_void_p(0x900000), 4, NULL, NULL,
                               FAKE, 1 << 30, NULL) == E_INVALID                 # index int32
    assert lib.det_scatter_add(FAKE, FAKE, 10, 1, 0, ctypes.c_void_p(0x900002), 4, NULL, NULL,
                               FAKE, 1 << 30, NULL) == E_INVALID                 # out f32


def test_debug_hook_range():
    lib = det.lib()
    assert lib.det_debug_set_launch(-1, 0) == E_INVALID
    assert lib.det_debug_set_launch(0, -1) == E_INVALID
    assert lib.det_debug_set_launch(0, 65537) == E_INVALID
    assert lib.det_debug_set_launch(5000, 65536) == 0
    assert lib.det_debug_set_launch(0, 0) == 0
    assert lib.det_debug_set_sum_chunk(13) == E_INVALID
    assert lib.det_debug_set_sum_chunk(25) == E_INVALID
    assert lib.det_debug_set_sum_chunk(24) == 0
    assert lib.det_debug_set_sum_chunk(0) == 0
    assert lib.det_debug_set_scan_delay(1, -1) == E_INVALID
    assert lib.det_debug_set_scan_delay(1, 1001) == E_INVALID
    assert lib.det_debug_set_scan_delay(0xFFFFFFFF, 1000) == 0
    assert lib.det_debug_set_scan_delay(0, 0) == 0
    last = det.det_debug_last_launch()
    assert set(last) == {"sum_grid", "scan_grid", "scan_per_cu"}
    assert lib.det_debug_set_scan_anchors(257, 0) == E_INVALID
    assert lib.det_debug_set_scan_anchors(0, -1) == E_INVALID
    assert lib.det_debug_set_scan_anchors(0, 0) == 0
    assert lib.det_debug_kernel_timing(2) == E_INVALID
    assert lib.det_debug_kernel_timing(-1) == E_INVALID
    assert lib.det_debug_kernel_timing(0) == 0
    assert det.det_debug_kernel_report() == {}          # nothing recorded: an empty report


def test_binding_rejects_cpu_tensors_and_bad_dtypes():
    import torch
    with pytest.raises(ValueError):
        det.det_sum(torch.ones(10))                 # host tensor: no CPU path exists
    with pytest.raises(TypeError):
        det.det_sum(torch.ones(10, dtype=torch.float16))
