"""ctypes binding of libdet.so (the HIP library), with the C interface's names.

Argument marshalling only: tensors become device pointers and sizes, the workspace is a
torch uint8 tensor from the caching allocator, and the current torch stream is passed
through.  Every step of every operation runs in the library's kernels; there is no CPU or
PyTorch fallback, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdet.so")

DET_F32 = 0
DET_F64 = 1
DET_I32 = 2      # det_scan only
DET_SCAN_EXCLUSIVE = 1
DET_SCAN_REVERSE = 2

_STATUS = {
    0: "DET_SUCCESS",
    1: "DET_ERROR_INVALID_VALUE",
    2: "DET_ERROR_UNSUPPORTED",
    3: "DET_ERROR_TOO_LARGE",
    4: "DET_ERROR_WORKSPACE",
    5: "DET_ERROR_LAUNCH",
}


class DetError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_STATUS.get(status, status)}")
        self.status = status


class ScanWaitError(RuntimeError):
    """A look-back wait of det_scan gave up (its health word is set): the output is unspecified."""


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdet.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python __graft_entry__.py` "
                           "(hipcc --offload-arch=gfx950); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, sz, u, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_uint, ctypes.c_int
    L.det_sum_workspace_size.argtypes, L.det_sum_workspace_size.restype = [i64, i], sz
    L.det_sum.argtypes, L.det_sum.restype = [p, i64, i, p, p, sz, p], i
    L.det_sum_noalloc.argtypes, L.det_sum_noalloc.restype = [p, i64, i, p, p], i
    L.det_scan_workspace_size.argtypes, L.det_scan_workspace_size.restype = [i64, i, u, i64], sz
    L.det_scan.argtypes, L.det_scan.restype = [p, p, i64, i, u, p, i64, p, sz, p], i
    L.det_scatter_add_workspace_size.argtypes = [i64, i64, i64, i]
    L.det_scatter_add_workspace_size.restype = sz
    L.det_scatter_add.argtypes = [p, p, i64, i64, i, p, i64, p, p, p, sz, p]
    L.det_scatter_add.restype = i
    L.det_scatter_sub.argtypes = [p, p, i64, i64, i, p, i64, p, p, p, sz, p]
    L.det_scatter_sub.restype = i
    L.det_scatter_add_running_workspace_size.argtypes = [i64, i64, i64, i]
    L.det_scatter_add_running_workspace_size.restype = sz
    L.det_scatter_add_running.argtypes = [p, p, i64, i64, i, p, i64, p, p, p, sz, p]
    L.det_scatter_add_running.restype = i
    L.det_spec_version.argtypes, L.det_spec_version.restype = [], i
    L.det_spec_constants.argtypes = [ctypes.POINTER(i64)] * 4
    L.det_spec_constants.restype = None
    L.det_status_string.argtypes, L.det_status_string.restype = [i], ctypes.c_char_p
    L.det_scan_error.argtypes, L.det_scan_error.restype = [p, p, p], i
    L.det_debug_set_launch.argtypes, L.det_debug_set_launch.restype = [i, i], i
    L.det_debug_set_sum_chunk.argtypes, L.det_debug_set_sum_chunk.restype = [i], i
    L.det_debug_last_launch.argtypes = [ctypes.POINTER(i64)] * 3
    L.det_debug_last_launch.restype = None
    L.det_debug_set_scan_delay.argtypes, L.det_debug_set_scan_delay.restype = [u, i], i
    L.det_debug_set_scan_anchors.argtypes, L.det_debug_set_scan_anchors.restype = [i, i], i
    L.det_debug_kernel_timing.argtypes, L.det_debug_kernel_timing.restype = [i], i
    L.det_debug_kernel_report.argtypes = [ctypes.c_char_p, sz]
    L.det_debug_kernel_report.restype = sz
    _lib = L
    return L


def _dtype_code(t: torch.Tensor, allow_int: bool = False) -> int:
    if t.dtype == torch.float32:
        return DET_F32
    if t.dtype == torch.float64:
        return DET_F64
    if allow_int and t.dtype == torch.int32:
        return DET_I32
    raise TypeError(f"det supports float32 and float64{' and int32' if allow_int else ''}, "
                    f"got {t.dtype}")


def _dev_ptr(t: Optional[torch.Tensor]):
    # plain integers: ctypes passes them as void* (the argument types are declared)
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("det operates on device tensors")
    return t.data_ptr()


# the current stream's raw handle without building a torch Stream object per call (what
# torch.cuda.current_stream(device).cuda_stream returns), when this torch has the accessor
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device) -> int:
    if _raw_stream is not None:
        return _raw_stream(device.index if device.index is not None
                           else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace of {nbytes} bytes needed")
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _check(st: int, what: str):
    if st != 0:
        raise DetError(st, what)


def _flat(t: torch.Tensor) -> torch.Tensor:
    if not t.is_contiguous():
        raise ValueError("det needs contiguous tensors (views with an offset are fine)")
    return t


# ------------------------------------------------------------------ sum

@functools.lru_cache(maxsize=256)
def det_sum_workspace_size(n: int, dtype_code: int) -> int:
    return lib().det_sum_workspace_size(n, dtype_code)


def det_sum(x: torch.Tensor, out: Optional[torch.Tensor] = None,
            ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Reproducible sum of all elements of ``x``; returns a 0-d tensor (or fills ``out``)."""
    x = _flat(x)
    dt = _dtype_code(x)
    n = x.numel()
    if out is None:
        out = torch.empty((), dtype=x.dtype, device=x.device)
    dev = x.device
    w = _workspace(det_sum_workspace_size(n, dt), dev, ws)
    _check(lib().det_sum(_dev_ptr(x), n, dt, _dev_ptr(out), _dev_ptr(w), w.numel(),
                         _stream(dev)), "det_sum")
    return out


def det_sum_noalloc(x: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """det_sum through the entry point that allocates nothing (its partials live in the
    library's per-GPU array); ``out`` (one element, dtype of x) is filled and returned.  Calls
    that overlap in time on one GPU race."""
    x = _flat(x)
    dt = _dtype_code(x)
    if out.dtype != x.dtype or out.numel() != 1:
        raise ValueError("out must be one element of x's dtype")
    _check(lib().det_sum_noalloc(_dev_ptr(x), x.numel(), dt, _dev_ptr(out), _stream(x.device)),
           "det_sum_noalloc")
    return out


# ------------------------------------------------------------------ scan

@functools.lru_cache(maxsize=256)
def det_scan_workspace_size(n: int, dtype_code: int, flags: int = 0, num_segments: int = 0) -> int:
    return lib().det_scan_workspace_size(n, dtype_code, flags, num_segments)


def det_scan(x: torch.Tensor, y: Optional[torch.Tensor] = None, exclusive: bool = False,
             reverse: bool = False, offsets: Optional[torch.Tensor] = None,
             ws: Optional[torch.Tensor] = None, check: bool = False,
             health: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Reproducible prefix sum of ``x`` (1-D).  ``offsets``: int64 device tensor [S+1]
    (0 = o_0 <= ... <= o_S = n) for a segmented scan.  int32 ``x`` gives wrapping integer
    sums (the slot-allocation scan of count-scan-write).

    The library's look-back waits are bounded; one that gives up leaves ``y`` unspecified and
    sets the workspace's health word.  ``health`` (device int32, one element) receives that
    word without synchronising; ``check=True`` waits for the scan and raises ScanWaitError
    when the word is set."""
    x = _flat(x)
    dt = _dtype_code(x, allow_int=True)
    n = x.numel()
    if y is None:
        y = torch.empty_like(x)
    flags = (DET_SCAN_EXCLUSIVE if exclusive else 0) | (DET_SCAN_REVERSE if reverse else 0)
    nseg = 0
    if offsets is not None:
        if offsets.dtype != torch.int64:
            raise TypeError("offsets must be int64")
        offsets = _flat(offsets)
        nseg = offsets.numel() - 1
    dev = x.device
    w = _workspace(det_scan_workspace_size(n, dt, flags, max(nseg, 0)), dev, ws)
    _check(lib().det_scan(_dev_ptr(x), _dev_ptr(y), n, dt, flags, _dev_ptr(offsets), nseg,
                          _dev_ptr(w), w.numel(), _stream(dev)), "det_scan")
    if check or health is not None:
        h = health if health is not None else torch.empty((), dtype=torch.int32, device=x.device)
        if h.dtype != torch.int32 or h.numel() != 1:
            raise ValueError("health must be an int32 tensor with one element")
        _check(lib().det_scan_error(_dev_ptr(w), _dev_ptr(h), _stream(x.device)),
               "det_scan_error")
        if check and int(h.item()) != 0:
            raise ScanWaitError("det_scan: a look-back wait gave up; the output is unspecified")
    return y


def det_scan_error(ws: torch.Tensor) -> torch.Tensor:
    """Health word of the last scan run in workspace ``ws`` (device int32: 0 = normal)."""
    out = torch.empty((), dtype=torch.int32, device=ws.device)
    _check(lib().det_scan_error(_dev_ptr(ws), _dev_ptr(out), _stream(ws.device)), "det_scan_error")
    return out


# ------------------------------------------------------------------ scatter-add

@functools.lru_cache(maxsize=256)
def det_scatter_add_workspace_size(n: int, num_out: int, row_len: int, dtype_code: int) -> int:
    return lib().det_scatter_add_workspace_size(n, num_out, row_len, dtype_code)


@functools.lru_cache(maxsize=256)
def det_scatter_add_running_workspace_size(n: int, num_out: int, row_len: int,
                                           dtype_code: int) -> int:
    return lib().det_scatter_add_running_workspace_size(n, num_out, row_len, dtype_code)


def _scatter(entry: str, values: torch.Tensor, index: torch.Tensor, out: torch.Tensor,
             prev: Optional[torch.Tensor], n_skipped: Optional[torch.Tensor],
             ws: Optional[torch.Tensor]) -> torch.Tensor:
    values = _flat(values)
    index = _flat(index)
    out = _flat(out)
    dt = _dtype_code(values)
    if out.dtype != values.dtype:
        raise TypeError("values and out must share a dtype")
    if index.dtype != torch.int32:
        raise TypeError("index must be int32")
    n = index.numel()
    row_len = values.numel() // n if n else (out[0].numel() if out.dim() > 1 and len(out) else 1)
    if n and values.numel() != n * row_len:
        raise ValueError("values and index disagree on n")
    if row_len < 1:
        row_len = 1
    num_out = out.numel() // row_len
    if out.numel() != num_out * row_len:
        raise ValueError("out is not a whole number of rows")
    if prev is not None:
        prev = _flat(prev)
        if prev.numel() != n * row_len or prev.dtype != values.dtype:
            raise ValueError("prev must match values")
    if n_skipped is not None and (n_skipped.dtype != torch.int64 or n_skipped.numel() < 1):
        raise ValueError("n_skipped must be an int64 tensor with one element")
    size_fn = (det_scatter_add_running_workspace_size if entry == "det_scatter_add_running"
               else det_scatter_add_workspace_size)
    dev = values.device
    w = _workspace(size_fn(n, num_out, row_len, dt), dev, ws)
    _check(getattr(lib(), entry)(_dev_ptr(values), _dev_ptr(index), n, row_len, dt, _dev_ptr(out),
                                 num_out, _dev_ptr(prev), _dev_ptr(n_skipped), _dev_ptr(w),
                                 w.numel(), _stream(dev)), entry)
    return out


def det_scatter_add(values: torch.Tensor, index: torch.Tensor, out: torch.Tensor,
                    prev: Optional[torch.Tensor] = None, n_skipped: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``out[index[i]] += values[i]`` along axis 0 in the fixed order; returns ``out``.

    ``values``: [n] or [n, *row]; ``index``: int32 [n]; ``out``: [num_out] or [num_out, *row].
    ``prev`` (same shape as values) receives the destination rows before the call;
    ``n_skipped`` (int64, one element) receives the number of out-of-range indices."""
    return _scatter("det_scatter_add", values, index, out, prev, n_skipped, ws)


def det_scatter_sub(values: torch.Tensor, index: torch.Tensor, out: torch.Tensor,
                    prev: Optional[torch.Tensor] = None, n_skipped: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``out[index[i]] -= values[i]``: the values negated, then added in the fixed order of
    det_scatter_add (arguments as there); returns ``out``."""
    return _scatter("det_scatter_sub", values, index, out, prev, n_skipped, ws)


def det_scatter_add_running(values: torch.Tensor, index: torch.Tensor, out: torch.Tensor,
                            prev: torch.Tensor, n_skipped: Optional[torch.Tensor] = None,
                            ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """det_scatter_add whose ``prev`` (required, shape of values) receives the running value:
    the destination's initial value plus the earlier contributions (ascending source index),
    summed by the exclusive segmented det_scan of the destination-grouped members; the first
    member of a destination gets the initial value itself.  Returns ``out``."""
    if prev is None:
        raise ValueError("det_scatter_add_running needs prev")
    return _scatter("det_scatter_add_running", values, index, out, prev, n_skipped, ws)


class _Gather(torch.autograd.Function):
    """``values[index]`` along axis 0; the gradient scatters back through det_scatter_add."""

    @staticmethod
    def forward(ctx, values, index):
        ctx.save_for_backward(index)
        ctx.shape = values.shape
        return values.index_select(0, index.long())

    @staticmethod
    def backward(ctx, grad_out):
        (index,) = ctx.saved_tensors
        grad = torch.zeros(ctx.shape, dtype=grad_out.dtype, device=grad_out.device)
        det_scatter_add(grad_out.contiguous(), index, grad)
        return grad, None


def gather(values: torch.Tensor, index: torch.Tensor) -> torch.Tensor:
    """Rows ``values[index[i]]`` (``index`` int32, in range).  The forward pass only moves data;
    in the backward pass the gradient rows that share a source row are accumulated by
    det_scatter_add, so the gradient's bits do not depend on scheduling (the gather case of the
    Warp guide's "Tape and Backward Passes")."""
    if index.dtype != torch.int32:
        raise TypeError("index must be int32")
    if index.numel() and (int(index.min()) < 0 or int(index.max()) >= values.shape[0]):
        raise IndexError("gather index out of range")
    return _Gather.apply(values, index)


# ------------------------------------------------------------------ introspection

def det_spec_version() -> int:
    return lib().det_spec_version()


def det_spec_constants():
    v, l_, a, a2 = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    lib().det_spec_constants(ctypes.byref(v), ctypes.byref(l_), ctypes.byref(a), ctypes.byref(a2))
    return v.value, l_.value, a.value, a2.value


def det_status_string(status: int) -> str:
    return lib().det_status_string(status).decode()


def det_debug_set_launch(grid_wgs: int = 0, extra_lds_bytes: int = 0) -> None:
    """Test hook: workgroups of the sum and look-back scan kernels (0 = default; may exceed the
    resident count) and extra dynamic LDS per workgroup (lowers occupancy)."""
    _check(lib().det_debug_set_launch(grid_wgs, extra_lds_bytes), "det_debug_set_launch")


def det_debug_set_sum_chunk(chunk_log2: int = 0) -> None:
    """Test hook: elements per partial of the sum's first level, as a power of two (0 = 14)."""
    _check(lib().det_debug_set_sum_chunk(chunk_log2), "det_debug_set_sum_chunk")


def det_debug_last_launch() -> dict:
    """Test hook: {sum_grid, scan_grid, scan_per_cu} of the library's most recent launches."""
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    lib().det_debug_last_launch(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    return {"sum_grid": a.value, "scan_grid": b.value, "scan_per_cu": c.value}


def det_debug_set_scan_delay(seed: int = 0, max_us: int = 0) -> None:
    """Test hook: seeded pauses of up to ``max_us`` microseconds before the look-back scan's
    status publications (0 = off)."""
    _check(lib().det_debug_set_scan_delay(seed & 0xFFFFFFFF, max_us), "det_debug_set_scan_delay")


def det_debug_set_scan_anchors(A: int = 0, A2: int = 0) -> None:
    """Test hook: scan anchor constants (0 = the spec's 256)."""
    _check(lib().det_debug_set_scan_anchors(A, A2), "det_debug_set_scan_anchors")


def det_debug_kernel_timing(enable: bool) -> None:
    """Test hook: bracket every library kernel launch with HIP events (drops earlier records)."""
    _check(lib().det_debug_kernel_timing(1 if enable else 0), "det_debug_kernel_timing")


def det_debug_kernel_report() -> dict:
    """Wait for the recorded launches; {kernel: (launches, total_ms, average_ms)}."""
    L = lib()
    need = L.det_debug_kernel_report(None, 0)
    buf = ctypes.create_string_buffer(need)
    L.det_debug_kernel_report(buf, need)
    rep = {}
    for line in buf.value.decode().splitlines():
        if line.startswith("#"):
            raise RuntimeError("kernel timing: " + line[1:].strip())
        name, cnt, tot, avg = line.rsplit(" ", 3)
        rep[name] = (int(cnt), float(tot), float(avg))
    return rep
