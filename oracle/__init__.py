"""CPU oracle for the reproducible add-reductions (sum, keyed scatter-add, anchored scan).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this package.  The GPU library (``scan_fixed_order_amd``) never imports,
loads or calls it; the two share no code.

The arithmetic lives in ``detref.c`` (plain C, single-threaded, one IEEE addition per
``+``); this module only builds it with gcc and marshals numpy arrays through ctypes.
Every function here follows the association order stated in ``detref.c``:

* ``pw``            -- adjacent-pair tree padded with -0.0 (course page "Floating point and
                       reproducibility", the fixed bracket over pairs).
* ``det_sum``       -- ``pw`` of the array, +0.0 when empty.
* ``scatter_add``   -- stable grouping by destination in ascending source index, ``pw`` per
                       destination and column, initial value added last (Warp "Deterministic
                       Execution", Pattern 1; ``warp.tile_atomic_add_indexed`` for rows).
* ``scatter_sub``   -- the values negated one by one, then ``scatter_add`` (Warp "Deterministic
                       Execution", Pattern 1: atomic_sub's values are negated and added in a
                       fixed order).
* ``scatter_add_running`` -- ``scatter_add`` whose ``prev`` is the destination's value after
                       the earlier contributions (in ascending source index): the initial
                       value plus the segmented exclusive ``scan`` of the destinations'
                       members laid end to end (reading R7 in ``detref.c``; the row-indexed
                       accumulate of Warp's ``warp.tile_atomic_add_indexed`` returns such
                       values, which that page calls not reproducible under repeats).
* ``scan_int32``    -- int32 prefix sums modulo 2^32 (Warp "Deterministic Execution", Pattern 2:
                       the count-scan-write prefix scan); integers need no order, so this is
                       the plain definition, written in numpy.
* ``scan``          -- tiles of V*W*NW elements, anchors every A tiles and every A*A2 tiles
                       (drjit-core pull request "Make CUDA floating-point prefix sums
                       deterministic").

``par_det_sum``, ``par_scatter_add`` and ``par_scan`` run the same C functions over
independent units (aligned sum chunks, destinations, scan tiles) on OpenMP threads
(``detref_par.c``), for the benchmark's multi-core CPU figure; the tests check that they give
the single-threaded oracle's bits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "detref.c")
_LIB_PATH = os.path.join(_HERE, "libdetref.so")
_PAR_SRC = os.path.join(_HERE, "detref_par.c")
_PAR_LIB_PATH = os.path.join(_HERE, "libdetref_par.so")

# Spec constants of the scan: V elements per lane, W lanes per wave, NW waves per tile
# (tile = V * W * NW = 8192 elements), A tiles per anchor interval, A2 intervals per
# super-interval.
SPEC_V = 32
SPEC_W = 64
SPEC_NW = 4
SPEC_A = 256
SPEC_A2 = 256

EXCLUSIVE = 1
REVERSE = 2

_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-std=c99", "-Wall"]


def _build_one(src: str, lib: str, extra) -> None:
    objs = []
    stem = os.path.splitext(os.path.basename(src))[0]
    for t, suf in (("float", "_f32"), ("double", "_f64")):
        obj = os.path.join(_HERE, f"{stem}{suf}.o")
        subprocess.check_call(["gcc", *_CFLAGS, *extra, f"-DDET_T={t}", f"-DDET_SUF={suf}", "-c",
                               src, "-o", obj])
        objs.append(obj)
    tmp = lib + ".tmp"
    subprocess.check_call(["gcc", "-shared", *extra, "-o", tmp, *objs])
    os.replace(tmp, lib)
    for o in objs:
        os.remove(o)


def build(force: bool = True) -> str:
    """Compile detref.c twice (f32, f64) with gcc and link libdetref.so; the same for the
    OpenMP driver detref_par.c (libdetref_par.so)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.exists(_PAR_LIB_PATH):
        return _LIB_PATH
    _build_one(_SRC, _LIB_PATH, [])
    _build_one(_PAR_SRC, _PAR_LIB_PATH, ["-fopenmp"])
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    for suf, ct in (("_f32", ctypes.c_float), ("_f64", ctypes.c_double)):
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        f = getattr(lib, "oref_pw" + suf)
        f.argtypes, f.restype = [p, i64], ct
        f = getattr(lib, "oref_sum" + suf)
        f.argtypes, f.restype = [p, i64], ct
        f = getattr(lib, "oref_scatter_add" + suf)
        f.argtypes, f.restype = [p, p, i64, i64, p, i64, p], i64
        f = getattr(lib, "oref_scan" + suf)
        f.argtypes = [p, p, i64, ctypes.c_uint, p, i64, i64, i64, i64, i64, i64]
        f.restype = ctypes.c_int
        f = getattr(lib, "oref_scatter_add_running" + suf)
        f.argtypes = [p, p, i64, i64, p, i64, p, i64, i64, i64, i64, i64]
        f.restype = i64
    _lib = lib
    return lib


_par = None


def _load_par():
    global _par
    if _par is not None:
        return _par
    if not os.path.exists(_PAR_LIB_PATH):
        build()
    lib = ctypes.CDLL(_PAR_LIB_PATH)
    for suf, ct in (("_f32", ctypes.c_float), ("_f64", ctypes.c_double)):
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        f = getattr(lib, "opar_sum" + suf)
        f.argtypes, f.restype = [p, i64], ct
        f = getattr(lib, "opar_scatter_add" + suf)
        f.argtypes, f.restype = [p, p, i64, i64, p, i64], i64
        f = getattr(lib, "opar_scan" + suf)
        f.argtypes = [p, p, i64, ctypes.c_uint, p, i64, i64, i64, i64, i64, i64]
        f.restype = ctypes.c_int
        getattr(lib, "opar_threads" + suf).restype = ctypes.c_int
    _par = lib
    return lib


def _suffix(dtype) -> str:
    dt = np.dtype(dtype)
    if dt == np.float32:
        return "_f32"
    if dt == np.float64:
        return "_f64"
    raise TypeError(f"oracle supports float32/float64, got {dt}")


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def pw(v: np.ndarray):
    """Pairwise tree over ``v`` (1-D float32/float64), returned as a numpy scalar."""
    v = np.ascontiguousarray(v)
    suf = _suffix(v.dtype)
    r = getattr(_load(), "oref_pw" + suf)(_ptr(v), v.size)
    return v.dtype.type(r)


def det_sum(x: np.ndarray):
    """Reproducible sum: ``pw(x)`` for n >= 1, +0.0 for an empty array."""
    x = np.ascontiguousarray(x).reshape(-1)
    suf = _suffix(x.dtype)
    r = getattr(_load(), "oref_sum" + suf)(_ptr(x), x.size)
    return x.dtype.type(r)


def scatter_add(values: np.ndarray, index: np.ndarray, out: np.ndarray,
                want_prev: bool = False) -> Tuple[np.ndarray, Optional[np.ndarray], int]:
    """Keyed scatter-add along axis 0.

    ``values`` has shape [n] or [n, d]; ``index`` int32 [n]; ``out`` shape [B] or [B, d].
    Returns ``(new_out, prev, n_skipped)``; ``out`` itself is not modified.  ``prev`` has the
    shape of ``values`` and holds the destination's value before the call for every valid
    source row (rows with an out-of-range index keep NaN there).
    """
    values = np.ascontiguousarray(values)
    index = np.ascontiguousarray(index, dtype=np.int32).reshape(-1)
    n = index.size
    row_len = 1 if values.ndim == 1 else int(np.prod(values.shape[1:]))
    if values.size != n * row_len:
        raise ValueError("values and index disagree on n")
    if out.dtype != values.dtype:
        raise TypeError("values and out must share a dtype")
    new = np.array(out, dtype=out.dtype, copy=True, order="C")
    num_out = new.size // row_len if row_len else 0
    if new.size != num_out * row_len:
        raise ValueError("out is not a whole number of rows")
    prev = np.full(values.shape, np.nan, dtype=values.dtype) if want_prev else None
    suf = _suffix(values.dtype)
    k = getattr(_load(), "oref_scatter_add" + suf)(_ptr(values), _ptr(index), n, row_len,
                                                    _ptr(new), num_out, _ptr(prev))
    if k < 0:
        raise RuntimeError(f"oracle scatter_add failed ({k})")
    return new, prev, int(k)


def scatter_add_running(values: np.ndarray, index: np.ndarray, out: np.ndarray
                        ) -> Tuple[np.ndarray, np.ndarray, int]:
    """``scatter_add`` with the running ``prev`` of reading R7: for the member at position g
    of the destination-grouped array (destination order, ascending source index inside),
    ``prev = out_init`` at its destination's first position, else ``out_init + E[g]`` with
    ``E`` the forward exclusive ``scan`` of that array (one segment per destination), per
    column.  Returns ``(new_out, prev, n_skipped)``; skipped rows keep NaN in ``prev``."""
    values = np.ascontiguousarray(values)
    index = np.ascontiguousarray(index, dtype=np.int32).reshape(-1)
    n = index.size
    row_len = 1 if values.ndim == 1 else int(np.prod(values.shape[1:]))
    if values.size != n * row_len:
        raise ValueError("values and index disagree on n")
    if out.dtype != values.dtype:
        raise TypeError("values and out must share a dtype")
    new = np.array(out, dtype=out.dtype, copy=True, order="C")
    num_out = new.size // row_len if row_len else 0
    if new.size != num_out * row_len:
        raise ValueError("out is not a whole number of rows")
    prev = np.full(values.shape, np.nan, dtype=values.dtype)
    suf = _suffix(values.dtype)
    k = getattr(_load(), "oref_scatter_add_running" + suf)(
        _ptr(values), _ptr(index), n, row_len, _ptr(new), num_out, _ptr(prev),
        SPEC_V, SPEC_W, SPEC_NW, SPEC_A, SPEC_A2)
    if k < 0:
        raise RuntimeError(f"oracle scatter_add_running failed ({k})")
    return new, prev, int(k)


def scatter_sub(values: np.ndarray, index: np.ndarray, out: np.ndarray,
                want_prev: bool = False) -> Tuple[np.ndarray, Optional[np.ndarray], int]:
    """Keyed scatter-subtract: each value negated (an exact sign flip), then ``scatter_add``.
    Not ``out - pw(M)``: when a destination's contributions cancel, the two differ in the
    sign of the zero."""
    return scatter_add(np.negative(np.ascontiguousarray(values)), index, out, want_prev)


def scan_int32(x: np.ndarray, exclusive: bool = False, reverse: bool = False,
               offsets: Optional[np.ndarray] = None) -> np.ndarray:
    """Inclusive/exclusive, forward/reverse, optionally segmented prefix sums of int32 values,
    wrapping modulo 2^32 as two's complement.  Segments restart the sum; an exclusive scan
    starts each segment at 0.  Reverse mirrors the values and the segments together."""
    x = np.ascontiguousarray(x, dtype=np.int32).reshape(-1)
    n = x.size
    offs = (np.array([0, n], np.int64) if offsets is None
            else np.ascontiguousarray(offsets, dtype=np.int64).reshape(-1))
    if reverse:
        x = x[::-1]
        offs = (n - offs[::-1]).astype(np.int64)
    y = np.empty(n, np.int64)
    for a, b in zip(offs[:-1], offs[1:]):
        if b <= a:
            continue
        run = np.cumsum(x[a:b].astype(np.int64))
        if exclusive:
            run = np.concatenate([[0], run[:-1]])
        y[a:b] = run
    out = (y & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
    return np.ascontiguousarray(out[::-1]) if reverse else out


def scan(x: np.ndarray, exclusive: bool = False, reverse: bool = False,
         offsets: Optional[np.ndarray] = None, V: int = SPEC_V, W: int = SPEC_W,
         NW: int = SPEC_NW, A: int = SPEC_A, A2: int = SPEC_A2) -> np.ndarray:
    """Anchored prefix sum; ``offsets`` (int64 [S+1], 0 = o_0 <= ... <= o_S = n) makes it
    segmented.  V, W, NW, A, A2 default to the spec constants."""
    x = np.ascontiguousarray(x).reshape(-1)
    y = np.empty_like(x)
    flags = (EXCLUSIVE if exclusive else 0) | (REVERSE if reverse else 0)
    offs = None
    nseg = 0
    if offsets is not None:
        offs = np.ascontiguousarray(offsets, dtype=np.int64).reshape(-1)
        nseg = offs.size - 1
        if nseg < 0:
            raise ValueError("offsets needs at least one entry")
    suf = _suffix(x.dtype)
    rc = getattr(_load(), "oref_scan" + suf)(_ptr(x), _ptr(y), x.size, flags, _ptr(offs), nseg,
                                             V, W, NW, A, A2)
    if rc != 0:
        raise ValueError(f"oracle scan rejected its arguments ({rc})")
    return y


# ---------------------------------------------------------------- the OpenMP driver


def par_threads() -> int:
    """Threads the OpenMP driver uses (OMP_NUM_THREADS, else the usable cores)."""
    return int(_load_par().opar_threads_f32())


def par_det_sum(x: np.ndarray):
    """``det_sum`` with aligned chunks of 2^20 elements on several threads (same bits)."""
    x = np.ascontiguousarray(x).reshape(-1)
    suf = _suffix(x.dtype)
    return x.dtype.type(getattr(_load_par(), "opar_sum" + suf)(_ptr(x), x.size))


def par_scatter_add(values: np.ndarray, index: np.ndarray, out: np.ndarray
                    ) -> Tuple[np.ndarray, int]:
    """``scatter_add`` (without prev) with the destinations on several threads (same bits).
    Returns ``(new_out, n_skipped)``."""
    values = np.ascontiguousarray(values)
    index = np.ascontiguousarray(index, dtype=np.int32).reshape(-1)
    n = index.size
    row_len = 1 if values.ndim == 1 else int(np.prod(values.shape[1:]))
    if values.size != n * row_len:
        raise ValueError("values and index disagree on n")
    if out.dtype != values.dtype:
        raise TypeError("values and out must share a dtype")
    new = np.array(out, dtype=out.dtype, copy=True, order="C")
    num_out = new.size // row_len
    suf = _suffix(values.dtype)
    k = getattr(_load_par(), "opar_scatter_add" + suf)(_ptr(values), _ptr(index), n, row_len,
                                                        _ptr(new), num_out)
    if k < 0:
        raise RuntimeError(f"oracle par_scatter_add failed ({k})")
    return new, int(k)


def par_scan(x: np.ndarray, exclusive: bool = False, reverse: bool = False,
             offsets: Optional[np.ndarray] = None, V: int = SPEC_V, W: int = SPEC_W,
             NW: int = SPEC_NW, A: int = SPEC_A, A2: int = SPEC_A2) -> np.ndarray:
    """``scan`` with the tiles' local parts and combines on several threads (same bits)."""
    x = np.ascontiguousarray(x).reshape(-1)
    y = np.empty_like(x)
    flags = (EXCLUSIVE if exclusive else 0) | (REVERSE if reverse else 0)
    offs = None
    nseg = 0
    if offsets is not None:
        offs = np.ascontiguousarray(offsets, dtype=np.int64).reshape(-1)
        nseg = offs.size - 1
        if nseg < 0:
            raise ValueError("offsets needs at least one entry")
    suf = _suffix(x.dtype)
    rc = getattr(_load_par(), "opar_scan" + suf)(_ptr(x), _ptr(y), x.size, flags, _ptr(offs),
                                                 nseg, V, W, NW, A, A2)
    if rc != 0:
        raise ValueError(f"oracle par_scan rejected its arguments ({rc})")
    return y
