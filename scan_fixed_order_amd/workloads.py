"""Seeded synthetic inputs shaped like the workloads on the reference pages.

This module holds no reduction arithmetic: it only draws random inputs.  It is the one
module shared by the GPU tests, the oracle tests and the benchmark.

Recipe (numpy PCG64).  An array of n elements is drawn in fixed chunks of ``CHUNK``
elements; chunk c uses ``np.random.default_rng(np.random.SeedSequence(seed,
spawn_key=(c,)))``.  Chunks are filled by a thread pool, so the values depend only on
(seed, n, generator), never on the thread count.

* sum:      uniform [0, 1) float32 (course page "Floating point and reproducibility"
            uses one sum over a few million floats; Warp's quick start sums ones).
* scatter:  standard-normal float32 values, int32 bins uniform over ``num_bins``.
* scan:     s * z * 10**u with z ~ N(0,1), u ~ U(-4, 4), s = +-1, drawn in float64 and
            rounded to the target dtype (magnitudes spread over 8 decades, so sums round).
* segments: lengths ~ Geometric(p = 1/mean) on {1, 2, ...}, the last one cut to fit n.
* rows:     float32 [rows x row_len] standard normal, int32 row ids uniform over the
            destination rows (repeats allowed).
* mixed:    s * (1 + f) * 2**e, e uniform on {-30..30}, f ~ U[0, 1), s = +-1 (float64).
* zipf:     bins k - 1 where k follows Zipf(s) truncated to [1, num_bins], drawn by
            inverse CDF.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Optional

import numpy as np

CHUNK = 1 << 22


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _rng(seed: int, chunk: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(chunk,)))


def _fill(n: int, dtype, seed: int, draw: Callable[[np.random.Generator, int], np.ndarray],
          out: Optional[np.ndarray] = None) -> np.ndarray:
    out = np.empty(n, dtype=dtype) if out is None else out
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(c):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        out[lo:hi] = draw(_rng(seed, c), hi - lo)

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def uniform01(n: int, seed: int = 0, dtype=np.float32) -> np.ndarray:
    return _fill(n, dtype, seed, lambda g, m: g.random(m, dtype=np.dtype(dtype).type))


def normal(n: int, seed: int = 1, dtype=np.float32) -> np.ndarray:
    dt = np.dtype(dtype)
    return _fill(n, dt, seed, lambda g, m: g.standard_normal(m, dtype=dt.type))


def bins_uniform(n: int, num_bins: int, seed: int = 1) -> np.ndarray:
    # seed offset so the bins are independent of the values drawn with the same seed
    return _fill(n, np.int32, seed + 1000,
                 lambda g, m: g.integers(0, num_bins, m, dtype=np.int32))


def scan_values(n: int, dtype=np.float32, seed: int = 2) -> np.ndarray:
    def draw(g, m):
        z = g.standard_normal(m)
        u = g.uniform(-4.0, 4.0, m)
        s = np.where(g.random(m) < 0.5, -1.0, 1.0)
        return (s * z * np.power(10.0, u)).astype(dtype)

    return _fill(n, dtype, seed, draw)


def segment_offsets(n: int, mean: float = 100.0, seed: int = 3) -> np.ndarray:
    """CSR offsets [S+1] with o_0 = 0, o_S = n, lengths Geometric(1/mean), last cut."""
    g = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(1 << 20,)))
    parts = []
    total = 0
    while total < n:
        m = max(1024, int((n - total) / mean * 1.1) + 16)
        lens = g.geometric(1.0 / mean, m).astype(np.int64)
        parts.append(lens)
        total += int(lens.sum())
    lens = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    ends = np.cumsum(lens)
    cut = int(np.searchsorted(ends, n, side="left"))  # first segment reaching n
    ends = ends[: cut + 1]
    if ends.size:
        ends[-1] = n
    return np.concatenate([[0], ends]).astype(np.int64)


def rows_case(num_src: int = 1 << 16, row_len: int = 256, num_dst: int = 1 << 14,
              seed: int = 3):
    """(src [num_src, row_len] f32, rows int32 [num_src], out_init [num_dst, row_len] f32)."""
    src = normal(num_src * row_len, seed=seed + 10).reshape(num_src, row_len)
    rows = _fill(num_src, np.int32, seed + 11,
                 lambda g, m: g.integers(0, num_dst, m, dtype=np.int32))
    out = normal(num_dst * row_len, seed=seed + 12).reshape(num_dst, row_len)
    return src, rows, out


def mixed_f64(n: int, seed: int = 4) -> np.ndarray:
    def draw(g, m):
        e = g.integers(-30, 31, m)
        f = g.random(m)
        s = np.where(g.random(m) < 0.5, -1.0, 1.0)
        return s * np.ldexp(1.0 + f, e)

    return _fill(n, np.float64, seed, draw)


def zipf_bins(n: int, num_bins: int = 1 << 20, s: float = 1.1, seed: int = 4) -> np.ndarray:
    k = np.arange(1, num_bins + 1, dtype=np.float64)
    cdf = np.cumsum(k ** (-s))
    cdf /= cdf[-1]

    def draw(g, m):
        u = g.random(m)
        b = np.searchsorted(cdf, u, side="right")
        return np.minimum(b, num_bins - 1).astype(np.int32)

    return _fill(n, np.int32, seed + 1000, draw)
