"""The OpenMP driver of the oracle gives the single-threaded oracle's bits (no GPU).

The driver runs the oracle's own functions over units the association order makes independent
(aligned sum chunks, destinations, scan tiles); these tests compare it with the plain oracle
bit for bit on rounding-sensitive data, at sizes that span several chunks, tiles, anchor
intervals and super-intervals, in every scan mode."""
import numpy as np
import pytest

import oracle
from conftest import bits_equal


def rounding(n, dtype, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 4, n)).astype(dtype)


def offsets(n, mean, seed):
    rng = np.random.default_rng(seed)
    cuts = np.concatenate([[0], np.cumsum(rng.geometric(1.0 / mean, size=n // mean + 8))])
    o = np.concatenate([cuts[cuts < n], [n]]).astype(np.int64)
    return np.sort(np.concatenate([o, o[1:-1:5]]))   # some empty segments


def test_threads():
    assert oracle.par_threads() >= 1


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("n", [0, 1, 1000, (1 << 20), (1 << 20) + 1, 3 * (1 << 20) + 7])
def test_par_sum(dtype, n):
    x = rounding(n, dtype, n + 3)
    assert bits_equal(np.asarray(oracle.par_det_sum(x)), np.asarray(oracle.det_sum(x)))


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("n,B,d", [(100003, 1000, 1), (50000, 3, 1), (4000, 64, 5),
                                   (200000, 65536, 1), (7, 1, 1)])
def test_par_scatter(dtype, n, B, d):
    rng = np.random.default_rng(n + B)
    v = rounding((n, d) if d > 1 else n, dtype, n)
    idx = rng.integers(-2, B + 2, n).astype(np.int32)
    o = rounding((B, d) if d > 1 else B, dtype, B)
    got, k = oracle.par_scatter_add(v, idx, o)
    want, _, wk = oracle.scatter_add(v, idx, o)
    assert bits_equal(got, want) and k == wk


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("excl", [False, True])
@pytest.mark.parametrize("rev", [False, True])
@pytest.mark.parametrize("seg", [False, True])
def test_par_scan_spec_constants(dtype, excl, rev, seg):
    n = 3 * 8192 * 256 + 12345          # four anchor intervals, a ragged last tile
    x = rounding(n, dtype, 7)
    offs = offsets(n, 100, 8) if seg else None
    got = oracle.par_scan(x, excl, rev, offs)
    want = oracle.scan(x, excl, rev, offs)
    assert bits_equal(got, want)


@pytest.mark.parametrize("excl", [False, True])
@pytest.mark.parametrize("rev", [False, True])
def test_par_scan_small_constants(excl, rev):
    # V=2, W=4, NW=2, A=3, A2=2: many tiles, intervals and super-intervals at small n
    n = 5003
    x = rounding(n, np.float32, 11)
    offs = offsets(n, 13, 12)
    for o in (None, offs):
        got = oracle.par_scan(x, excl, rev, o, V=2, W=4, NW=2, A=3, A2=2)
        want = oracle.scan(x, excl, rev, o, V=2, W=4, NW=2, A=3, A2=2)
        assert bits_equal(got, want)
