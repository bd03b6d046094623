"""Pins for the oracle's running ``prev`` of the keyed scatter-add (reading R7 of the oracle).

Warp's ``warp.tile_atomic_add_indexed`` returns the destination rows "as they were before"
the accumulate; under repeated indices the page leaves those values unspecified.  The
reading pinned here: a loop of atomic adds in ascending source index would hand member k of
a destination the initial value plus the members before it, and the sum of those members is
formed in a fixed order: the forward exclusive segmented scan of the destination-grouped
array (destinations in order, members in ascending source index, one segment each), added
to the initial value; a destination's first member gets the initial value itself.

Checks: the page's printed example (no repeats, so running and snapshot agree); a sequential
loop of adds on integer-valued data (every order is exact there, so this pins grouping,
member order, head handling, skipped indices and where each value lands); closed forms of
the scan's order inside one lane run (a left fold) and across a lane-run boundary (the lane
total, then the fold of the next run), on values where other orders round differently;
columns of a row accumulate equal scalar accumulates; ``out`` equals ``scatter_add``'s.
"""
import json
import os

import numpy as np
import pytest

import oracle

F32 = np.float32
F64 = np.float64
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def same_bits(a, b):
    return np.asarray(a).tobytes() == np.asarray(b).tobytes()


def sequential_atomics(values, index, out):
    """A loop of atomic adds in ascending source index: returns (out, prev)."""
    vals = values.reshape(index.size, -1)
    cur = np.array(out, copy=True).reshape(-1, vals.shape[1])
    prev = np.full(vals.shape, np.nan, values.dtype)
    for i, r in enumerate(index):
        if 0 <= r < cur.shape[0]:
            prev[i] = cur[r]
            cur[r] = cur[r] + vals[i]
    return cur.reshape(out.shape), prev.reshape(values.shape)


def test_worked_example_has_no_repeats_so_prev_is_the_snapshot():
    g = json.load(open(os.path.join(GOLDEN, "tile_atomic_add_indexed_example.json")))
    x = np.array(g["x"], F32)
    y, prev, skipped = oracle.scatter_add_running(x, np.array(g["rows"], np.int32),
                                                  np.array(g["y_init"], F32))
    assert np.array_equal(y, np.array(g["y_expected"], F32))
    assert np.array_equal(prev, np.array(g["previous_expected"], F32))
    assert skipped == 0


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("row_len", [1, 3])
def test_integer_data_equals_a_loop_of_atomics(dtype, row_len):
    rng = np.random.default_rng(40 + row_len)
    n, B = 20000, 37                  # 20,000 members over 37 destinations: several tiles
    index = rng.integers(-2, B + 2, n).astype(np.int32)
    shape = (n,) if row_len == 1 else (n, row_len)
    values = rng.integers(-8, 9, shape).astype(dtype)
    values[rng.random(shape) < 0.05] = -0.0
    out = rng.integers(-50, 51, (B,) if row_len == 1 else (B, row_len)).astype(dtype)
    out.reshape(-1)[::7] = -0.0       # a signed-zero initial value must come back as is
    want_out, want_prev = sequential_atomics(values, index, out)
    got_out, got_prev, k = oracle.scatter_add_running(values, index, out)
    assert k == int(np.sum((index < 0) | (index >= B)))
    assert same_bits(got_prev, want_prev)
    assert same_bits(got_out, want_out)
    assert same_bits(got_out, oracle.scatter_add(values, index, out)[0])


def spread(rng, n, dtype):
    return (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 6, n)).astype(dtype)


def half_ulp_of_one(dtype):
    return dtype(np.finfo(dtype).eps / 2)


@pytest.mark.parametrize("dtype", [F32, F64])
def test_one_lane_run_is_a_left_fold(dtype):
    # one destination whose 32 members fill grouped positions 0..31, the first lane's run:
    # the scan's lane-serial prefix is the left fold, so prev_k = init + (((v1 + v2) + ...)
    rng = np.random.default_rng(7)
    v = spread(rng, 32, dtype)
    h = half_ulp_of_one(dtype)
    v[:2] = h                         # init + (h + h) = 1 + 2h, but (1 + h) + h = 1
    init = dtype(1.0)
    _, prev, _ = oracle.scatter_add_running(v, np.zeros(32, np.int32), np.array([init], dtype))
    want = [init]
    acc = v[0]
    for k in range(1, 32):
        want.append(dtype(init + acc))
        acc = dtype(acc + v[k])
    assert same_bits(prev, np.array(want, dtype))
    # the pin discriminates: a sequential loop of adds rounds differently somewhere
    _, seq = sequential_atomics(v, np.zeros(32, np.int32), np.array([init], dtype))
    assert not same_bits(prev, seq)


@pytest.mark.parametrize("dtype", [F32, F64])
def test_across_a_lane_run_boundary(dtype):
    # destination 0 takes grouped positions 0..29, destination 1 positions 30..35: its running
    # sums combine the first lane's total (v30 + v31) with the fold of the second lane's run
    rng = np.random.default_rng(8)
    n = 36
    index = np.array([0] * 30 + [1] * 6, np.int32)
    v = spread(rng, n, dtype)
    h = half_ulp_of_one(dtype)
    v[30:34] = [1.0, 0.0, h, h]       # (v30 + v31) + (h + h) = 1 + 2h, but ((1 + h) + h) = 1
    init = np.array([dtype(0.5), dtype(-1.25)], dtype)
    _, prev, _ = oracle.scatter_add_running(v, index, init)
    a, b = init[1], v[30:]
    l0 = dtype(b[0] + b[1])
    want = [a,
            dtype(a + b[0]),
            dtype(a + l0),
            dtype(a + dtype(l0 + b[2])),
            dtype(a + dtype(l0 + dtype(b[2] + b[3]))),
            dtype(a + dtype(l0 + dtype(dtype(b[2] + b[3]) + b[4])))]
    assert same_bits(prev[30:], np.array(want, dtype))
    # a fold straight through the boundary is a different order, and rounds differently
    fold = [a, dtype(a + b[0])]
    acc = dtype(b[0] + b[1])
    for k in range(2, 6):
        fold.append(dtype(a + acc))
        acc = dtype(acc + b[k])
    assert not same_bits(np.array(want, dtype), np.array(fold, dtype))


@pytest.mark.parametrize("dtype", [F32, F64])
def test_row_columns_equal_scalar_running_scatters(dtype):
    rng = np.random.default_rng(9)
    n, B, d = 9000, 11, 4
    index = rng.integers(-1, B + 1, n).astype(np.int32)
    values = spread(rng, n * d, dtype).reshape(n, d)
    out = spread(rng, B * d, dtype).reshape(B, d)
    got_out, got_prev, _ = oracle.scatter_add_running(values, index, out)
    for c in range(d):
        o, p, _ = oracle.scatter_add_running(np.ascontiguousarray(values[:, c]), index,
                                             np.ascontiguousarray(out[:, c]))
        assert same_bits(got_out[:, c], o)
        assert same_bits(got_prev[:, c], p)


def test_no_valid_member_and_empty_input():
    v = np.ones(5, F32)
    o, p, k = oracle.scatter_add_running(v, np.full(5, 9, np.int32), np.zeros(3, F32))
    assert k == 5 and np.all(np.isnan(p)) and same_bits(o, np.zeros(3, F32))
    o, p, k = oracle.scatter_add_running(np.zeros(0, F64), np.zeros(0, np.int32),
                                         np.ones(2, F64))
    assert k == 0 and p.size == 0 and same_bits(o, np.ones(2, F64))
