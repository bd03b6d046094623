"""Pins for the oracle's keyed scatter-add (scalar bins and row-indexed accumulate).

Order: contributions to one destination are taken in ascending source index (Warp
"Deterministic Execution": records sorted stably by destination and thread index, then
each group reduced in a fixed order; "Writing Manual Deterministic Code": one output,
inputs visited in index order) and combined by the adjacent-pair tree; the destination's
initial value is added once, last.  Rows follow ``warp.tile_atomic_add_indexed``: axis-0
indices, out-of-range destinations skipped, previous values returned.

Checks: the page's printed worked example (tests/golden), Warp's quick-start shape (4,096
ones into bin 0), cross-op identities (all-in-one-bin equals +0.0 plus the reproducible sum;
identity bins are an elementwise add), relabelling, brute-force grouping by boolean masks,
columns of a row scatter equal scalar scatters, skipped indices, and a per-bin error bound.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

F32 = np.float32
F64 = np.float64
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def same_bits(a, b):
    return np.asarray(a).tobytes() == np.asarray(b).tobytes()


def test_tile_atomic_add_indexed_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "tile_atomic_add_indexed_example.json")))
    x = np.array(g["x"], F32)
    y0 = np.array(g["y_init"], F32)
    rows = np.array(g["rows"], np.int32)
    y, prev, skipped = oracle.scatter_add(x, rows, y0, want_prev=True)
    assert np.array_equal(y, np.array(g["y_expected"], F32))
    assert np.array_equal(prev, np.array(g["previous_expected"], F32))
    assert skipped == 0


def test_quickstart_4096_ones_into_bin0():
    out, _, k = oracle.scatter_add(np.ones(4096, F32), np.zeros(4096, np.int32),
                                   np.zeros(1, F32))
    assert out[0] == 4096.0 and k == 0


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("n", [1, 7, 1000, 65537])
def test_contended_equals_plus_zero_plus_sum(dtype, n):
    v = (np.random.default_rng(n).standard_normal(n) * 10.0 ** np.random.default_rng(n + 1)
         .uniform(-3, 3, n)).astype(dtype)
    out, _, _ = oracle.scatter_add(v, np.zeros(n, np.int32), np.zeros(1, dtype))
    assert same_bits(out[0], dtype(0.0) + oracle.det_sum(v))


@pytest.mark.parametrize("dtype", [F32, F64])
def test_identity_bins_elementwise(dtype):
    rng = np.random.default_rng(2)
    v = rng.standard_normal(500).astype(dtype)
    o = rng.standard_normal(500).astype(dtype)
    out, prev, _ = oracle.scatter_add(v, np.arange(500, dtype=np.int32), o, want_prev=True)
    assert same_bits(out, o + v)
    assert same_bits(prev, o)


@pytest.mark.parametrize("dtype", [F32, F64])
def test_brute_force_grouping(dtype):
    rng = np.random.default_rng(3)
    n, B = 3000, 37
    v = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 4, n)).astype(dtype)
    idx = rng.integers(-3, B + 3, n).astype(np.int32)          # some out of range
    o = rng.standard_normal(B).astype(dtype)
    out, prev, skipped = oracle.scatter_add(v, idx, o, want_prev=True)
    assert skipped == int(((idx < 0) | (idx >= B)).sum())
    for b in range(B):
        members = v[idx == b]                                   # ascending source index
        want = o[b] + oracle.pw(members) if members.size else o[b]
        assert same_bits(out[b], want), b
    valid = (idx >= 0) & (idx < B)
    assert same_bits(prev[valid], o[idx[valid]])
    assert np.isnan(prev[~valid]).all()                         # skipped rows not written


def test_relabelling_permutes_outputs():
    rng = np.random.default_rng(4)
    n, B = 2000, 50
    v = rng.standard_normal(n).astype(F32)
    idx = rng.integers(0, B, n).astype(np.int32)
    perm = rng.permutation(B).astype(np.int32)
    o = np.zeros(B, F32)
    a, _, _ = oracle.scatter_add(v, idx, o)
    b, _, _ = oracle.scatter_add(v, perm[idx], o)
    assert same_bits(b[perm], a)


def test_empty_bins_untouched_bits():
    o = np.array([np.nan, -0.0, 1.5, np.inf], F32)
    out, _, _ = oracle.scatter_add(np.array([2.0], F32), np.array([2], np.int32), o)
    assert same_bits(out[[0, 1, 3]], o[[0, 1, 3]]) and out[2] == 3.5


@pytest.mark.parametrize("dtype", [F32, F64])
def test_rows_columns_equal_scalar_scatter(dtype):
    rng = np.random.default_rng(5)
    n, d, B = 400, 6, 23
    v = (rng.standard_normal((n, d)) * 10.0 ** rng.uniform(-3, 3, (n, d))).astype(dtype)
    idx = rng.integers(-1, B + 1, n).astype(np.int32)
    o = rng.standard_normal((B, d)).astype(dtype)
    out, prev, skipped = oracle.scatter_add(v, idx, o, want_prev=True)
    for c in range(d):
        oc, pc, kc = oracle.scatter_add(v[:, c].copy(), idx, o[:, c].copy(), want_prev=True)
        assert same_bits(out[:, c], oc) and kc == skipped
        valid = (idx >= 0) & (idx < B)
        assert same_bits(prev[valid, c], pc[valid])


@pytest.mark.parametrize("dtype,u", [(F32, 2.0**-24), (F64, 2.0**-53)])
def test_per_bin_error_bound(dtype, u):
    rng = np.random.default_rng(6)
    n, B = 20000, 16
    v = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 4, n)).astype(dtype)
    idx = rng.integers(0, B, n).astype(np.int32)
    o = rng.standard_normal(B).astype(dtype)
    out, _, _ = oracle.scatter_add(v, idx, o)
    for b in range(B):
        m = v[idx == b].astype(np.float64)
        exact = math.fsum([float(o[b])] + m.tolist())
        k = math.ceil(math.log2(m.size)) + 1
        g = k * u / (1 - k * u)
        assert abs(float(out[b]) - exact) <= g * (abs(float(o[b])) + np.abs(m).sum()) * (1 + 1e-9)


# ---------------------------------------------------------------- scatter-subtract
# Warp "Deterministic Execution", Pattern 1, table of atomics: atomic_sub's values are negated
# and added in a fixed order.  Pins worked by hand, each separating that reading from the
# plausible alternatives.

def test_sub_signed_zero_is_negate_then_add():
    # out = -0.0, contributions [+0.0, -0.0] and [1, -1]: negated they still cancel to +0.0,
    # and -0.0 + +0.0 = +0.0.  Subtracting the reduced sum instead gives -0.0 - (+0.0) = -0.0.
    for vals in ([0.0, -0.0], [1.0, -1.0]):
        v = np.array(vals, np.float32)
        got, _, _ = oracle.scatter_sub(v, np.zeros(2, np.int32), np.array([-0.0], np.float32))
        assert got.view(np.uint32)[0] == 0x00000000, vals


def test_sub_keeps_the_tree():
    # [1, 2^-24, 2^-24, 2^-24] into bin 0 (out = +0.0), negated: (-1 - 2^-24) rounds to -1,
    # (-2^-24 - 2^-24) = -2^-23, so the tree gives -(1 + 2^-23) = 0xbf800001; a left-to-right
    # walk would give -1.0 (0xbf800000).
    u = np.float32(2.0 ** -24)
    v = np.array([1.0, u, u, u], np.float32)
    got, _, _ = oracle.scatter_sub(v, np.zeros(4, np.int32), np.zeros(1, np.float32))
    assert got.view(np.uint32)[0] == 0xBF800001
    got64, _, _ = oracle.scatter_sub(np.array([1.0, 2.0 ** -53, 2.0 ** -53, 2.0 ** -53]),
                                     np.zeros(4, np.int32), np.zeros(1))
    assert got64[0] == -(1.0 + 2.0 ** -52)


def test_sub_ones_and_integers_exact():
    got, _, _ = oracle.scatter_sub(np.ones(4096, np.float32), np.zeros(4096, np.int32),
                                   np.zeros(1, np.float32))
    assert got[0] == -4096.0
    rng = np.random.default_rng(5)
    v = rng.integers(-1000, 1000, 20000).astype(np.float64)
    idx = rng.integers(0, 37, 20000).astype(np.int32)
    o = rng.integers(-10 ** 6, 10 ** 6, 37).astype(np.float64)
    got, _, k = oracle.scatter_sub(v, idx, o)
    want = o.copy()
    np.subtract.at(want, idx, v)        # integers: exact in any order
    assert k == 0 and np.array_equal(got, want)
