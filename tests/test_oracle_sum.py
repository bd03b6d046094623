"""Pins for the oracle's pairwise tree (PW) and reproducible sum.

Each test checks the oracle against something other than itself: values derived by hand
from the definition of the adjacent-pair tree, closed forms (sums of ones, integer-valued
data), the textbook error bound of pairwise summation against an exactly rounded sum
(``math.fsum``), and a top-down recursive evaluation of the same tree.

Sources: course page "Floating point and reproducibility" (a sum is one bracketing; the
fixed tree pairs neighbours round after round; test on values that round) and Warp's
"Deterministic Execution" quick start (4,096 ones summed into one bin).
"""
import math

import numpy as np
import pytest

import oracle

F32 = np.float32
F64 = np.float64


def bits32(x):
    return int(np.array(x, dtype=F32).view(np.uint32))


def bits64(x):
    return int(np.array(x, dtype=F64).view(np.uint64))


# ---------------------------------------------------------------- hand-derived values

def test_adjacent_pairs_not_halving_not_sequential_f32():
    # [1, 2^-23, 2^-24, -1]
    #   adjacent pairs: (1 + 2^-23) + (2^-24 - 1) = 2^-23 + 2^-24 (both inner sums exact)
    #   halving pairs:  (1 + 2^-24) + (2^-23 - 1) = 1 + (2^-23 - 1) = 2^-23  (tie to even)
    #   left to right:  ((1 + 2^-23) + 2^-24) - 1 = 2^-22                    (tie to even)
    x = np.array([1, 2.0**-23, 2.0**-24, -1], F32)
    assert bits32(oracle.pw(x)) == 0x34400000          # 1.5 * 2^-23
    assert bits32(oracle.det_sum(x)) == 0x34400000


def test_five_elements_three_different_trees_f32():
    # [1, e, e, e, e] with e = 2^-24; 1 + e ties to 1.0
    #   adjacent, padded to 8: ((1+e)+(e+e)) + (e + pad) = (1 + 2^-23) + e -> 1 + 2^-22
    #   halving, padded to 8:  (1 + e) + (e + e) -> 1 + 2^-23
    #   left to right:         1.0
    e = 2.0**-24
    x = np.array([1, e, e, e, e], F32)
    assert bits32(oracle.pw(x)) == 0x3F800002


def test_ragged_tail_groups_left_f32():
    # [1, e, e]: (1 + e) + e = 1.0, whereas 1 + (e + e) = 1 + 2^-23
    e = 2.0**-24
    assert bits32(oracle.pw(np.array([1, e, e], F32))) == 0x3F800000
    # [e, e, 1]: (e + e) + 1 = 1 + 2^-23
    assert bits32(oracle.pw(np.array([e, e, 1], F32))) == 0x3F800001


def test_discriminator_f64():
    e = 2.0**-53
    x = np.array([1, e, e, e, e], F64)
    assert bits64(oracle.pw(x)) == 0x3FF0000000000002      # 1 + 2^-51
    x = np.array([1, 2.0**-52, 2.0**-53, -1], F64)
    assert oracle.pw(x) == 1.5 * 2.0**-52


def test_signed_zero_identity_and_empty_sum():
    assert bits32(oracle.det_sum(np.zeros(0, F32))) == 0x00000000      # empty -> +0.0
    assert bits64(oracle.det_sum(np.zeros(0, F64))) == 0
    assert bits32(oracle.det_sum(np.array([-0.0], F32))) == 0x80000000
    assert bits32(oracle.det_sum(np.full(5, -0.0, F32))) == 0x80000000  # padding is -0.0
    assert bits32(oracle.det_sum(np.array([0.0, -0.0], F32))) == 0
    assert bits32(oracle.det_sum(np.array([-0.0, -0.0, 0.0], F32))) == 0
    assert bits64(oracle.det_sum(np.full(3, -0.0, F64))) == 0x8000000000000000


def test_non_finite_and_subnormal():
    assert oracle.det_sum(np.array([np.inf, 1], F32)) == np.inf
    assert np.isnan(oracle.det_sum(np.array([np.inf, -np.inf, 1], F32)))
    assert np.isnan(oracle.det_sum(np.array([1, np.nan, 2], F64)))
    tiny = np.array([2.0**-149, 2.0**-149, 2.0**-149], F32)       # subnormals kept
    assert bits32(oracle.det_sum(tiny)) == 3
    assert oracle.det_sum(np.array([3e38, 3e38], F32)) == np.inf


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("n", [1, 2, 3, 5, 4096, 100003, 1 << 20])
def test_sum_of_ones_is_n(n):
    assert oracle.det_sum(np.ones(n, F32)) == n
    assert oracle.det_sum(np.ones(n, F64)) == n


def test_quickstart_4096_ones():
    # Warp quick start: 4,096 ones accumulated into one bin
    r = oracle.det_sum(np.ones(4096, F32))
    assert bits32(r) == bits32(4096.0)


@pytest.mark.parametrize("dtype,lim", [(F32, 1 << 8), (F64, 1 << 30)])
def test_integer_valued_sums_are_exact(dtype, lim):
    rng = np.random.default_rng(11)
    for n in (7, 1000, 65537):
        v = rng.integers(-lim, lim, n)
        assert int(np.abs(v).sum()) < (1 << 24 if dtype == F32 else 1 << 53)
        assert oracle.det_sum(v.astype(dtype)) == int(v.sum())


# ---------------------------------------------------------------- error bound

def _gamma(k, u):
    return k * u / (1 - k * u)


@pytest.mark.parametrize("dtype,u", [(F32, 2.0**-24), (F64, 2.0**-53)])
@pytest.mark.parametrize("n", [3, 1000, 1 << 16, 300007])
def test_pairwise_error_bound(dtype, u, n):
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 4, n)).astype(dtype)
    exact = math.fsum(x.astype(np.float64).tolist())
    s = float(oracle.det_sum(x))
    absum = float(np.abs(x.astype(np.float64)).sum())
    depth = math.ceil(math.log2(n))
    assert abs(s - exact) <= _gamma(depth, u) * absum * (1 + 1e-12) + 1e-300
    assert abs(s - exact) <= n * u * absum                # the looser n*u*sum|x| bound


def test_uniform01_relative_error():
    # same-sign data: the course page's 1e-5 relative check against a double reference
    x = np.random.default_rng(0).random(1 << 20, dtype=F32)
    exact = math.fsum(x.astype(np.float64).tolist())
    assert abs(float(oracle.det_sum(x)) - exact) / exact < 1e-5


# ---------------------------------------------------------------- same tree, other evaluation

def _pw_top_down(v):
    """Split at the largest power of two below m, add the two halves (numpy scalars)."""
    m = len(v)
    if m == 0:
        return v.dtype.type(-0.0)
    if m == 1:
        return v[0]
    k = 1
    while 2 * k < m:
        k *= 2
    return _pw_top_down(v[:k]) + _pw_top_down(v[k:])


@pytest.mark.parametrize("dtype", [F32, F64])
def test_top_down_recursion_matches(dtype):
    rng = np.random.default_rng(5)
    eps = float(np.finfo(dtype).eps)
    alphabet = np.array([1.0, eps, eps / 2, -1.0, 3.0, -eps / 2, 0.5], dtype)
    for m in list(range(1, 70)) + [127, 128, 129, 255, 257, 1000]:
        v = alphabet[rng.integers(0, alphabet.size, m)]
        assert oracle.pw(v).tobytes() == _pw_top_down(v).tobytes(), m


@pytest.mark.parametrize("dtype", [F32, F64])
def test_identity_padding_and_split_lemmas(dtype):
    rng = np.random.default_rng(6)
    for m in (5, 33, 100, 1025):
        v = (rng.standard_normal(m) * 10.0 ** rng.uniform(-3, 3, m)).astype(dtype)
        ref = oracle.pw(v).tobytes()
        for r in (1, 3, m, 2 * m + 1):                      # appended identities change nothing
            assert oracle.pw(np.concatenate([v, np.full(r, -0.0, dtype)])).tobytes() == ref
        k = 1
        while 2 * k < m:
            k *= 2
        assert (oracle.pw(v[:k]) + oracle.pw(v[k:])).tobytes() == ref
        # right-nested fold over the dyadic blocks of m's binary expansion
        blocks, pos = [], 0
        for bit in reversed(range(m.bit_length())):
            if m >> bit & 1:
                blocks.append(oracle.pw(v[pos:pos + (1 << bit)]))
                pos += 1 << bit
        acc = blocks[-1]
        for b in reversed(blocks[:-1]):
            acc = b + acc
        assert acc.tobytes() == ref


def test_ones_closed_form_matches_tree_and_oracle():
    # the O(log m) closed form used by the largest-size GPU tests, against a literal level-by-
    # level evaluation of the tree (small m) and against the oracle (m past 2^24, where the
    # f32 sums of ones start to round)
    from conftest import pw_ones

    def levels(m):
        p = 1
        while p < m:
            p *= 2
        v = [np.float32(1.0)] * m + [np.float32(-0.0)] * (p - m)
        while len(v) > 1:
            v = [np.float32(v[i] + v[i + 1]) for i in range(0, len(v), 2)]
        return v[0]

    for m in (1, 2, 3, 5, 7, 100, 1000, 4097):
        assert pw_ones(m, np.float32) == levels(m), m
    for m in ((1 << 24) + 1, (1 << 25) + 12345, (1 << 26) - 1):
        want = oracle.det_sum(np.ones(m, np.float32))
        got = pw_ones(m, np.float32)
        assert np.float32(want).view(np.uint32) == got.view(np.uint32), m
    assert float(pw_ones((1 << 26) - 1, np.float32)) != (1 << 26) - 1   # the sum does round
