"""Pins for the oracle's anchored prefix scan.

The scan's order (tiles of NW waves x W lanes x V elements, lane-serial runs, Kogge-Stone
passes over lane totals inside each wave and over the wave totals, pairwise trees over tile
totals inside anchor intervals of A tiles and over interval totals inside super-intervals of
A2 intervals, and a carry that only crosses super-intervals) follows drjit-core pull request
"Make CUDA floating-point prefix sums deterministic" (sections "Implementation" and
"Validation").  The oracle takes V, W, NW, A, A2 as parameters so tiny instances can be worked
out by hand.

Checks, none of which reuses the oracle's code:
* hand-written expressions for tiny (V, W, NW, A, A2) instances, evaluated with numpy scalars;
* a top-down brute-force evaluator that builds every output's expression tree from the
  stated order and evaluates it (tiny n, many tiles and intervals);
* textbook special cases: n <= V is a sequential cumulative sum (numpy's ``cumsum``);
  all-ones inputs give exact integers in every mode;
* invariants at the real constants: exclusive is inclusive shifted, reverse is the mirror
  of forward, one segment equals the unsegmented scan, a segment's outputs equal the
  unsegmented scan with everything before the segment replaced by the identity;
* the error bound of the expression depth against exact prefix sums.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle

F32 = np.float32
F64 = np.float64


def rounding_values(n, dtype, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 4, n)
            * np.where(rng.random(n) < 0.5, -1, 1)).astype(dtype)


def same_bits(a, b):
    return np.asarray(a).tobytes() == np.asarray(b).tobytes()


# ---------------------------------------------------------------- hand-written tiny instances

@pytest.mark.parametrize("seed", range(20))
def test_hand_V2_W2_A2_two_tiles(seed):
    x = rounding_values(8, F32, seed)
    x0, x1, x2, x3, x4, x5, x6, x7 = x
    agg0 = (x0 + x1) + (x2 + x3)
    want = [x0, x0 + x1, (x0 + x1) + x2, (x0 + x1) + (x2 + x3),
            agg0 + x4, agg0 + (x4 + x5), (agg0 + (x4 + x5)) + x6, (agg0 + (x4 + x5)) + (x6 + x7)]
    y = oracle.scan(x, V=2, W=2, NW=1, A=2)
    assert same_bits(y, np.array(want, F32))


@pytest.mark.parametrize("seed", range(20))
def test_hand_V1_W1_A1_A2_2_carry_chain(seed):
    # one element per tile and per interval; super-intervals of two; the carry into
    # super-interval Q+1 is CC_Q + (x_2Q + x_2Q+1), while the last output of Q is
    # (CC_Q + x_2Q) + x_2Q+1
    x = rounding_values(7, F32, seed)
    c1 = x[0] + x[1]
    c2 = c1 + (x[2] + x[3])
    c3 = c2 + (x[4] + x[5])
    want = [x[0], x[0] + x[1], c1 + x[2], (c1 + x[2]) + x[3], c2 + x[4], (c2 + x[4]) + x[5],
            c3 + x[6]]
    assert same_bits(oracle.scan(x, V=1, W=1, NW=1, A=1, A2=2), np.array(want, F32))


@pytest.mark.parametrize("seed", range(20))
def test_hand_V1_W1_A4_lookback_tree(seed):
    x = rounding_values(8, F32, seed)
    x0, x1, x2, x3, x4, x5, x6, x7 = x
    c1 = (x0 + x1) + (x2 + x3)
    want = [x0, x0 + x1, (x0 + x1) + x2, ((x0 + x1) + x2) + x3,
            c1 + x4, (c1 + x4) + x5, (c1 + (x4 + x5)) + x6, (c1 + ((x4 + x5) + x6)) + x7]
    assert same_bits(oracle.scan(x, V=1, W=1, NW=1, A=4), np.array(want, F32))


@pytest.mark.parametrize("seed", range(20))
def test_hand_interval_tree_A1_A2_8(seed):
    # intervals of one tile, super-intervals of 8: the carry into interval q is the pairwise
    # tree of the earlier interval totals (not a left-to-right chain)
    x = rounding_values(9, F32, seed)
    x0, x1, x2, x3, x4, x5, x6, x7, x8 = x
    p4 = (x0 + x1) + (x2 + x3)
    p8 = p4 + ((x4 + x5) + (x6 + x7))
    want = [x0, x0 + x1, (x0 + x1) + x2, ((x0 + x1) + x2) + x3, p4 + x4, (p4 + x4) + x5,
            (p4 + (x4 + x5)) + x6, (p4 + ((x4 + x5) + x6)) + x7, p8 + x8]
    assert same_bits(oracle.scan(x, V=1, W=1, NW=1, A=1, A2=8), np.array(want, F32))


@pytest.mark.parametrize("seed", range(20))
def test_hand_A2_A2_2_two_level_anchors(seed):
    # tiles of one element, intervals of 2 tiles, super-intervals of 2 intervals
    x = rounding_values(9, F32, seed)
    x0, x1, x2, x3, x4, x5, x6, x7, x8 = x
    g0, g1, g2, g3 = x0 + x1, x2 + x3, x4 + x5, x6 + x7
    cc1 = g0 + g1
    c3 = cc1 + g2
    cc2 = cc1 + (g2 + g3)
    want = [x0, x0 + x1, g0 + x2, (g0 + x2) + x3, cc1 + x4, (cc1 + x4) + x5, c3 + x6,
            (c3 + x6) + x7, cc2 + x8]
    assert same_bits(oracle.scan(x, V=1, W=1, NW=1, A=2, A2=2), np.array(want, F32))


@pytest.mark.parametrize("seed", range(20))
def test_hand_V1_W4_A1_kogge_stone(seed):
    x = rounding_values(8, F32, seed)
    x0, x1, x2, x3, x4, x5, x6, x7 = x
    a0 = (x0 + x1) + (x2 + x3)
    want = [x0, x0 + x1, (x0 + x1) + x2, (x0 + (x1 + x2)) + x3,
            a0 + x4, (a0 + x4) + x5, (a0 + (x4 + x5)) + x6, (a0 + (x4 + (x5 + x6))) + x7]
    assert same_bits(oracle.scan(x, V=1, W=4, NW=1, A=1), np.array(want, F32))


@pytest.mark.parametrize("seed", range(20))
def test_hand_V1_W2_NW2_A1_two_level(seed):
    # two waves of two lanes: lane prefixes inside a wave, then the wave totals
    # (a single Kogge-Stone over four lanes would give y3 = (x0 + (x1 + x2)) + x3 instead)
    x = rounding_values(8, F32, seed)
    x0, x1, x2, x3, x4, x5, x6, x7 = x
    a0 = (x0 + x1) + (x2 + x3)
    want = [x0, x0 + x1, (x0 + x1) + x2, ((x0 + x1) + x2) + x3,
            a0 + x4, (a0 + x4) + x5, (a0 + (x4 + x5)) + x6, ((a0 + (x4 + x5)) + x6) + x7]
    assert same_bits(oracle.scan(x, V=1, W=2, NW=2, A=1), np.array(want, F32))


@pytest.mark.parametrize("seed", range(20))
def test_hand_segmented_and_exclusive(seed):
    # V=1, W=4, NW=1, A=1, segments [0,2) [2,5) [5,8)
    x = rounding_values(8, F32, seed)
    x0, x1, x2, x3, x4, x5, x6, x7 = x
    offs = np.array([0, 2, 5, 8])
    incl = [x0, x0 + x1, x2, x2 + x3, (x2 + x3) + x4, x5, x5 + x6, (x5 + x6) + x7]
    assert same_bits(oracle.scan(x, offsets=offs, V=1, W=4, NW=1, A=1), np.array(incl, F32))
    excl = [0.0, incl[0], 0.0, incl[2], incl[3], 0.0, incl[5], incl[6]]
    assert same_bits(oracle.scan(x, exclusive=True, offsets=offs, V=1, W=4, NW=1, A=1),
                     np.array(excl, F32))


# ---------------------------------------------------------------- brute force, top down

def _pw_expr(items):
    if not items:
        return None
    if len(items) == 1:
        return items[0]
    k = 1
    while 2 * k < len(items):
        k *= 2
    return (_pw_expr(items[:k]), _pw_expr(items[k:]))


def _brute_exprs(n, V, W, NW, A, A2):
    """Expression of every forward inclusive output; leaves are indices, None = identity."""
    T = V * W * NW

    def leaf(i):
        return i if i < n else None

    def lane_prefix(j, t, k):
        e = leaf(j * T + t * V)
        for r in range(1, k + 1):
            e = (e, leaf(j * T + t * V + r))
        return e

    def pow2_at_least(m):
        d = 1
        while d < m:
            d *= 2
        return d

    DW, DN = pow2_at_least(W), pow2_at_least(NW)

    def ks(j, t, d):  # lane t after the in-wave Kogge-Stone steps with offsets < d
        if d == 1:
            return lane_prefix(j, t, V - 1)
        h = d // 2
        return (ks(j, t - h, h), ks(j, t, h)) if t % W >= h else ks(j, t, h)

    def wks(j, w, d):  # wave total w after the wave-level steps with offsets < d
        if d == 1:
            return ks(j, w * W + W - 1, DW)
        h = d // 2
        return (wks(j, w - h, h), wks(j, w, h)) if w >= h else wks(j, w, h)

    def agg(j):
        return wks(j, NW - 1, DN)

    nt = (n + T - 1) // T
    nq = (nt + A - 1) // A

    def g(q):        # interval total
        return _pw_expr([agg(jj) for jj in range(q * A, min(q * A + A, nt))])

    def cc(Q):       # carry into super-interval Q
        if Q == 0:
            return None
        return (cc(Q - 1), _pw_expr([g(qq) for qq in range((Q - 1) * A2, min(Q * A2, nq))]))

    def carry(q):    # carry into interval q
        Q = q // A2
        return (cc(Q), _pw_expr([g(qq) for qq in range(Q * A2, q)]))

    out = []
    for i in range(n):
        j, r = divmod(i, T)
        t, k = divmod(r, V)
        w, l = divmod(t, W)
        q = j // A
        e = (carry(q), _pw_expr([agg(jj) for jj in range(q * A, j)]))
        pw_ = wks(j, w - 1, DN) if w > 0 else None
        p = ks(j, t - 1, DW) if l > 0 else None
        out.append((((e, pw_), p), lane_prefix(j, t, k)))
    return out


def _eval(expr, x, ident):
    if expr is None:
        return ident
    if isinstance(expr, tuple):
        return _eval(expr[0], x, ident) + _eval(expr[1], x, ident)
    return x[expr]


@pytest.mark.parametrize("V,W,NW,A,A2", [(2, 2, 1, 2, 3), (1, 4, 1, 2, 2), (3, 2, 2, 3, 1),
                                          (2, 2, 2, 1, 4), (1, 1, 3, 3, 2), (4, 3, 2, 2, 5),
                                          (1, 2, 3, 2, 256), (2, 4, 4, 2, 2), (1, 1, 1, 1, 3)])
@pytest.mark.parametrize("dtype", [F32, F64])
def test_brute_force_expressions(V, W, NW, A, A2, dtype):
    rng = np.random.default_rng(V * 10000 + W * 1000 + NW * 100 + A * 10 + A2)
    eps = float(np.finfo(dtype).eps)
    alphabet = np.array([1.0, eps, eps / 2, -1.0, 3.0, -eps / 2, 0.75], dtype)
    ident = dtype(-0.0)
    for n in (1, 5, V * W * NW * A + 1, 3 * V * W * NW * A + 2, 40,
              min(300, 2 * V * W * NW * A * A2 + 3)):
        exprs = _brute_exprs(n, V, W, NW, A, A2)
        for trial in range(4):
            x = alphabet[rng.integers(0, alphabet.size, n)]
            want = np.array([_eval(e, x, ident) for e in exprs], dtype)
            assert same_bits(oracle.scan(x, V=V, W=W, NW=NW, A=A, A2=A2), want), (n, trial)
            # reverse: mirror of the forward scan of the flipped input
            wr = np.array([_eval(e, x[::-1].copy(), ident) for e in exprs], dtype)[::-1]
            assert same_bits(oracle.scan(x, reverse=True, V=V, W=W, NW=NW, A=A, A2=A2), wr)
            # segmented: mask everything before the segment start with the identity
            cuts = np.sort(rng.choice(np.arange(1, n), size=min(3, max(0, n - 1)),
                                      replace=False)) if n > 1 else np.zeros(0, int)
            offs = np.concatenate([[0], cuts, [n]])
            ws = np.empty(n, dtype)
            for a, b in zip(offs[:-1], offs[1:]):
                xm = x.copy()
                xm[:a] = ident
                for i in range(a, b):
                    ws[i] = _eval(exprs[i], xm, ident)
            assert same_bits(oracle.scan(x, offsets=offs, V=V, W=W, NW=NW, A=A, A2=A2), ws), (n, offs)


# ---------------------------------------------------------------- textbook special cases

@pytest.mark.parametrize("dtype", [F32, F64])
def test_single_lane_is_sequential_cumsum(dtype):
    for n in range(1, 33):
        x = rounding_values(n, dtype, n)
        assert same_bits(oracle.scan(x), np.cumsum(x, dtype=dtype))


@pytest.mark.parametrize("n", [1, 31, 32, 33, 8191, 8192, 8193, 16384, 164738])
def test_all_ones_every_mode(n):
    x = np.ones(n, F32)
    i = np.arange(n, dtype=np.float64)
    assert np.array_equal(oracle.scan(x), i + 1)
    assert np.array_equal(oracle.scan(x, exclusive=True), i)
    assert np.array_equal(oracle.scan(x, reverse=True), n - i)
    assert np.array_equal(oracle.scan(x, exclusive=True, reverse=True), n - 1 - i)
    offs = np.unique(np.concatenate([[0], np.arange(0, n, 97), [n]]))
    start = offs[np.searchsorted(offs, np.arange(n), side="right") - 1]
    assert np.array_equal(oracle.scan(x, offsets=offs), np.arange(n) - start + 1)


def test_all_ones_many_intervals():
    n = 3 * 256 * 8192 + 5                     # four anchor intervals at the spec constants
    y = oracle.scan(np.ones(n, F32))
    assert np.array_equal(y, np.arange(1, n + 1, dtype=np.float64))


# ---------------------------------------------------------------- invariants at spec constants

@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("n", [16384, 164738, 2 * 256 * 8192 + 4097])
def test_shift_mirror_and_segment_relations(dtype, n):
    x = rounding_values(n, dtype, 7)
    inc = oracle.scan(x)
    exc = oracle.scan(x, exclusive=True)
    assert same_bits(exc[1:], inc[:-1]) and same_bits(exc[:1], np.zeros(1, dtype))
    rev = oracle.scan(x, reverse=True)
    assert same_bits(rev, oracle.scan(x[::-1].copy())[::-1])
    rex = oracle.scan(x, exclusive=True, reverse=True)
    assert same_bits(rex[:-1], rev[1:]) and same_bits(rex[-1:], np.zeros(1, dtype))
    one = np.array([0, n])
    assert same_bits(oracle.scan(x, offsets=one), inc)
    assert same_bits(oracle.scan(x, offsets=one, reverse=True, exclusive=True), rex)
    # a few long segments, one empty: masking equivalence for each segment
    offs = np.array([0, 5000, 5000, n // 2 + 3, n - 1, n])
    seg = oracle.scan(x, offsets=offs)
    for a, b in zip(offs[:-1], offs[1:]):
        if a == b:
            continue
        xm = x.copy()
        xm[:a] = -0.0
        assert same_bits(seg[a:b], oracle.scan(xm)[a:b])
    segr = oracle.scan(x, offsets=offs, reverse=True)
    for a, b in zip(offs[:-1], offs[1:]):
        if a == b:
            continue
        xm = x.copy()
        xm[b:] = -0.0
        assert same_bits(segr[a:b], oracle.scan(xm, reverse=True)[a:b])


def test_heads_everywhere_copy_input():
    x = rounding_values(1000, F32, 3)
    offs = np.arange(0, 1001)
    assert same_bits(oracle.scan(x, offsets=offs), x)
    assert same_bits(oracle.scan(x, offsets=offs, exclusive=True), np.zeros(1000, F32))


def test_signed_zero_and_nonfinite():
    x = np.full(10, -0.0, F32)
    assert same_bits(oracle.scan(x), x)                        # -0.0 prefixes stay -0.0
    ex = oracle.scan(x, exclusive=True)
    assert ex[0].tobytes() == np.float32(0.0).tobytes()       # exclusive starts at +0.0
    x = np.array([1, np.inf, 1, -np.inf, 2], F32)
    y = oracle.scan(x)
    assert y[0] == 1 and y[1] == np.inf and y[2] == np.inf and np.isnan(y[3]) and np.isnan(y[4])


def test_bad_offsets_rejected():
    x = np.ones(10, F32)
    for offs in ([1, 10], [0, 9], [0, 6, 4, 10]):
        with pytest.raises(ValueError):
            oracle.scan(x, offsets=np.array(offs))


# ---------------------------------------------------------------- error bound

@pytest.mark.parametrize("dtype,u", [(F32, 2.0**-24), (F64, 2.0**-53)])
def test_error_bound_against_exact_prefix(dtype, u):
    V, W, NW, A, A2 = 4, 2, 2, 2, 3                   # many tiles, intervals and super-intervals
    n = 3000
    x = rounding_values(n, dtype, 9)
    y = oracle.scan(x, V=V, W=W, NW=NW, A=A, A2=A2)
    T = V * W * NW
    nQ = -(-(-(-(-(-n // T)) // A)) // A2)
    depth = (V + math.ceil(math.log2(W)) + math.ceil(math.log2(NW)) + math.ceil(math.log2(A))
             + math.ceil(math.log2(A2)) + nQ + 6)
    g = depth * u / (1 - depth * u)
    acc = Fraction(0)
    absacc = 0.0
    for i in range(n):
        acc += Fraction(float(x[i]))
        absacc += abs(float(x[i]))
        assert abs(Fraction(float(y[i])) - acc) <= Fraction(g * absacc * (1 + 1e-9)), i


# ---------------------------------------------------------------- int32 scan (slot allocation)
# Warp "Deterministic Execution", Pattern 2: count-scan-write's prefix scan over int32 counts.
# Integer sums wrap modulo 2^32 and need no order; pinned by hand-worked values, a Python-int
# loop, and the float oracle on integer data (whose sums are exact).

def test_int32_scan_wraps_by_hand():
    x = np.array([2 ** 31 - 1, 1, 5, -7], np.int32)
    assert oracle.scan_int32(x).tolist() == [2147483647, -2147483648, -2147483643, -2147483650 + 2 ** 32]
    assert oracle.scan_int32(x, exclusive=True).tolist() == [0, 2147483647, -2147483648, -2147483643]
    assert oracle.scan_int32(x, reverse=True).tolist() == [2147483646, -1, -2, -7]
    assert oracle.scan_int32(np.zeros(0, np.int32)).size == 0


def _loop_scan(x, exclusive, reverse, offs):
    # Python ints, one segment at a time, walked from its first element (its last for reverse)
    xs = [int(v) for v in x]
    y = [0] * len(xs)
    for a, b in zip(offs[:-1], offs[1:]):
        acc = 0
        for i in (range(int(b) - 1, int(a) - 1, -1) if reverse else range(int(a), int(b))):
            y[i] = acc if exclusive else acc + xs[i]
            acc += xs[i]
    return np.array([(v + 2 ** 31) % 2 ** 32 - 2 ** 31 for v in y], np.int64).astype(np.int32)


def test_int32_scan_against_python_ints():
    rng = np.random.default_rng(8)
    for n in (1, 2, 7, 64, 300):
        x = rng.integers(-2 ** 31, 2 ** 31, n).astype(np.int32)
        cuts = np.sort(rng.choice(np.arange(1, n + 1), min(n, 5), replace=False)) if n > 1 else []
        offs = np.unique(np.concatenate([[0], cuts, [n]])).astype(np.int64)
        for excl in (False, True):
            for rev in (False, True):
                for o in (None, offs):
                    oo = np.array([0, n], np.int64) if o is None else o
                    want = _loop_scan(x, excl, rev, oo)
                    got = oracle.scan_int32(x, exclusive=excl, reverse=rev, offsets=o)
                    assert np.array_equal(got, want), (n, excl, rev, o is not None)


def test_int32_scan_equals_float_oracle_on_integers():
    rng = np.random.default_rng(9)
    n = 3 * 8192 + 77
    x = rng.integers(-1000, 1000, n).astype(np.int32)
    offs = np.unique(np.concatenate([[0], rng.integers(1, n, 40), [n]])).astype(np.int64)
    for excl in (False, True):
        for rev in (False, True):
            f = oracle.scan(x.astype(np.float64), exclusive=excl, reverse=rev, offsets=offs)
            i = oracle.scan_int32(x, exclusive=excl, reverse=rev, offsets=offs)
            assert np.array_equal(f.astype(np.int64), i.astype(np.int64)), (excl, rev)
