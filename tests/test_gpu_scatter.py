"""det_scatter_add on the GPU against the oracle, bit for bit (through the C interface).

Scalar bins (f32, f64) across radix-pass counts (1, 2, 3 digit passes), out-of-range indices,
the fully contended case (every value into one bin, so the split of long destinations into
blocks and block values is exercised), identity bins, prev snapshots and skip counts; rows
(the tile accumulate) including the worked example on the "warp.tile_atomic_add_indexed"
page, row lengths that are not multiples of 64, and destinations with more than 64 rows.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from scan_fixed_order_amd import det, workloads
from conftest import bits_equal, first_mismatch

pytestmark = pytest.mark.gpu

F32, F64 = np.float32, np.float64
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_scatter(v, idx, out0, dev, want_prev=False):
    vt = torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    it = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to(dev)
    ot = torch.from_numpy(np.array(out0, copy=True)).to(dev)
    pt = torch.full(v.shape, float("nan"), dtype=vt.dtype, device=dev) if want_prev else None
    sk = torch.full((1,), -7, dtype=torch.int64, device=dev)
    det.det_scatter_add(vt, it, ot, prev=pt, n_skipped=sk)
    return ot.cpu().numpy(), (pt.cpu().numpy() if want_prev else None), int(sk.item())


def rounding(shape, dtype, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * 10.0 ** rng.uniform(-4, 4, shape)).astype(dtype)


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("n,B", [(1, 1), (7, 1), (1000, 7), (65537, 256), (65537, 257),
                                 (100003, 1000), (300007, 65536), (300007, 65537),
                                 (1 << 20, 1 << 20), (200000, 3), (2000003, 131073),
                                 (500009, (1 << 24) - 1), (500009, 1 << 24),
                                 (300007, (1 << 24) + 1),
                                 # 256 and 257 chunks of 1024 keys: the last size whose
                                 # bucket offsets take one launch, and the first that takes three
                                 (1 << 18, 300), ((1 << 18) + 1, 300), (3 * 1024 + 5, 70001),
                                 # three passes with a short last chunk (f64: 4096 keys per
                                 # chunk, f32: 8192): destination offsets counted from either
                                 # end of a chunk, and from the end of a bucket
                                 (3 * 4096 + 100, 70001), (2 * 8192 + 50, 200003)])
def test_scalar_parity(dev, dtype, n, B):
    rng = np.random.default_rng(n + B)
    v = rounding(n, dtype, n)
    idx = rng.integers(-2, B + 2, n).astype(np.int32)
    o = rounding(B, dtype, B)
    got, prev, k = gpu_scatter(v, idx, o, dev, want_prev=True)
    want, wprev, wk = oracle.scatter_add(v, idx, o, want_prev=True)
    assert bits_equal(got, want), (n, B, first_mismatch(got, want))
    assert k == wk
    assert bits_equal(prev, wprev)


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("B", [65536, 1 << 20])
@pytest.mark.parametrize("n", [1, 4096, 8192, 8193, 100003, 3 * 8192 * 8192 // 1024 + 1])
def test_contended_one_bin(dev, dtype, n, B):
    v = rounding(n, dtype, 1)
    idx = np.zeros(n, np.int32)
    o = np.zeros(B, dtype)
    got, _, k = gpu_scatter(v, idx, o, dev)
    want, _, _ = oracle.scatter_add(v, idx, o)
    assert bits_equal(got, want), (B, first_mismatch(got, want))
    assert k == 0
    # cross-op identity: +0.0 plus the reproducible sum
    s = det.det_sum(torch.from_numpy(v).to(dev)).cpu().numpy()
    assert bits_equal(got[:1], (dtype(0.0) + s).reshape(1))


def test_quickstart(dev):
    got, _, k = gpu_scatter(np.ones(4096, F32), np.zeros(4096, np.int32), np.zeros(1, F32), dev)
    assert got[0] == 4096.0 and k == 0


def test_identity_bins_and_all_skipped(dev):
    n = 70000
    v = rounding(n, F32, 2)
    o = rounding(n, F32, 3)
    got, prev, k = gpu_scatter(v, np.arange(n, dtype=np.int32), o, dev, want_prev=True)
    assert bits_equal(got, o + v) and bits_equal(prev, o) and k == 0
    idx = np.full(n, -1, np.int32)
    got, prev, k = gpu_scatter(v, idx, o, dev, want_prev=True)
    assert bits_equal(got, o) and k == n and np.isnan(prev).all()


def test_empty_inputs(dev):
    got, _, k = gpu_scatter(np.zeros(0, F32), np.zeros(0, np.int32), np.ones(5, F32), dev)
    assert bits_equal(got, np.ones(5, F32)) and k == 0
    got, _, k = gpu_scatter(np.ones(9, F32), np.zeros(9, np.int32), np.zeros(0, F32), dev)
    assert got.size == 0 and k == 9


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("B", [160, 256, 400, 505])
def test_blocks_between_2048_and_8192(dev, dtype, B):
    # destinations of about 2,000 to 6,600 members: blocks longer than 2048 values, up to four
    # of them starting in one 8192-position range, at every offset
    n = 1 << 20
    rng = np.random.default_rng(B)
    v = rounding(n, dtype, B + 1)
    idx = rng.integers(-1, B + 1, n).astype(np.int32)
    o = rounding(B, dtype, B + 2)
    got, _, k = gpu_scatter(v, idx, o, dev)
    want, _, wk = oracle.scatter_add(v, idx, o)
    assert bits_equal(got, want), (B, first_mismatch(got, want))
    assert k == wk


def test_c2_shape_2_24(dev):
    n = 1 << 24
    v = workloads.normal(n, seed=1)
    idx = workloads.bins_uniform(n, 65536, seed=1)
    o = np.zeros(65536, F32)
    got, _, _ = gpu_scatter(v, idx, o, dev)
    want, _, _ = oracle.scatter_add(v, idx, o)
    assert bits_equal(got, want), first_mismatch(got, want)


def test_zipf_f64(dev):
    n = 1 << 22
    v = workloads.mixed_f64(n, seed=4)
    idx = workloads.zipf_bins(n, 1 << 20, seed=4)
    o = np.zeros(1 << 20, F64)
    got, _, _ = gpu_scatter(v, idx, o, dev)
    want, _, _ = oracle.scatter_add(v, idx, o)
    assert bits_equal(got, want), first_mismatch(got, want)


# f64 into (65536, 2^20] destinations with more than 2^22 values: two 10-bit digit passes
@pytest.mark.parametrize("n,B", [((1 << 22) + 4097, 65537), ((1 << 22) + 1, 1 << 20),
                                 (5_000_011, 300_007)])
def test_ten_bit_passes_parity(dev, n, B):
    rng = np.random.default_rng(n ^ B)
    v = rounding(n, F64, n % 1000)
    idx = rng.integers(-2, B + 2, n).astype(np.int32)   # a few out of range
    o = rounding(B, F64, B % 1000)
    got, prev, k = gpu_scatter(v, idx, o, dev, want_prev=True)
    want, wprev, wk = oracle.scatter_add(v, idx, o, want_prev=True)
    assert bits_equal(got, want), (n, B, first_mismatch(got, want))
    assert k == wk
    assert bits_equal(prev, wprev)


@pytest.mark.parametrize("kind", ["zipf", "one_low_digit", "one_high_digit", "one_bin", "sub",
                                  "all_out"])
def test_ten_bit_passes_skew(dev, kind):
    n, B = (1 << 22) + 777, 1 << 20
    rng = np.random.default_rng(7)
    v = rounding(n, F64, 3)
    if kind == "zipf":
        idx = workloads.zipf_bins(n, B, seed=5)
    elif kind == "one_low_digit":    # every key in one bucket of the first pass
        idx = (rng.integers(0, B >> 10, n) * 1024 + 5).astype(np.int32)
    elif kind == "one_high_digit":   # every key in one bucket of the second pass
        idx = rng.integers(0, 1024, n).astype(np.int32)
    elif kind == "one_bin":
        idx = np.full(n, B - 1, np.int32)
    elif kind == "all_out":          # every key out of range: nothing is added
        idx = np.where(rng.random(n) < 0.5, -1, B + 7).astype(np.int32)
    else:
        idx = rng.integers(0, B, n).astype(np.int32)
    o = rounding(B, F64, 11)
    if kind == "sub":
        vt = torch.from_numpy(v).to(dev)
        it = torch.from_numpy(idx).to(dev)
        ot = torch.from_numpy(o.copy()).to(dev)
        det.det_scatter_sub(vt, it, ot)
        got = ot.cpu().numpy()
        want = oracle.scatter_sub(v, idx, o)
        want = want[0] if isinstance(want, tuple) else want
    else:
        got, _, k = gpu_scatter(v, idx, o, dev)
        want, _, wk = oracle.scatter_add(v, idx, o)
        assert k == wk
    assert bits_equal(got, want), (kind, first_mismatch(got, want))


def test_ten_bit_path_is_taken(dev):
    # f64 into (65536, 2^20] destinations: two radix passes above 2^22 values, three 8-bit
    # passes up to 2^22 (same bits either way, checked above)
    B = 1 << 20
    for n, passes in [((1 << 22) + 1, 2), (1 << 22, 3)]:
        v = torch.zeros(n, dtype=torch.float64, device=dev)
        idx = torch.zeros(n, dtype=torch.int32, device=dev)
        out = torch.zeros(B, dtype=torch.float64, device=dev)
        torch.cuda.synchronize()
        det.det_debug_kernel_timing(True)
        try:
            det.det_scatter_add(v, idx, out)
            torch.cuda.synchronize()
            rep = det.det_debug_kernel_report()
        finally:
            det.det_debug_kernel_timing(False)
        assert rep["k_radix_scatter"][0] == passes, (n, rep["k_radix_scatter"])


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("B", [100, 300])
def test_scalar_piece_boundaries(dev, dtype, B):
    # member counts around the reduction's cuts: one lane (<= 32), a piece of 512 or 1024
    # positions, several 1024-position pieces of one block (up to 8), whole 8192-position
    # blocks and the long-destination combine; B = 100 takes the 32-bit-key reduction, 300 the
    # byte path's
    sizes = [1, 32, 33, 512, 513, 1023, 1024, 1025, 2047, 2049, 4096, 5000, 8191, 8192, 8193,
             3 * 8192 + 1000]
    rng = np.random.default_rng(B + len(sizes))
    listed = [(7 * k) % B for k in range(len(sizes))]
    others = np.array([b for b in range(-1, B + 1) if b not in listed], np.int32)
    idx = np.concatenate([np.full(c, b, np.int32) for b, c in zip(listed, sizes)]
                         + [others[rng.integers(0, others.size, 3001)]])
    idx = idx[rng.permutation(idx.size)]
    v = rounding(idx.size, dtype, B)
    o = rounding(B, dtype, B + 1)
    got, prev, k = gpu_scatter(v, idx, o, dev, want_prev=True)
    want, wprev, wk = oracle.scatter_add(v, idx, o, want_prev=True)
    assert bits_equal(got, want), (B, first_mismatch(got, want))
    assert k == wk and bits_equal(prev, wprev)


# ---------------------------------------------------------------- rows

def test_rows_worked_example(dev):
    g = json.load(open(os.path.join(GOLDEN, "tile_atomic_add_indexed_example.json")))
    got, prev, k = gpu_scatter(np.array(g["x"], F32), np.array(g["rows"], np.int32),
                               np.array(g["y_init"], F32), dev, want_prev=True)
    assert np.array_equal(got, np.array(g["y_expected"], F32))
    assert np.array_equal(prev, np.array(g["previous_expected"], F32)) and k == 0


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("n,d,B", [(100, 3, 10), (1000, 100, 37), (4096, 256, 1 << 10),
                                   (5000, 65, 1), (3000, 300, 2), (20000, 8, 1 << 15)])
def test_rows_parity(dev, dtype, n, d, B):
    rng = np.random.default_rng(n * d + B)
    v = rounding((n, d), dtype, n)
    idx = rng.integers(-1, B + 1, n).astype(np.int32)
    o = rounding((B, d), dtype, d)
    got, prev, k = gpu_scatter(v, idx, o, dev, want_prev=True)
    want, wprev, wk = oracle.scatter_add(v, idx, o, want_prev=True)
    assert bits_equal(got, want), (n, d, B, first_mismatch(got, want))
    assert k == wk and bits_equal(prev, wprev)


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("sizes,d", [
    # member counts chosen for the long-destination counter: 2..7 blocks of 64, whole groups of
    # 8 blocks (one and several counter levels), groups plus a partial last group
    ((65, 64 * 7 + 1, 64 * 8, 64 * 8 + 1, 64 * 8 * 3 + 64 * 5 + 10, 64 * 64 * 2 + 3), 5),
    ((1024,) * 16, 256),
    # more than 64 chunks of 64 columns: a wave walks the column chunks
    ((150, 151), 4160)])
def test_rows_long_destinations(dev, dtype, sizes, d):
    rng = np.random.default_rng(sum(sizes) + d)
    idx = np.concatenate([np.full(c, b, np.int32) for b, c in enumerate(sizes)])
    idx = np.concatenate([idx, np.array([-1, len(sizes)], np.int32)])
    idx = idx[rng.permutation(idx.size)]
    v = rounding((idx.size, d), dtype, d)
    o = rounding((len(sizes), d), dtype, 1)
    got, prev, k = gpu_scatter(v, idx, o, dev, want_prev=True)
    want, wprev, wk = oracle.scatter_add(v, idx, o, want_prev=True)
    assert bits_equal(got, want), (sizes, d, first_mismatch(got, want))
    assert k == wk == 2 and bits_equal(prev, wprev)


@pytest.mark.parametrize("dtype", [F32, F64])
def test_rows_long_destinations_far_apart(dev, dtype):
    # 2^20 destinations of 2 columns: the long-destination search walks them in rounds of
    # 64 per wave, so long destinations sit in the first round, past 2^19 and at the end
    B, d = 1 << 20, 2
    rng = np.random.default_rng(17)
    long_ones = {3: 100, 600_000: 130, 1_000_003: 64 * 9 + 1, B - 1: 700}
    idx = np.concatenate([np.full(c, b, np.int32) for b, c in long_ones.items()]
                         + [rng.integers(0, B, 3000).astype(np.int32)])
    idx = idx[rng.permutation(idx.size)]
    v = rounding((idx.size, d), dtype, 5)
    o = rounding((B, d), dtype, 6)
    got, _, k = gpu_scatter(v, idx, o, dev)
    want, _, _ = oracle.scatter_add(v, idx, o)
    assert bits_equal(got, want), first_mismatch(got, want)
    assert k == 0


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("d", [70, 256, 300])
def test_rows_special_values_short_blocks(dev, dtype, d):
    # a few members per destination (blocks of at most 8 rows, taken two per wave when the row
    # fits one pass of columns), ragged column counts, NaN, infinities, signed zeros and
    # subnormals, out-of-range rows
    rng = np.random.default_rng(d)
    n, B = 20000, 5000
    v = rounding((n, d), dtype, d + 1)
    tiny = np.finfo(dtype).smallest_subnormal
    special = np.array([np.nan, np.inf, -np.inf, -0.0, 0.0, tiny, -tiny], dtype)
    flat = v.reshape(-1)
    pos = rng.choice(flat.size, 5000, replace=False)
    flat[pos] = special[rng.integers(0, special.size, pos.size)]
    idx = rng.integers(-1, B + 1, n).astype(np.int32)
    o = rounding((B, d), dtype, d + 2)
    o.reshape(-1)[::7] = -0.0
    got, prev, k = gpu_scatter(v, idx, o, dev, want_prev=True)
    want, wprev, wk = oracle.scatter_add(v, idx, o, want_prev=True)
    assert bits_equal(got, want), (d, first_mismatch(got, want))
    assert k == wk and bits_equal(prev, wprev)


def test_rows_c4_shape(dev):
    src, rows, out0 = workloads.rows_case()
    got, _, _ = gpu_scatter(src, rows, out0, dev)
    want, _, _ = oracle.scatter_add(src, rows, out0)
    assert bits_equal(got, want), first_mismatch(got, want)


# ---------------------------------------------------------------- scatter-subtract, gather

def gpu_scatter_sub(v, idx, out0, dev, want_prev=False):
    vt = torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    it = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to(dev)
    ot = torch.from_numpy(np.array(out0, copy=True)).to(dev)
    pt = torch.full(v.shape, float("nan"), dtype=vt.dtype, device=dev) if want_prev else None
    sk = torch.full((1,), -7, dtype=torch.int64, device=dev)
    det.det_scatter_sub(vt, it, ot, prev=pt, n_skipped=sk)
    return ot.cpu().numpy(), (pt.cpu().numpy() if want_prev else None), int(sk.item())


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("n,B", [(7, 1), (100003, 1000), (300007, 65536), (300007, 65537),
                                 (200000, 3), (3 * 8192 * 8 + 5, 1)])
def test_scatter_sub_parity(dev, dtype, n, B):
    rng = np.random.default_rng(n * 7 + B)
    v = rounding(n, dtype, n + 1)
    idx = rng.integers(-2, B + 2, n).astype(np.int32)
    o = rounding(B, dtype, B + 1)
    got, prev, k = gpu_scatter_sub(v, idx, o, dev, want_prev=True)
    want, wprev, wk = oracle.scatter_sub(v, idx, o, want_prev=True)
    assert bits_equal(got, want), (n, B, first_mismatch(got, want))
    assert k == wk and bits_equal(prev, wprev)


@pytest.mark.parametrize("dtype", [F32, F64])
def test_scatter_sub_signed_zero_and_tree(dev, dtype):
    # -0.0 minus contributions that cancel is +0.0 (negate, then add); the tree is kept
    v = np.array([0.0, -0.0, 1.0, -1.0], dtype)
    got, _, _ = gpu_scatter_sub(v, np.array([0, 0, 1, 1], np.int32), np.array([-0.0, -0.0], dtype),
                                dev)
    want, _, _ = oracle.scatter_sub(v, np.array([0, 0, 1, 1], np.int32),
                                    np.array([-0.0, -0.0], dtype))
    assert bits_equal(got, want) and not np.signbit(got).any()
    e = np.finfo(dtype).eps / 2
    v = np.array([1.0, e, e, e], dtype)
    got, _, _ = gpu_scatter_sub(v, np.zeros(4, np.int32), np.zeros(1, dtype), dev)
    assert got[0] == -(1.0 + 2 * e)


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("n,rows,d", [(5000, 300, 96), (20000, 8, 33)])
def test_scatter_sub_rows_parity(dev, dtype, n, rows, d):
    rng = np.random.default_rng(n + d)
    v = rounding((n, d), dtype, n)
    idx = rng.integers(0, rows, n).astype(np.int32)
    o = rounding((rows, d), dtype, rows)
    got, _, _ = gpu_scatter_sub(v, idx, o, dev)
    want, _, _ = oracle.scatter_sub(v, idx, o)
    assert bits_equal(got, want), first_mismatch(got, want)


@pytest.mark.parametrize("dtype", [F32, F64])
def test_gather_gradient_is_the_fixed_scatter(dev, dtype):
    # the gradient of values[index] accumulates out.grad rows sharing a source row through
    # det_scatter_add: bit-equal to the oracle, and the same over repeated backward passes
    rng = np.random.default_rng(11)
    src, m, d = 4096, 100003, 4
    vals = torch.from_numpy(rounding((src, d), dtype, 1)).to(dev).requires_grad_(True)
    idx_h = rng.integers(0, src, m).astype(np.int32)
    idx = torch.from_numpy(idx_h).to(dev)
    g_h = rounding((m, d), dtype, 2)
    g = torch.from_numpy(g_h).to(dev)
    out = det.gather(vals, idx)
    assert torch.equal(out, vals.detach()[idx.long()])
    grads = set()
    for _ in range(3):
        vals.grad = None
        det.gather(vals, idx).backward(g)
        grads.add(vals.grad.cpu().numpy().tobytes())
    assert len(grads) == 1
    want, _, _ = oracle.scatter_add(g_h, idx_h, np.zeros((src, d), dtype))
    assert bits_equal(vals.grad.cpu().numpy(), want)
    with pytest.raises(IndexError):
        det.gather(vals, torch.tensor([src], dtype=torch.int32, device=dev))


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("n,B", [(1000, 7), (300007, 1000), (70000, 1)])
def test_scatter_special_values(dev, dtype, n, B):
    # infinities, NaNs, signed zeros, subnormals and overflowing sums inside destinations, in
    # the old values too; add and subtract
    fi = np.finfo(dtype)
    rng = np.random.default_rng(n + B)
    v = rounding(n, dtype, n)
    pool = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, fi.tiny / 4, fi.max / 3, -fi.max / 3],
                    dtype)
    pos = rng.choice(n, size=max(1, n // 40), replace=False)
    v[pos] = pool[rng.integers(0, pool.size, pos.size)]
    idx = rng.integers(0, B, n).astype(np.int32)
    o = rounding(B, dtype, B)
    o[: min(B, 3)] = np.array([-0.0, np.inf, fi.tiny / 2], dtype)[: min(B, 3)]
    got, _, _ = gpu_scatter(v, idx, o, dev)
    want, _, _ = oracle.scatter_add(v, idx, o)
    assert bits_equal(got, want), first_mismatch(got, want)
    got, _, _ = gpu_scatter_sub(v, idx, o, dev)
    want, _, _ = oracle.scatter_sub(v, idx, o)
    assert bits_equal(got, want), first_mismatch(got, want)
