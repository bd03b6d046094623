"""det_scan on the GPU against the oracle, bit for bit (through the C interface).

Sizes straddle lanes (32), waves (2048), tiles (8192) and anchor intervals (256 tiles), in
f32 and f64, inclusive/exclusive x forward/reverse x full/segmented (drjit-core pull request
"Make CUDA floating-point prefix sums deterministic", "Validation": the same matrix, and 20
repeated scans of 164,738 elements).  Also: in-place scans, unaligned views, empty segments,
and grid caps that must not move a bit.
"""
import numpy as np
import pytest
import torch

import oracle
from scan_fixed_order_amd import det, workloads
from conftest import bits_equal, first_mismatch

pytestmark = pytest.mark.gpu

F32, F64 = np.float32, np.float64
T = 8192
A = 256
MODES = [(False, False), (True, False), (False, True), (True, True)]


def gpu_scan(x, dev, exclusive=False, reverse=False, offsets=None):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    o = None if offsets is None else torch.from_numpy(np.asarray(offsets, np.int64)).to(dev)
    return det.det_scan(t, exclusive=exclusive, reverse=reverse, offsets=o, check=True).cpu().numpy()


def random_offsets(n, mean, seed, empty_every=0):
    rng = np.random.default_rng(seed)
    cuts = [0]
    while cuts[-1] < n:
        cuts.append(min(n, cuts[-1] + int(rng.geometric(1.0 / mean))))
        if empty_every and len(cuts) % empty_every == 0:
            cuts.append(cuts[-1])                    # an empty segment
    return np.array(cuts, np.int64)


SIZES = [1, 31, 32, 33, 2047, 2048, 2049, 8191, 8192, 8193, 16384, 164738, 1048577,
         A * T + 1, 3 * A * T + 5]


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("n", SIZES)
def test_scan_parity_all_modes(dev, dtype, n):
    x = workloads.scan_values(n, dtype, seed=n % 97)
    for excl, rev in MODES:
        got = gpu_scan(x, dev, excl, rev)
        want = oracle.scan(x, exclusive=excl, reverse=rev)
        assert bits_equal(got, want), (n, excl, rev, first_mismatch(got, want))


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("n,mean", [(1, 5), (100, 3), (8193, 40), (164738, 100),
                                    (1048577, 5000), (A * T + 77, 100), (3 * A * T + 5, 1e6)])
def test_segmented_parity(dev, dtype, n, mean):
    x = workloads.scan_values(n, dtype, seed=3)
    offs = random_offsets(n, mean, seed=n, empty_every=7)
    for excl, rev in MODES:
        got = gpu_scan(x, dev, excl, rev, offs)
        want = oracle.scan(x, exclusive=excl, reverse=rev, offsets=offs)
        assert bits_equal(got, want), (n, excl, rev, first_mismatch(got, want))


def test_segment_edge_layouts(dev):
    n = 3 * T + 17
    x = workloads.scan_values(n, F32, seed=11)
    layouts = [
        np.array([0, n]),                                        # one segment
        np.arange(0, n + 1),                                     # every element a head
        np.array([0, 0, 0, n, n]),                               # empty segments at both ends
        np.array([0, T - 1, T, T + 1, 2 * T, n]),                # heads around tile borders
        np.concatenate([[0], np.arange(32, n, 32), [n]]),        # heads at lane starts
        np.concatenate([np.repeat(np.arange(0, n, 3), 2), [n]]),  # every offset twice (empty
                                                                  # segments between dense heads)
    ]
    for offs in layouts:
        for excl, rev in MODES:
            got = gpu_scan(x, dev, excl, rev, offs)
            want = oracle.scan(x, exclusive=excl, reverse=rev, offsets=offs)
            assert bits_equal(got, want), (offs[:6], excl, rev, first_mismatch(got, want))


@pytest.mark.parametrize("n", [1, 8193, 3 * A * T + 5])
def test_all_ones_exact(dev, n):
    x = np.ones(n, F32)
    i = np.arange(n, dtype=np.float64)
    assert np.array_equal(gpu_scan(x, dev), i + 1)
    assert np.array_equal(gpu_scan(x, dev, exclusive=True), i)
    assert np.array_equal(gpu_scan(x, dev, reverse=True), n - i)
    assert np.array_equal(gpu_scan(x, dev, exclusive=True, reverse=True), n - 1 - i)


@pytest.mark.parametrize("dtype", [F32, F64])
def test_repeat_164738_twenty_times(dev, dtype):
    # the regression size of the drjit-core pull request, repeated 20 times per mode
    x = workloads.scan_values(164738, dtype, seed=2)
    t = torch.from_numpy(x).to(dev)
    for excl, rev in MODES:
        want = oracle.scan(x, exclusive=excl, reverse=rev)
        outs = [det.det_scan(t, exclusive=excl, reverse=rev, check=True) for _ in range(20)]
        for o in outs:
            assert bits_equal(o.cpu().numpy(), want), (excl, rev)


@pytest.mark.parametrize("dtype", [F32, F64])
def test_in_place_and_unaligned(dev, dtype):
    n = 2 * A * T + 333
    x = workloads.scan_values(n, dtype, seed=5)
    want = oracle.scan(x)
    t = torch.from_numpy(x).to(dev)
    det.det_scan(t, y=t, check=True)                                     # inclusive in place
    assert bits_equal(t.cpu().numpy(), want)
    t = torch.from_numpy(x).to(dev)
    for k in (1, 3):
        for excl, rev in MODES:
            got = det.det_scan(t[k:], exclusive=excl, reverse=rev, check=True).cpu().numpy()
            assert bits_equal(got, oracle.scan(x[k:], exclusive=excl, reverse=rev)), (k, excl, rev)


@pytest.mark.parametrize("dtype", [F32, F64])
def test_grid_invariance(dev, dtype):
    n = 3 * A * T + 5
    x = workloads.scan_values(n, dtype, seed=6)
    offs = random_offsets(n, 3000, seed=1)
    t = torch.from_numpy(x).to(dev)
    o = torch.from_numpy(offs).to(dev)
    want = oracle.scan(x)
    wseg = oracle.scan(x, offsets=offs, reverse=True)
    try:
        for grid in (1, 2, 7, 64, 256, 1000):
            det.det_debug_set_launch(grid, 0)
            assert bits_equal(det.det_scan(t, check=True).cpu().numpy(), want), grid
            assert bits_equal(det.det_scan(t, offsets=o, reverse=True, check=True).cpu().numpy(), wseg), grid
    finally:
        det.det_debug_set_launch(0, 0)


def test_empty_scan(dev):
    t = torch.empty(0, device=dev)
    assert det.det_scan(t, check=True).numel() == 0
    assert det.det_scan(t, exclusive=True, offsets=torch.zeros(1, dtype=torch.int64,
                                                               device=dev), check=True).numel() == 0


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("A,A2", [(1, 1), (2, 3), (3, 2), (256, 1), (1, 256), (7, 5)])
def test_small_anchor_variants(dev, dtype, A, A2):
    # many anchor intervals and super-interval carries at small n: the kernel run with anchor
    # constants (A, A2) against the oracle run with the same constants
    n = 37 * T + 123
    x = workloads.scan_values(n, dtype, seed=A * 10 + A2)
    offs = random_offsets(n, 20000, seed=A + A2)
    t = torch.from_numpy(x).to(dev)
    o = torch.from_numpy(offs).to(dev)
    try:
        det.det_debug_set_scan_anchors(A, A2)
        for grid in (0, 1, 3):
            det.det_debug_set_launch(grid, 0)
            for excl, rev in MODES:
                got = det.det_scan(t, exclusive=excl, reverse=rev, check=True).cpu().numpy()
                want = oracle.scan(x, exclusive=excl, reverse=rev, A=A, A2=A2)
                assert bits_equal(got, want), (grid, excl, rev, first_mismatch(got, want))
                got = det.det_scan(t, exclusive=excl, reverse=rev, offsets=o, check=True).cpu().numpy()
                want = oracle.scan(x, exclusive=excl, reverse=rev, offsets=offs, A=A, A2=A2)
                assert bits_equal(got, want), (grid, excl, rev, "seg", first_mismatch(got, want))
    finally:
        det.det_debug_set_scan_anchors(0, 0)
        det.det_debug_set_launch(0, 0)


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("A,A2", [(2, 2), (4, 3)])
def test_many_super_intervals_on_a_full_grid(dev, dtype, A, A2):
    # Hundreds of super-interval carries with the full persistent grid: a workgroup's next tile
    # is often the last of a later interval, so the carry must not wait behind that tile's
    # local step (it once did, and about 1% of the scans of 2^31 - 1 f64 elements stalled
    # until the bounded wait gave up).  Bits against the oracle, and a clear health word.
    n = 1500 * T + 77
    x = workloads.scan_values(n, dtype, seed=A * 7 + A2)
    t = torch.from_numpy(x).to(dev)
    code = 0 if dtype == F32 else 1
    try:
        det.det_debug_set_scan_anchors(A, A2)
        for excl, rev in ((False, False), (True, True)):
            flags = (1 if excl else 0) | (2 if rev else 0)
            ws = torch.empty(det.det_scan_workspace_size(n, code, flags, 0), dtype=torch.uint8,
                             device=dev)
            got = det.det_scan(t, exclusive=excl, reverse=rev, ws=ws, check=True).cpu().numpy()
            assert int(det.det_scan_error(ws).item()) == 0, (A, A2, excl, rev, "health word")
            want = oracle.scan(x, exclusive=excl, reverse=rev, A=A, A2=A2)
            assert bits_equal(got, want), (A, A2, excl, rev, first_mismatch(got, want))
    finally:
        det.det_debug_set_scan_anchors(0, 0)


@pytest.mark.parametrize("dtype", [F32, F64])
def test_exclusive_into_unaligned_output(dev, dtype):
    # the exclusive readout aligns its 16-byte stores to y's address: y views at every
    # element offset within 16 bytes, both directions, ragged n
    n = 2 * A * T // 64 + 4099
    x = workloads.scan_values(n, dtype, seed=8)
    offs = random_offsets(n, 700, seed=8)
    t = torch.from_numpy(x).to(dev)
    o = torch.from_numpy(offs).to(dev)
    buf = torch.empty(n + 8, dtype=t.dtype, device=dev)
    for k in range(4):
        for rev in (False, True):
            y = buf[k:k + n]
            det.det_scan(t, y=y, exclusive=True, reverse=rev, check=True)
            want = oracle.scan(x, exclusive=True, reverse=rev)
            assert bits_equal(y.cpu().numpy(), want), (k, rev, first_mismatch(y.cpu().numpy(), want))
            det.det_scan(t, y=y, exclusive=True, reverse=rev, offsets=o, check=True)
            want = oracle.scan(x, exclusive=True, reverse=rev, offsets=offs)
            assert bits_equal(y.cpu().numpy(), want), (k, rev, "seg")


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("n", [5 * T + 77, 2 * A * T + 333])
def test_unaligned_input_and_output(dev, dtype, n):
    # x and y views at independent element offsets within 16 bytes: each wave's coalesced
    # loads take the aligned interior and load the elements around it one per lane, and the
    # readout aligns its stores to y; both launch paths (a few tiles, and more than one anchor
    # interval), every mode, with and without segments
    x = workloads.scan_values(n + 4, dtype, seed=n % 97)
    offs = random_offsets(n, 900, seed=n % 89)
    xb = torch.from_numpy(x).to(dev)
    o = torch.from_numpy(offs).to(dev)
    yb = torch.empty(n + 4, dtype=xb.dtype, device=dev)
    for kx, ky in ((1, 0), (2, 0), (3, 0), (0, 2), (1, 3), (2, 1), (3, 3)):
        xs = x[kx:kx + n]
        for excl, rev in MODES:
            for seg in (None, offs):
                y = yb[ky:ky + n]
                y.fill_(float("nan"))
                det.det_scan(xb[kx:kx + n], y=y, exclusive=excl, reverse=rev,
                             offsets=o if seg is not None else None, check=True)
                want = oracle.scan(xs, exclusive=excl, reverse=rev, offsets=seg)
                got = y.cpu().numpy()
                assert bits_equal(got, want), (kx, ky, excl, rev, seg is not None,
                                               first_mismatch(got, want))


@pytest.mark.parametrize("dtype", [F32, F64])
def test_scan_health_word_stays_clear(dev, dtype):
    # every look-back wait of these scans ends normally: the workspace's health word reads 0
    n = 5 * A * T + 77
    x = workloads.scan_values(n, dtype, seed=9)
    offs = random_offsets(n, 900, seed=9)
    t = torch.from_numpy(x).to(dev)
    o = torch.from_numpy(offs).to(dev)
    code = det.DET_F32 if dtype == F32 else det.DET_F64
    ws = torch.empty(det.det_scan_workspace_size(n, code, 3, len(offs) - 1), dtype=torch.uint8,
                     device=dev)
    for excl, rev in MODES:
        for seg in (None, o):
            det.det_scan(t, exclusive=excl, reverse=rev, offsets=seg, ws=ws, check=True)
            assert int(det.det_scan_error(ws).item()) == 0, (excl, rev, seg is not None)


# ---------------------------------------------------------------- int32 (slot allocation)

@pytest.mark.parametrize("n", [1, 7, 8192, 8193, 164738, 1048577, 2 * 256 * 8192 + 5])
def test_int32_scan_parity(dev, n):
    rng = np.random.default_rng(n)
    x = rng.integers(-2 ** 31, 2 ** 31, n).astype(np.int32)     # sums wrap
    offs = random_offsets(n, max(1, n // 50), seed=n)
    t = torch.from_numpy(x).to(dev)
    o = torch.from_numpy(offs).to(dev)
    for excl, rev in MODES:
        got = det.det_scan(t, exclusive=excl, reverse=rev, check=True).cpu().numpy()
        assert np.array_equal(got, oracle.scan_int32(x, excl, rev)), (excl, rev)
        got = det.det_scan(t, exclusive=excl, reverse=rev, offsets=o, check=True).cpu().numpy()
        assert np.array_equal(got, oracle.scan_int32(x, excl, rev, offs)), (excl, rev, "seg")


def test_count_scan_write_compaction(dev):
    # Warp "Deterministic Execution", Pattern 2: slot = atomic_add(count, 0, 1) for every
    # positive value becomes count (1 or 0 per thread), exclusive scan (the slot), write.  The
    # compacted array keeps thread order, the same on every run.
    rng = np.random.default_rng(3)
    n = 1_000_003
    v = rng.standard_normal(n).astype(np.float32)
    vt = torch.from_numpy(v).to(dev)
    outs = set()
    for _ in range(3):
        want = (vt > 0).to(torch.int32)
        slot = det.det_scan(want, exclusive=True, check=True)
        total = int(slot[-1].item() + want[-1].item())
        comp = torch.empty(total, dtype=torch.float32, device=dev)
        keep = want.bool()
        comp[slot[keep].long()] = vt[keep]
        outs.add(comp.cpu().numpy().tobytes())
    assert len(outs) == 1
    assert np.array_equal(np.frombuffer(outs.pop(), np.float32), v[v > 0])


# ---------------------------------------------------------------- special values

def special_values(n, dtype, seed):
    # mixed-magnitude values with infinities, NaNs, signed zeros, subnormals and values that
    # overflow when summed, spread across tiles, waves and lanes
    fi = np.finfo(dtype)
    rng = np.random.default_rng(seed)
    x = workloads.scan_values(n, dtype, seed=seed)
    pool = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, fi.tiny / 4, -fi.tiny / 8,
                     fi.max / 3, -fi.max / 3, fi.eps, 1.0], dtype)
    pos = rng.choice(n, size=max(1, n // 50), replace=False)
    x[pos] = pool[rng.integers(0, pool.size, pos.size)]
    return x


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("n", [33, 8193, 3 * 8192 + 17, 300007])
def test_scan_special_values(dev, dtype, n):
    x = special_values(n, dtype, seed=n)
    offs = random_offsets(n, 700, seed=n + 1)
    t = torch.from_numpy(x).to(dev)
    o = torch.from_numpy(offs).to(dev)
    for excl, rev in MODES:
        got = det.det_scan(t, exclusive=excl, reverse=rev, check=True).cpu().numpy()
        want = oracle.scan(x, exclusive=excl, reverse=rev)
        assert bits_equal(got, want), (excl, rev, first_mismatch(got, want))
        got = det.det_scan(t, exclusive=excl, reverse=rev, offsets=o, check=True).cpu().numpy()
        want = oracle.scan(x, exclusive=excl, reverse=rev, offsets=offs)
        assert bits_equal(got, want), (excl, rev, "seg", first_mismatch(got, want))


@pytest.mark.parametrize("dtype", [F32, F64])
def test_scan_all_negative_zero(dev, dtype):
    # -0.0 + -0.0 = -0.0 all along; the exclusive scan starts at +0.0
    n = 3 * 8192 + 5
    x = np.full(n, -0.0, dtype)
    t = torch.from_numpy(x).to(dev)
    for excl, rev in MODES:
        got = det.det_scan(t, exclusive=excl, reverse=rev, check=True).cpu().numpy()
        assert bits_equal(got, oracle.scan(x, exclusive=excl, reverse=rev))
        first = got[-1] if rev else got[0]
        assert np.signbit(first) == (not excl)
