"""Launch shape, occupancy and observation order must not move a bit (GPU, through the C ABI).

* Grids of 1x, 2x and 4x the compute-unit count for the f64 sum and scan of 2^29 mixed-
  magnitude values, each at the default occupancy and with extra LDS per workgroup that
  lowers it; the launched grids and the scan's per-CU occupancy are read back from the
  library, so the test fails if the shapes it asks for were not the ones that ran.
* The look-back scan with seeded pauses before its status publications, so tiles find their
  predecessors' status words ready or not at different moments (drjit-core pull request "Make
  CUDA floating-point prefix sums deterministic", section "Root cause": the original kernel's
  bits depended on which predecessor states a block observed).  Every mode, plain and
  segmented, at three anchor intervals and with small anchor constants, five seeds.
* One result over 100 runs for every output element: each run compared with the first on the
  device, the first with the oracle.  At 2^28 (sum, scan in four modes, scatter-add) and at
  3 * 2^21 + 5 elements (the look-back kernel's path), f32 and f64, plain and small anchors.
* The non-temporal kernel variants (inputs of 512 MiB and more) on rounding-sensitive data:
  the f64 scan of 2^28 in every mode, segmented f64 at 2^26 and segmented f32 at 2^27.
* The health word: cleared by every launch path, whatever the workspace held before.
"""
import numpy as np
import pytest
import torch

import oracle
from scan_fixed_order_amd import det, workloads
from conftest import first_mismatch

pytestmark = pytest.mark.gpu

F32, F64 = np.float32, np.float64
T = 8192
A = 256
MODES = [(False, False), (True, False), (False, True), (True, True)]


def cu_count():
    return torch.cuda.get_device_properties(0).multi_processor_count


def ibits(t):
    """Integer view of a float tensor (bitwise comparison on the device)."""
    return t.view(torch.int64 if t.dtype == torch.float64 else torch.int32)


def dev_equal(got, want_dev):
    return torch.equal(ibits(got), ibits(want_dev))


def mismatch(got, want_np):
    return first_mismatch(got.cpu().numpy(), want_np)


def random_offsets(n, mean, seed):
    rng = np.random.default_rng(seed)
    lengths = rng.geometric(1.0 / mean, size=int(n / mean * 1.2) + 16)
    cuts = np.concatenate([[0], np.cumsum(lengths)])
    cuts = cuts[cuts < n]
    return np.concatenate([cuts, [n]]).astype(np.int64)


@pytest.fixture(autouse=True)
def _reset_hooks():
    yield
    det.det_debug_set_launch(0, 0)
    det.det_debug_set_scan_delay(0, 0)
    det.det_debug_set_scan_anchors(0, 0)


# ---------------------------------------------------------------- grids and occupancy

def test_f64_2_29_sum_and_scan_grids_and_occupancy(dev):
    n = 1 << 29
    x = workloads.mixed_f64(n, seed=4)
    want_sum = np.float64(oracle.det_sum(x))
    want_scan = oracle.scan(x)
    t = torch.from_numpy(x).to(dev)
    w = torch.from_numpy(want_scan).to(dev)
    del want_scan
    y = torch.empty_like(t)
    cus = cu_count()
    # f64 look-back workgroups hold about 69 KB of LDS, two per CU; 24 KB more leaves one
    lds_low = 24576
    shapes = [(cus, 0), (2 * cus, 0), (4 * cus, 0), (cus, lds_low), (2 * cus, lds_low),
              (4 * cus, lds_low), (0, lds_low)]
    grids, occupancy = set(), set()
    for grid, lds in shapes:
        det.det_debug_set_launch(grid, lds)
        s = det.det_sum(t).item()
        assert np.float64(s).view(np.int64) == want_sum.view(np.int64), (grid, lds, s, want_sum)
        det.det_scan(t, y=y, check=True)
        assert dev_equal(y, w), (grid, lds, "scan")
        last = det.det_debug_last_launch()
        if grid:
            assert last["scan_grid"] == grid and last["sum_grid"] == grid, (grid, lds, last)
        grids.add(last["scan_grid"])
        occupancy.add(last["scan_per_cu"])
    assert {cus, 2 * cus, 4 * cus} <= grids, grids
    assert len(occupancy) >= 2, occupancy            # the extra LDS really lowered it


@pytest.mark.parametrize("dtype", [F32, F64])
def test_look_back_grids_beyond_resident_and_low_occupancy(dev, dtype):
    n = 3 * A * T + 5
    x = workloads.scan_values(n, dtype, seed=16)
    offs = random_offsets(n, 500, seed=16)
    t = torch.from_numpy(x).to(dev)
    o = torch.from_numpy(offs).to(dev)
    cus = cu_count()
    wants = {(e, r, s): torch.from_numpy(oracle.scan(x, exclusive=e, reverse=r,
                                                     offsets=offs if s else None)).to(dev)
             for e, r in MODES for s in (False, True)}
    y = torch.empty_like(t)
    occupancy = set()
    for grid, lds in ((1, 0), (13, 0), (cus, 0), (4 * cus, 0), (16 * cus, 0), (0, 40000),
                      (4 * cus, 40000), (0, 65536)):
        det.det_debug_set_launch(grid, lds)
        for (e, r, s), w in wants.items():
            det.det_scan(t, y=y, exclusive=e, reverse=r, offsets=o if s else None, check=True)
            assert dev_equal(y, w), (grid, lds, e, r, s)
            if grid:
                assert det.det_debug_last_launch()["scan_grid"] == grid
        occupancy.add(det.det_debug_last_launch()["scan_per_cu"])
    assert len(occupancy) >= 2, occupancy


def test_scatter_radix_occupancy(dev):
    # extra LDS on the radix-sort kernels (one workgroup per CU instead of two): same bits
    n, B = (1 << 22) + 3, 65536
    v = workloads.normal(n, seed=21)
    b = workloads.bins_uniform(n, B, seed=21)
    want, _, _ = oracle.scatter_add(v, b, np.zeros(B, F32))
    vt, bt = torch.from_numpy(v).to(dev), torch.from_numpy(b).to(dev)
    wt = torch.from_numpy(want).to(dev)
    for lds in (0, 8192, 65536):
        det.det_debug_set_launch(0, lds)
        out = torch.zeros(B, dtype=torch.float32, device=dev)
        det.det_scatter_add(vt, bt, out)
        assert dev_equal(out, wt), lds


# ---------------------------------------------------------------- forced observation orders

@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("n,anchors", [(3 * A * T + 5, (0, 0)), (37 * T + 123, (2, 3)),
                                       (400 * T + 77, (4, 3))])
def test_seeded_publication_delays(dev, dtype, n, anchors):
    x = workloads.scan_values(n, dtype, seed=n % 101)
    offs = random_offsets(n, 3000, seed=n % 89)
    t = torch.from_numpy(x).to(dev)
    o = torch.from_numpy(offs).to(dev)
    Aa, A2a = anchors
    kw = {} if not Aa else {"A": Aa, "A2": A2a}
    wants = {(e, r, s): torch.from_numpy(oracle.scan(x, exclusive=e, reverse=r,
                                                     offsets=offs if s else None, **kw)).to(dev)
             for e, r in MODES for s in (False, True)}
    det.det_debug_set_scan_anchors(Aa, A2a)
    y = torch.empty_like(t)
    for seed in range(1, 6):
        det.det_debug_set_scan_delay(seed * 7919, 20)
        det.det_debug_set_launch(4 * cu_count() if seed == 5 else 0, 0)
        for (e, r, s), w in wants.items():
            det.det_scan(t, y=y, exclusive=e, reverse=r, offsets=o if s else None, check=True)
            assert dev_equal(y, w), (seed, e, r, s)


# ---------------------------------------------------------------- 100 runs, every output

def hundred_runs(fn, runs=100):
    """Run fn (returning a device tensor) `runs` times; every run bit-equal to the first."""
    first = fn().clone()
    for i in range(1, runs):
        assert dev_equal(fn(), first), i
    return first


def test_hundred_runs_every_output_2_28(dev):
    n = 1 << 28
    xs = workloads.uniform01(n, seed=0)
    want = np.float32(oracle.det_sum(xs))
    t = torch.from_numpy(xs).to(dev)
    out = torch.empty((), dtype=torch.float32, device=dev)
    first = hundred_runs(lambda: det.det_sum(t, out=out))
    assert first.cpu().numpy().view(np.int32) == want.view(np.int32)
    del t, xs
    x = workloads.scan_values(n, F32, seed=2)
    t = torch.from_numpy(x).to(dev)
    y = torch.empty_like(t)
    h = torch.empty((), dtype=torch.int32, device=dev)
    for e, r in MODES:
        w = torch.from_numpy(oracle.scan(x, exclusive=e, reverse=r)).to(dev)

        def run():
            det.det_scan(t, y=y, exclusive=e, reverse=r, health=h)
            assert int(h.item()) == 0
            return y

        first = hundred_runs(run)
        assert dev_equal(first, w), (e, r)
        del w
    del t, y, x
    v = workloads.normal(n, seed=1)
    b = workloads.bins_uniform(n, 65536, seed=1)
    want, _, _ = oracle.scatter_add(v, b, np.zeros(65536, F32))
    vt, bt = torch.from_numpy(v).to(dev), torch.from_numpy(b).to(dev)
    o = torch.zeros(65536, dtype=torch.float32, device=dev)

    def scat():
        o.zero_()
        return det.det_scatter_add(vt, bt, o)

    first = hundred_runs(scat)
    assert dev_equal(first, torch.from_numpy(want).to(dev))


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("anchors", [(0, 0), (2, 2)])
def test_hundred_runs_every_output_look_back(dev, dtype, anchors):
    n = 3 * A * T + 5
    x = workloads.scan_values(n, dtype, seed=2)
    offs = random_offsets(n, 100, seed=2)
    t = torch.from_numpy(x).to(dev)
    o = torch.from_numpy(offs).to(dev)
    Aa, A2a = anchors
    kw = {} if not Aa else {"A": Aa, "A2": A2a}
    det.det_debug_set_scan_anchors(Aa, A2a)
    y = torch.empty_like(t)
    h = torch.empty((), dtype=torch.int32, device=dev)
    for e, r in MODES:
        for seg in (False, True):
            def run():
                det.det_scan(t, y=y, exclusive=e, reverse=r, offsets=o if seg else None, health=h)
                return y

            first = hundred_runs(run)
            assert int(h.item()) == 0
            want = oracle.scan(x, exclusive=e, reverse=r, offsets=offs if seg else None, **kw)
            assert dev_equal(first, torch.from_numpy(want).to(dev)), (e, r, seg,
                                                                      mismatch(first, want))


# ---------------------------------------------------------------- non-temporal variants

@pytest.mark.parametrize("excl,rev", MODES)
def test_scan_f64_2_28_every_mode(dev, excl, rev):
    n = 1 << 28
    x = workloads.scan_values(n, F64, seed=2)
    t = torch.from_numpy(x).to(dev)
    want = oracle.scan(x, exclusive=excl, reverse=rev)
    got = det.det_scan(t, exclusive=excl, reverse=rev, check=True)
    assert dev_equal(got, torch.from_numpy(want).to(dev)), mismatch(got, want)


@pytest.mark.parametrize("dtype,log2n", [(F64, 26), (F32, 27)])
def test_segmented_scan_at_512_mib(dev, dtype, log2n):
    # 512 MiB of input: the non-temporal kernel variants, with segments (mean length 100)
    n = 1 << log2n
    x = workloads.scan_values(n, dtype, seed=3)
    offs = workloads.segment_offsets(n, 100.0, seed=3)
    t = torch.from_numpy(x).to(dev)
    o = torch.from_numpy(offs).to(dev)
    for excl, rev in MODES:
        want = oracle.scan(x, exclusive=excl, reverse=rev, offsets=offs)
        got = det.det_scan(t, exclusive=excl, reverse=rev, offsets=o, check=True)
        assert dev_equal(got, torch.from_numpy(want).to(dev)), (excl, rev, mismatch(got, want))


# ---------------------------------------------------------------- the health word

@pytest.mark.parametrize("n", [100, 2 * T, 200 * T + 1, 3 * A * T + 5])
def test_health_word_cleared_on_every_path(dev, n):
    # a workspace full of ones before the scan: one tile (one launch), a few tiles (two
    # launches that never wait), the look-back kernel; each leaves the word at 0
    x = torch.from_numpy(workloads.scan_values(n, F32, seed=4)).to(dev)
    ws = torch.full((det.det_scan_workspace_size(n, 0, 3, 0),), 255, dtype=torch.uint8,
                    device=dev)
    det.det_scan(x, ws=ws, check=True)
    assert int(det.det_scan_error(ws).item()) == 0, n
