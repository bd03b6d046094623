"""The measured workloads at their full sizes, bit for bit against the oracle (through the C
interface), plus one SHA-256 over 100 repeated runs for each operation.

Sizes follow the benchmark and the configurations it stands for: f32 sum, inclusive and
exclusive scans (both directions) and scatter-add into 65,536 uniform bins at n = 2^28; the
segmented scan at 2^26 with geometric segment lengths of mean 100, and the f64 scatter-add of
2^29 mixed-magnitude values (binary exponents in [-30, 30]) into 2^20 Zipf(1.1) bins.  The
f64 sum and scan of those 2^29 values, across launch grids and occupancies, are in
test_gpu_invariance.py.  The large cases run
the single-threaded oracle for tens of seconds each.
"""
import hashlib

import numpy as np
import pytest
import torch

import oracle
from scan_fixed_order_amd import det, workloads
from conftest import bits_equal, first_mismatch

pytestmark = pytest.mark.gpu

F32, F64 = np.float32, np.float64


@pytest.fixture(scope="module")
def scan_2_28():
    return workloads.scan_values(1 << 28, F32, seed=2)


@pytest.fixture(scope="module")
def mixed_2_29():
    return workloads.mixed_f64(1 << 29, seed=4)


def cu_count():
    return torch.cuda.get_device_properties(0).multi_processor_count


def sha_runs(fn, runs=100):
    """SHA-256 of each run's output bytes; the set must hold one digest."""
    return {hashlib.sha256(fn().cpu().numpy().tobytes()).hexdigest() for _ in range(runs)}


def test_sum_f32_2_28(dev):
    x = workloads.uniform01(1 << 28, seed=0)
    got = det.det_sum(torch.from_numpy(x).to(dev)).cpu().numpy()
    assert bits_equal(got.reshape(1), np.array([oracle.det_sum(x)], F32))


@pytest.mark.parametrize("excl,rev", [(False, False), (True, False), (False, True), (True, True)])
def test_scan_f32_2_28(dev, scan_2_28, excl, rev):
    x = scan_2_28
    t = torch.from_numpy(x).to(dev)
    got = det.det_scan(t, exclusive=excl, reverse=rev, check=True).cpu().numpy()
    want = oracle.scan(x, exclusive=excl, reverse=rev)
    assert bits_equal(got, want), first_mismatch(got, want)


@pytest.mark.parametrize("excl,rev", [(False, True), (True, False)])
def test_scan_unaligned_views_above_512_mib(dev, scan_2_28, excl, rev):
    # inputs of 512 MiB and more take non-temporal loads: views of 2^27 + 5 f32 elements at
    # element offsets 1 (input) and 2 (output)
    n = (1 << 27) + 5
    xs = scan_2_28[1:1 + n]
    t = torch.from_numpy(scan_2_28[: n + 4]).to(dev)
    yb = torch.empty(n + 4, dtype=torch.float32, device=dev)
    y = yb[2:2 + n]
    det.det_scan(t[1:1 + n], y=y, exclusive=excl, reverse=rev, check=True)
    want = oracle.scan(xs, exclusive=excl, reverse=rev)
    got = y.cpu().numpy()
    assert bits_equal(got, want), first_mismatch(got, want)


def test_scatter_f32_2_28_65536_bins(dev):
    n, B = 1 << 28, 65536
    v = workloads.normal(n, seed=1)
    b = workloads.bins_uniform(n, B, seed=1)
    out = torch.zeros(B, dtype=torch.float32, device=dev)
    det.det_scatter_add(torch.from_numpy(v).to(dev), torch.from_numpy(b).to(dev), out)
    want, _, _ = oracle.scatter_add(v, b, np.zeros(B, F32))
    got = out.cpu().numpy()
    assert bits_equal(got, want), first_mismatch(got, want)


@pytest.mark.parametrize("excl,rev", [(False, False), (True, False), (False, True), (True, True)])
def test_segmented_scan_f32_2_26(dev, excl, rev):
    n = 1 << 26
    x = workloads.scan_values(n, F32, seed=3)
    offs = workloads.segment_offsets(n, 100.0, seed=3)
    got = det.det_scan(torch.from_numpy(x).to(dev), exclusive=excl, reverse=rev,
                       offsets=torch.from_numpy(offs).to(dev), check=True).cpu().numpy()
    want = oracle.scan(x, exclusive=excl, reverse=rev, offsets=offs)
    assert bits_equal(got, want), first_mismatch(got, want)


def test_scatter_f64_2_29_zipf_2_20_bins(dev, mixed_2_29):
    n, B = 1 << 29, 1 << 20
    v = mixed_2_29
    b = workloads.zipf_bins(n, B, seed=4)
    vt, bt = torch.from_numpy(v).to(dev), torch.from_numpy(b).to(dev)
    outs = []
    for _ in range(2):
        out = torch.zeros(B, dtype=torch.float64, device=dev)
        det.det_scatter_add(vt, bt, out)
        outs.append(out.cpu().numpy())
    want, _, _ = oracle.scatter_add(v, b, np.zeros(B, F64))
    assert bits_equal(outs[0], want), first_mismatch(outs[0], want)
    assert bits_equal(outs[1], want)


def test_hundred_runs_one_hash(dev):
    # sum (n = 2^20, the measured configuration), scan (the drjit-core regression size and
    # 1,048,577, all modes) and scatter-add (2^24 values into 65,536 bins, and all into bin 0)
    x = torch.from_numpy(workloads.uniform01(1 << 20, seed=0)).to(dev)
    out = torch.empty((), dtype=torch.float32, device=dev)
    assert len(sha_runs(lambda: det.det_sum(x, out=out))) == 1
    for n in (164738, 1048577):
        s = torch.from_numpy(workloads.scan_values(n, F32, seed=2)).to(dev)
        y = torch.empty_like(s)
        for excl in (False, True):
            for rev in (False, True):
                assert len(sha_runs(lambda: det.det_scan(s, y=y, exclusive=excl,
                                                         reverse=rev, check=True))) == 1, (n, excl, rev)
    v = torch.from_numpy(workloads.normal(1 << 24, seed=1)).to(dev)
    for b in (workloads.bins_uniform(1 << 24, 65536, seed=1), np.zeros(1 << 24, np.int32)):
        bt = torch.from_numpy(b).to(dev)
        o = torch.zeros(65536, dtype=torch.float32, device=dev)

        def run():
            o.zero_()
            return det.det_scatter_add(v, bt, o)

        assert len(sha_runs(run)) == 1
