"""The largest size the interface accepts, n = DET_MAX_N = 2^31 - 1, on the GPU.

The oracle would need minutes and tens of GB of host memory here, so the expected values are
closed forms that follow from the spec, computed independently of both the library and the
oracle:

* the sum of m ones: PW splits at the largest power of two 2^k below m (padding lemma and
  split lemma of the adjacent-pair tree), and a full block of 2^k ones sums to 2^k exactly, so
  PW(ones(m)) = 2^k + PW(ones(m - 2^k)) in the element type, folded right to left;
* scans of ones in f64 and int32: every partial sum is an exact integer (below 2^53), so the
  inclusive scan is i + 1, the exclusive i, reversed n - i and n - 1 - i;
* the scatter of ones with index i mod 65,536: destination b receives
  floor((n - 1 - b) / 65536) + 1 ones, an exact integer, added to +0.0.

Inputs are made and checked on the device in slices, so host memory stays small.
"""
import numpy as np
import pytest
import torch

from scan_fixed_order_amd import det
from conftest import pw_ones

pytestmark = pytest.mark.gpu

NMAX = 2 ** 31 - 1
SLICE = 1 << 27


def test_max_n_sum_of_ones(dev):
    x = torch.ones(NMAX, dtype=torch.float32, device=dev)
    got = det.det_sum(x).item()
    want = pw_ones(NMAX, np.float32)
    assert np.float32(got).view(np.uint32) == want.view(np.uint32), (got, want)
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [torch.float64, torch.int32])
def test_max_n_scan_of_ones(dev, dtype):
    x = torch.ones(NMAX, dtype=dtype, device=dev)
    y = torch.empty_like(x)
    code = 1 if dtype == torch.float64 else 2
    for excl, rev in ((False, False), (True, False), (False, True), (True, True)):
        flags = (1 if excl else 0) | (2 if rev else 0)
        ws = torch.empty(det.det_scan_workspace_size(NMAX, code, flags, 0), dtype=torch.uint8,
                         device=dev)
        det.det_scan(x, y=y, exclusive=excl, reverse=rev, ws=ws)
        # every bounded wait of the scan ended normally
        assert int(det.det_scan_error(ws).item()) == 0, (dtype, excl, rev, "health word")
        for a in range(0, NMAX, SLICE):
            b = min(NMAX, a + SLICE)
            i = torch.arange(a, b, dtype=torch.int64, device=dev)
            want = (NMAX - i if rev else i + 1) - (1 if excl else 0)
            got = y[a:b].to(torch.int64)
            if not torch.equal(got, want):
                bad = torch.nonzero(got != want).flatten()
                k = int(bad[0])
                raise AssertionError((dtype, excl, rev, "slice", a, "mismatches", bad.numel(),
                                      "first index", a + k, "got", int(got[k]), "want",
                                      int(want[k]), "last index", a + int(bad[-1])))
        del ws
    del x, y
    torch.cuda.empty_cache()


def test_max_n_scatter_of_ones(dev):
    B = 65536
    v = torch.ones(NMAX, dtype=torch.float32, device=dev)
    idx = torch.empty(NMAX, dtype=torch.int32, device=dev)
    for a in range(0, NMAX, SLICE):
        b = min(NMAX, a + SLICE)
        idx[a:b] = (torch.arange(a, b, dtype=torch.int64, device=dev) % B).to(torch.int32)
    out = torch.zeros(B, dtype=torch.float32, device=dev)
    sk = torch.full((1,), -1, dtype=torch.int64, device=dev)
    det.det_scatter_add(v, idx, out, n_skipped=sk)
    bins = torch.arange(B, dtype=torch.int64, device=dev)
    want = ((NMAX - 1 - bins) // B + 1).to(torch.float32)
    assert torch.equal(out, want) and int(sk.item()) == 0
    del v, idx
    torch.cuda.empty_cache()
