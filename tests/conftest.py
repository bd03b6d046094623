import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")


@pytest.fixture(autouse=True)
def _announce(request):
    # name the case on the real stderr before it runs, so a run that dies mid-test says where
    if request.node.get_closest_marker("gpu"):
        sys.__stderr__.write(f"\n[start] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield


@pytest.fixture(scope="session")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU (deselect with -m 'not gpu')")
    return torch.device("cuda:0")


def bits_equal(got, want):
    """Bitwise equality of two float arrays, NaN compared by class (payloads may differ)."""
    got = np.ascontiguousarray(got)
    want = np.ascontiguousarray(want)
    if got.shape != want.shape or got.dtype != want.dtype:
        return False
    gn, wn = np.isnan(got), np.isnan(want)
    if not np.array_equal(gn, wn):
        return False
    it = np.uint32 if got.dtype == np.float32 else np.uint64
    return np.array_equal(got.view(it)[~gn], want.view(it)[~wn])


def first_mismatch(got, want):
    got = np.ascontiguousarray(got).reshape(-1)
    want = np.ascontiguousarray(want).reshape(-1)
    it = np.uint32 if got.dtype == np.float32 else np.uint64
    bad = (got.view(it) != want.view(it)) & ~(np.isnan(got) & np.isnan(want))
    idx = np.flatnonzero(bad)
    if idx.size == 0:
        return "no mismatch"
    i = int(idx[0])
    return f"{idx.size} mismatches, first at {i}: got {got[i]!r} want {want[i]!r}"


def pw_ones(m, dtype):
    """The adjacent-pair tree's sum of m ones in dtype, in O(log m): by the split lemma
    PW(v) = PW(v[:2^k]) + PW(v[2^k:]) for 2^k < m <= 2^(k+1), and a full block of 2^k ones sums
    to 2^k exactly, so PW(ones(m)) = 2^k + PW(ones(m - 2^k)), folded right to left."""
    if m == 0:
        return dtype(-0.0)
    parts = []
    while True:
        k = 1 << (m.bit_length() - 1)
        if k == m:
            parts.append(dtype(m))
            break
        parts.append(dtype(k))
        m -= k
    acc = parts[-1]
    for p in reversed(parts[:-1]):
        acc = dtype(p + acc)
    return acc
