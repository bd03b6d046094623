"""The benchmark's non-deterministic comparison kernels compute what they claim (GPU).

The adaptive look-back scan (det_scan's kernel with the anchors replaced by the nearest
finished predecessor's inclusive prefix) must be a correct prefix sum in every mode, or its
timings would compare the library with something else.  On integer-valued data whose partial
sums are exact in the element type every bracketing gives the same numbers, so it must equal
the oracle bit for bit; on rounding data it must stay within the normwise bound of a
prefix sum of its depth.  The atomic sum and scatter are checked the same way on exact data.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from scan_fixed_order_amd import workloads

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
T = 8192
A = 256
MODES = [(False, False), (True, False), (False, True), (True, True)]


@pytest.fixture(scope="module")
def bl():
    lib = ctypes.CDLL(os.path.join(ROOT, "scan_fixed_order_amd", "libdet_baselines.so"))
    lib.detbase_adaptive_scan_workspace_size.restype = ctypes.c_size_t
    return lib


def adaptive(bl, x, exclusive=False, reverse=False, offsets=None):
    code = 0 if x.dtype == torch.float32 else 1
    nseg = 0 if offsets is None else offsets.numel() - 1
    n = x.numel()
    ws = torch.empty(bl.detbase_adaptive_scan_workspace_size(ctypes.c_int64(n), code,
                                                             ctypes.c_int64(nseg)),
                     dtype=torch.uint8, device=x.device)
    y = torch.empty_like(x)
    flags = (1 if exclusive else 0) | (2 if reverse else 0)
    st = bl.detbase_adaptive_scan(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                  ctypes.c_int64(n), code, flags,
                                  None if offsets is None else ctypes.c_void_p(offsets.data_ptr()),
                                  ctypes.c_int64(nseg), ctypes.c_void_p(ws.data_ptr()),
                                  ctypes.c_size_t(ws.numel()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    return y


def offsets_of(n, mean, seed):
    rng = np.random.default_rng(seed)
    cuts = np.concatenate([[0], np.cumsum(rng.geometric(1.0 / mean, size=n // mean + 64))])
    return np.concatenate([cuts[cuts < n], [n]]).astype(np.int64)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("n", [1, 8193, 164738, 3 * A * T + 5])
def test_adaptive_scan_exact_on_integer_data(dev, bl, dtype, n):
    rng = np.random.default_rng(n)
    x = rng.integers(-8, 9, n).astype(dtype)          # every partial sum exact (|s| < 2^24)
    offs = offsets_of(n, 1000, n)
    t = torch.from_numpy(x).to(dev)
    o = torch.from_numpy(offs).to(dev)
    for e, r in MODES:
        for seg in (False, True):
            got = adaptive(bl, t, e, r, o if seg else None).cpu().numpy()
            want = oracle.scan(x, exclusive=e, reverse=r, offsets=offs if seg else None)
            assert np.array_equal(got, want), (n, e, r, seg)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_adaptive_scan_error_bound_on_rounding_data(dev, bl, dtype):
    n = 3 * A * T + 5
    x = workloads.scan_values(n, dtype, seed=2)
    got = adaptive(bl, torch.from_numpy(x).to(dev)).cpu().numpy().astype(np.float64)
    ref = np.cumsum(x.astype(np.float64))
    norm = np.cumsum(np.abs(x.astype(np.float64)))
    u = np.finfo(dtype).eps / 2
    # lane run, wave, tile and look-back trees, combine; each tile's inclusive prefix may build
    # on a predecessor's, so the chain can add one level per tile
    depth = 32 + 6 + 2 + 9 + 4 + (n + T - 1) // T
    assert np.all(np.abs(got - ref) <= depth * u * norm + 1e-300)


def test_atomic_baselines_exact_on_integer_data(dev, bl):
    n, B = (1 << 20) + 7, 1000
    rng = np.random.default_rng(5)
    x = rng.integers(0, 4, n).astype(np.float32)
    b = rng.integers(0, B, n).astype(np.int32)
    xt = torch.from_numpy(x).to(dev)
    s = torch.zeros((), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert bl.detbase_atomic_sum(ctypes.c_void_p(xt.data_ptr()), ctypes.c_int64(n), 0,
                                 ctypes.c_void_p(s.data_ptr()), stream) == 0
    assert s.item() == float(x.sum(dtype=np.float64))
    out = torch.zeros(B, dtype=torch.float32, device=dev)
    bt = torch.from_numpy(b).to(dev)
    assert bl.detbase_atomic_scatter(ctypes.c_void_p(xt.data_ptr()), ctypes.c_void_p(bt.data_ptr()),
                                     ctypes.c_int64(n), 0, ctypes.c_void_p(out.data_ptr()),
                                     ctypes.c_int64(B), stream) == 0
    assert np.array_equal(out.cpu().numpy(), np.bincount(b, weights=x, minlength=B))
