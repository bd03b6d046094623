"""det_sum_noalloc, the entry point that allocates nothing, against det_sum (through the C ABI).

Two calls in a row on one stream, the second with a smaller input, must each give det_sum's
bits (and the oracle's): the second call reuses the per-GPU array the first one filled, so a
partial left over from the first would show.  Sizes take one and two levels of partials."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from scan_fixed_order_amd import det, workloads

pytestmark = pytest.mark.gpu

F32, F64 = np.float32, np.float64


def noalloc(x, out):
    lib = det.lib()
    code = det.DET_F32 if x.dtype == torch.float32 else det.DET_F64
    stream = ctypes.c_void_p(torch.cuda.current_stream(x.device).cuda_stream)
    return lib.det_sum_noalloc(ctypes.c_void_p(x.data_ptr()), x.numel(), code,
                               ctypes.c_void_p(out.data_ptr()), stream)


def bits(v, dtype):
    return np.asarray(v, dtype).view(np.int32 if dtype == F32 else np.int64)


@pytest.mark.parametrize("dtype", [F32, F64])
def test_noalloc_two_calls_match_det_sum(dev, dtype):
    tdt = torch.float32 if dtype == F32 else torch.float64
    for n in ((1 << 27) + 12345, 3_000_017, 100_003, 1):
        x = workloads.scan_values(n, dtype, seed=n % 1009)
        t = torch.from_numpy(x).to(dev)
        out = torch.full((), float("nan"), dtype=tdt, device=dev)
        assert noalloc(t, out) == 0
        ref = det.det_sum(t)
        got = out.cpu().numpy()
        assert bits(got, dtype) == bits(ref.cpu().numpy(), dtype), n
        assert bits(got, dtype) == bits(oracle.det_sum(x), dtype), n


def test_noalloc_empty_and_limits(dev):
    out = torch.full((), 7.0, dtype=torch.float32, device=dev)
    x = torch.empty(0, dtype=torch.float32, device=dev)
    assert noalloc(x, out) == 0
    got = out.cpu().numpy()
    assert got == 0.0 and not np.signbit(got)          # the empty sum is +0.0
    lib = det.lib()
    fake = ctypes.c_void_p(0x10000)
    assert lib.det_sum_noalloc(fake, (1 << 31), 0, fake, None) == 3     # TOO_LARGE
    assert lib.det_sum_noalloc(fake, -1, 0, fake, None) == 1            # INVALID_VALUE
    assert lib.det_sum_noalloc(fake, 10, 5, fake, None) == 2            # UNSUPPORTED


def test_noalloc_under_graph_capture(dev):
    # the callers it is for: a captured graph whose replays allocate nothing
    x = torch.from_numpy(workloads.uniform01(1 << 20, seed=0)).to(dev)
    out = torch.empty((), dtype=torch.float32, device=dev)
    want = det.det_sum(x).cpu().numpy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        assert noalloc(x, out) == 0
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert bits(out.cpu().numpy(), F32) == bits(want, F32)
