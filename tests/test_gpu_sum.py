"""det_sum on the GPU against the oracle, bit for bit (through the C interface).

Covers ragged sizes around the kernel's blocks (256), wave steps (4096), workgroup steps
(16384) and levels, special values, unaligned views, repeated runs hashed, and launch-shape
changes (grid caps and partial-chunk sizes) that must not move a bit.
"""
import hashlib

import numpy as np
import pytest
import torch

import oracle
from scan_fixed_order_amd import det, workloads
from conftest import bits_equal

pytestmark = pytest.mark.gpu

F32, F64 = np.float32, np.float64


def rounding(n, dtype, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 4, n)).astype(dtype)


def gpu_sum(x, dev):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    return det.det_sum(t).cpu().numpy()


SIZES = [0, 1, 2, 3, 5, 255, 256, 257, 1023, 4095, 4096, 4097, 16383, 16384, 16385, 65537,
         100003, (1 << 20) + 7, (1 << 14) * (1 << 14) // 1024 + 3]


@pytest.mark.parametrize("dtype", [F32, F64])
@pytest.mark.parametrize("n", SIZES)
def test_sum_parity(dev, dtype, n):
    x = rounding(n, dtype, n + 1)
    got = gpu_sum(x, dev)
    want = np.asarray(oracle.det_sum(x), dtype=dtype)
    assert bits_equal(got, want), (n, got, want)


def test_empty_sum_is_plus_zero(dev):
    for dt in (torch.float32, torch.float64):
        r = det.det_sum(torch.empty(0, dtype=dt, device=dev)).cpu()
        assert r.item() == 0.0 and not torch.signbit(r).item()


def test_quickstart_ones(dev):
    r = det.det_sum(torch.ones(4096, device=dev)).cpu()
    assert r.numpy().tobytes() == np.float32(4096.0).tobytes()


@pytest.mark.parametrize("dtype", [F32, F64])
def test_special_values(dev, dtype):
    cases = [
        np.full(5, -0.0, dtype), np.array([0.0, -0.0], dtype), np.array([-0.0, -0.0, 0.0], dtype),
        np.array([np.inf, 1.0], dtype), np.array([np.inf, -np.inf, 1.0], dtype),
        np.array([1.0, np.nan, 2.0], dtype), np.full(3000, np.finfo(dtype).tiny / 4, dtype),
        np.full(20000, np.finfo(dtype).max / 4, dtype),
    ]
    e = np.finfo(dtype).eps
    cases.append(np.array([1, e, e / 2, -1], dtype))
    cases.append(np.array([1, e / 2, e / 2, e / 2, e / 2], dtype))
    for x in cases:
        assert bits_equal(gpu_sum(x, dev), np.asarray(oracle.det_sum(x), dtype)), x[:8]


def test_c1_uniform_2_20_hundred_runs(dev):
    x = workloads.uniform01(1 << 20, seed=0)
    want = np.asarray(oracle.det_sum(x), F32)
    t = torch.from_numpy(x).to(dev)
    outs = torch.empty(100, dtype=torch.float32, device=dev)
    for r in range(100):
        det.det_sum(t, out=outs[r])
    got = outs.cpu().numpy()
    digest = {hashlib.sha256(v.tobytes()).hexdigest() for v in got}
    assert len(digest) == 1
    assert got[0].tobytes() == want.tobytes()


@pytest.mark.parametrize("dtype", [F32, F64])
def test_unaligned_view(dev, dtype):
    x = rounding(300001, dtype, 9)
    t = torch.from_numpy(x).to(dev)
    for k in (1, 2, 3):
        got = det.det_sum(t[k:]).cpu().numpy()
        assert bits_equal(got, np.asarray(oracle.det_sum(x[k:]), dtype)), k


@pytest.mark.parametrize("dtype", [F32, F64])
def test_launch_shape_invariance(dev, dtype):
    x = rounding(3_000_017, dtype, 4)
    want = np.asarray(oracle.det_sum(x), dtype)
    t = torch.from_numpy(x).to(dev)
    try:
        for grid, clog2, lds in [(0, 0, 0), (1, 0, 0), (7, 0, 0), (256, 0, 0), (512, 0, 0),
                                 (1024, 0, 0), (0, 16, 0), (3, 18, 0), (0, 20, 0), (1, 24, 0),
                                 (100000, 0, 0), (0, 0, 40000), (2048, 0, 65536)]:
            det.det_debug_set_launch(grid, lds)
            det.det_debug_set_sum_chunk(clog2)
            got = det.det_sum(t).cpu().numpy()
            assert bits_equal(got, want), (grid, clog2, lds)
            if grid:
                assert det.det_debug_last_launch()["sum_grid"] == grid
    finally:
        det.det_debug_set_launch(0, 0)
        det.det_debug_set_sum_chunk(0)


@pytest.mark.parametrize("dtype", [F32, F64])
def test_finishing_launch_reuses_workspace(dev, dtype):
    """Sums of 2 to 1,024 chunks finish in the launch that writes the chunk values: each value
    goes to a workspace slot tagged for the call, and the grid's last workgroup waits for every
    tag, reduces the values and clears the tags.  Whatever the slots hold beforehand (a fresh
    workspace's bytes, another size's values, a captured graph's earlier replay with the same
    tag), every call must give the oracle's bits."""
    # 2, 65, 184 and 1024 chunk values finish in one launch; 1025 take a second one
    sizes = [16385, (1 << 20) + 7, 3_000_017, (1 << 24) - 5, (1 << 24) + 3]
    xs = [rounding(n, dtype, n) for n in sizes]
    wants = [np.asarray(oracle.det_sum(x), dtype) for x in xs]
    ts = [torch.from_numpy(x).to(dev) for x in xs]
    ws = torch.empty(det.det_sum_workspace_size(max(sizes), 0 if dtype == F32 else 1),
                     dtype=torch.uint8, device=dev)
    tdt = torch.float32 if dtype == F32 else torch.float64
    outs = [torch.empty((), dtype=tdt, device=dev) for _ in sizes]

    def check(k, tag):
        assert bits_equal(outs[k].cpu().numpy(), wants[k]), (sizes[k], tag)

    for fill in (0x00, 0xFF, 0x5A):
        ws.fill_(fill)
        for k in range(len(sizes)):
            det.det_sum(ts[k], out=outs[k], ws=ws)
            check(k, f"fill {fill:#x}")
    gen = torch.Generator(device="cpu").manual_seed(7)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, generator=gen))
    graphs = []
    side = torch.cuda.Stream()
    for k in (0, 3):
        det.det_sum(ts[k], out=outs[k], ws=ws)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=side):
            det.det_sum(ts[k], out=outs[k], ws=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs.append((k, g))
    for rep in range(3):
        for k, g in graphs:
            outs[k].fill_(0.0)
            g.replay()
            torch.cuda.synchronize()
            check(k, f"replay {rep}")
            for j in (1, 2, 4):
                outs[j].fill_(0.0)
                det.det_sum(ts[j], out=outs[j], ws=ws)
                torch.cuda.synchronize()
                check(j, f"eager between replays {rep}")
