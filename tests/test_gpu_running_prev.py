"""det_scatter_add_running on the GPU against the oracle, bit for bit.

prev is the running value (the destination's initial value plus the earlier contributions in
ascending source index, summed by the exclusive segmented scan of the destination-grouped
members); out must equal det_scatter_add's.  Shapes cover one and several scan tiles, more
than one anchor interval of tiles, out-of-range indices, one contended destination, 16-bit
and wider destination counts, rows with ragged column tiles, and the empty cases.
"""
import numpy as np
import pytest
import torch

import oracle
from scan_fixed_order_amd import det
from conftest import bits_equal, first_mismatch

pytestmark = pytest.mark.gpu


def spread(rng, shape, dtype):
    return (rng.standard_normal(shape) * 10.0 ** rng.uniform(-4, 4, shape)).astype(dtype)


def run_case(dev, dtype, n, B, d, seed, lo=-3, contended=False):
    rng = np.random.default_rng(seed)
    shape = (n,) if d == 1 else (n, d)
    v = spread(rng, shape, dtype)
    if contended:
        idx = np.zeros(n, np.int32)
    else:
        idx = rng.integers(lo, B + 3, n).astype(np.int32)
    o = spread(rng, (B,) if d == 1 else (B, d), dtype)
    o.reshape(-1)[::5] = -0.0
    print(f"[case] running prev dtype={np.dtype(dtype).name} n={n} B={B} d={d} seed={seed}",
          flush=True)
    want_out, want_prev, want_k = oracle.scatter_add_running(v, idx, o)
    tv = torch.from_numpy(v).to(dev)
    ti = torch.from_numpy(idx).to(dev)
    to = torch.from_numpy(o).to(dev)
    tp = torch.full(shape, float("nan"), dtype=tv.dtype, device=dev)
    nk = torch.full((1,), -1, dtype=torch.int64, device=dev)
    det.det_scatter_add_running(tv, ti, to, prev=tp, n_skipped=nk)
    got_prev = tp.cpu().numpy()
    assert bits_equal(got_prev, want_prev), first_mismatch(got_prev, want_prev)
    assert bits_equal(to.cpu().numpy(), want_out), first_mismatch(to.cpu().numpy(), want_out)
    assert int(nk.item()) == want_k
    # out is det_scatter_add's
    to2 = torch.from_numpy(o).to(dev)
    det.det_scatter_add(tv, ti, to2)
    assert bits_equal(to2.cpu().numpy(), to.cpu().numpy())


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("n,B", [(1, 1), (1000, 7), (300007, 4099), (70001, 70000),
                                 (2 * 256 * 8192 + 777, 65536),
                                 # either side of the size from which f32 values travel
                                 # through the sort beside their source indices
                                 (1 << 21, 3), ((1 << 21) + 1, 3), ((1 << 21) + 7, 1 << 20),
                                 # the prev writes through windows of 2^16 sources written in
                                 # two parts, 256 windows and 257 (two radix passes over them)
                                 (1 << 24, 65536), ((1 << 24) + 3, 70001)])
def test_scalar_parity(dev, dtype, n, B):
    run_case(dev, dtype, n, B, 1, seed=n % 1000 + B)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_one_contended_destination(dev, dtype):
    # 600,000 members of destination 0: one segment over 74 tiles
    run_case(dev, dtype, 600000, 3, 1, seed=5, contended=True)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("n,B,d", [(5000, 300, 96), (20011, 997, 33), (3, 2, 1000),
                                   (300007, 50000, 2), (256 * 8192, 9, 2),
                                   (256 * 8192 + 5, 9, 2)])
def test_rows_parity(dev, dtype, n, B, d):
    run_case(dev, dtype, n, B, d, seed=d)


def test_rows_accumulate_shape(dev):
    # the row-accumulate workload: 2^16 source rows of 256 into 2^14 destinations
    run_case(dev, np.float32, 1 << 16, 1 << 14, 256, seed=3, lo=0)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_special_values_above_the_packing_size(dev, dtype):
    # f32 values travel through the sort as bits beside their source indices above 2^21
    # members: NaN, infinities, signed zeros and subnormals must come out bit for bit, and
    # skipped sources keep their prev untouched
    rng = np.random.default_rng(23)
    n, B = (1 << 21) + 9, 5000
    v = spread(rng, n, dtype)
    tiny = np.finfo(dtype).smallest_subnormal
    special = np.array([np.nan, np.inf, -np.inf, -0.0, 0.0, tiny, -tiny], dtype)
    pos = rng.choice(n, 7000, replace=False)
    v[pos] = special[rng.integers(0, special.size, pos.size)]
    idx = rng.integers(-2, B + 2, n).astype(np.int32)
    o = spread(rng, B, dtype)
    print(f"[case] running prev special values dtype={np.dtype(dtype).name} n={n}", flush=True)
    want_out, want_prev, want_k = oracle.scatter_add_running(v, idx, o)
    tv, ti, to = (torch.from_numpy(a).to(dev) for a in (v, idx, o))
    tp = torch.full((n,), 7.0, dtype=tv.dtype, device=dev)
    nk = torch.full((1,), -1, dtype=torch.int64, device=dev)
    det.det_scatter_add_running(tv, ti, to, prev=tp, n_skipped=nk)
    got_prev = tp.cpu().numpy()
    skipped = (idx < 0) | (idx >= B)
    assert (got_prev[skipped] == 7.0).all()
    assert bits_equal(got_prev[~skipped], want_prev[~skipped]), \
        first_mismatch(got_prev[~skipped], want_prev[~skipped])
    assert bits_equal(to.cpu().numpy(), want_out)
    assert int(nk.item()) == want_k == int(skipped.sum())


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_all_skipped_and_empty(dev, dtype):
    tdt = torch.float32 if dtype == np.float32 else torch.float64
    v = torch.ones(50, dtype=tdt, device=dev)
    idx = torch.full((50,), 9, dtype=torch.int32, device=dev)
    out = torch.zeros(4, dtype=tdt, device=dev)
    prev = torch.full((50,), float("nan"), dtype=tdt, device=dev)
    nk = torch.full((1,), -1, dtype=torch.int64, device=dev)
    det.det_scatter_add_running(v, idx, out, prev=prev, n_skipped=nk)
    assert int(nk.item()) == 50
    assert torch.isnan(prev).all() and (out == 0).all()
    e = torch.zeros(0, dtype=tdt, device=dev)
    det.det_scatter_add_running(e, torch.zeros(0, dtype=torch.int32, device=dev), out,
                                prev=e.clone(), n_skipped=nk)
    assert int(nk.item()) == 0
    det.det_scatter_add_running(v, idx, torch.zeros(0, dtype=tdt, device=dev), prev=prev,
                                n_skipped=nk)
    assert int(nk.item()) == 50
    # every source skipped above the size from which f32 values ride through the sort and
    # prev goes out through source windows: no pair in any window
    n = (1 << 21) + 1
    v = torch.ones(n, dtype=tdt, device=dev)
    idx = torch.full((n,), -1, dtype=torch.int32, device=dev)
    idx[::2] = 4
    prev = torch.full((n,), float("nan"), dtype=tdt, device=dev)
    det.det_scatter_add_running(v, idx, out, prev=prev, n_skipped=nk)
    assert int(nk.item()) == n and torch.isnan(prev).all() and (out == 0).all()


def test_integer_data_is_a_loop_of_atomics(dev):
    # small integers: every order is exact, so prev equals a loop of atomic adds
    rng = np.random.default_rng(17)
    n, B = 100000, 513
    v = rng.integers(-8, 9, n).astype(np.float32)
    idx = rng.integers(0, B, n).astype(np.int32)
    o = rng.integers(-50, 51, B).astype(np.float32)
    cur = o.astype(np.float64).copy()
    want = np.empty(n, np.float64)
    for i in range(n):
        want[i] = cur[idx[i]]
        cur[idx[i]] += v[i]
    tp = torch.empty(n, dtype=torch.float32, device=dev)
    to = torch.from_numpy(o).to(dev)
    det.det_scatter_add_running(torch.from_numpy(v).to(dev), torch.from_numpy(idx).to(dev), to,
                                prev=tp)
    assert np.array_equal(tp.cpu().numpy().astype(np.float64), want)
    assert np.array_equal(to.cpu().numpy().astype(np.float64), cur)
