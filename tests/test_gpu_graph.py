"""The three operations captured in one HIP graph and replayed: same bits as direct calls.

The library enqueues only kernels on the caller's stream (no allocation, no memset, no host
synchronisation, no read-back), so a caller can record it once into a graph and replay it,
the workflow the Warp guide's "CUDA Graph Capture" section asks of deterministic code.  The
graph holds det_sum, four det_scan modes (forward/reverse, inclusive/exclusive, full and
segmented) and both det_scatter_add shapes (scalar bins with prev snapshot and skip count;
rows).  It is replayed several times, with the program's own eager work between replays
(the same workspaces reused by direct calls on other data, outputs overwritten), and every
replay must give the direct calls' bits, which must in turn equal the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from scan_fixed_order_amd import det
from conftest import bits_equal, first_mismatch

pytestmark = pytest.mark.gpu

TILE = 8192


def rounding(n, dtype, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 4, n)).astype(dtype)


def ws_for(nbytes, dev):
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_graph_replay_matches_direct_and_oracle(dev, dtype):
    tdt = torch.float32 if dtype == np.float32 else torch.float64
    code = 0 if dtype == np.float32 else 1
    # scan: two anchor intervals and a ragged tail; segments of mixed length
    n = 2 * 256 * TILE + 12345
    x_h = rounding(n, dtype, 11)
    rng = np.random.default_rng(12)
    cuts = np.sort(rng.choice(np.arange(1, n), 500, replace=False))
    offs_h = np.concatenate([[0], cuts, [n]]).astype(np.int64)
    # scatter: scalar bins with out-of-range indices; rows of 96 into 300 destinations
    m, B = 300007, 4099
    v_h = rounding(m, dtype, 13)
    i_h = rng.integers(-3, B + 3, m).astype(np.int32)
    o_h = rounding(B, dtype, 14)
    rn, rd, rl = 5000, 300, 96
    rv_h = rounding(rn * rl, dtype, 15).reshape(rn, rl)
    ri_h = rng.integers(0, rd, rn).astype(np.int32)
    ro_h = rounding(rd * rl, dtype, 16).reshape(rd, rl)

    x = torch.from_numpy(x_h).to(dev)
    offs = torch.from_numpy(offs_h).to(dev)
    v = torch.from_numpy(v_h).to(dev)
    idx = torch.from_numpy(i_h).to(dev)
    rv = torch.from_numpy(rv_h).to(dev)
    ri = torch.from_numpy(ri_h).to(dev)
    o_init = torch.from_numpy(o_h).to(dev)
    ro_init = torch.from_numpy(ro_h).to(dev)

    modes = [(False, False, False), (True, True, False), (False, True, True), (True, False, True)]
    ws_sum = ws_for(det.det_sum_workspace_size(n, code), dev)
    ws_scan = [ws_for(det.det_scan_workspace_size(n, code, (1 if e else 0) | (2 if r else 0),
                                                  len(offs_h) - 1 if s else 0), dev)
               for e, r, s in modes]
    ws_sc = ws_for(det.det_scatter_add_workspace_size(m, B, 1, code), dev)
    ws_rows = ws_for(det.det_scatter_add_workspace_size(rn, rd, rl, code), dev)

    s_out = torch.empty((), dtype=tdt, device=dev)
    ys = [torch.empty(n, dtype=tdt, device=dev) for _ in modes]
    out = torch.empty(B, dtype=tdt, device=dev)
    prev = torch.empty(m, dtype=tdt, device=dev)
    nsk = torch.empty(1, dtype=torch.int64, device=dev)
    rout = torch.empty(rd, rl, dtype=tdt, device=dev)

    def work():
        det.det_sum(x, out=s_out, ws=ws_sum)
        for (e, r, s), y, w in zip(modes, ys, ws_scan):
            det.det_scan(x, y=y, exclusive=e, reverse=r, offsets=offs if s else None, ws=w)
        det.det_scatter_add(v, idx, out, prev=prev, n_skipped=nsk, ws=ws_sc)
        det.det_scatter_add(rv, ri, rout, ws=ws_rows)

    def reset():
        out.copy_(o_init)
        rout.copy_(ro_init)
        for y in ys:
            y.fill_(float("nan"))
        prev.fill_(float("nan"))
        nsk.fill_(-1)
        s_out.fill_(float("nan"))

    def snapshot():
        torch.cuda.synchronize()
        return ([s_out.cpu().numpy().reshape(1)] + [y.cpu().numpy() for y in ys] +
                [out.cpu().numpy(), prev.cpu().numpy(), nsk.cpu().numpy().astype(np.float64),
                 rout.cpu().numpy()])

    # direct calls
    reset()
    work()
    direct = snapshot()

    # the oracle on the same inputs
    want = [np.asarray(oracle.det_sum(x_h), dtype).reshape(1)]
    for e, r, s in modes:
        want.append(oracle.scan(x_h, exclusive=e, reverse=r, offsets=offs_h if s else None))
    wo, wp, wk = oracle.scatter_add(v_h, i_h, o_h, want_prev=True)
    wr, _, _ = oracle.scatter_add(rv_h, ri_h, ro_h)
    want += [wo, wp, np.array([wk], np.float64), wr]      # prev: NaN where the index is skipped
    for k, (g, w) in enumerate(zip(direct, want)):
        assert bits_equal(g, w), ("direct vs oracle", k, first_mismatch(g, w))

    # capture once (side stream, as the graph API requires), replay several times
    torch.cuda.synchronize()
    reset()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    other = torch.from_numpy(rounding(n, dtype, 99)).to(dev)
    for rep in range(4):
        # eager work between replays reuses the graph's workspaces on other data
        det.det_sum(other, ws=ws_sum)
        det.det_scan(other, exclusive=True, ws=ws_scan[0])
        det.det_scatter_add(v[: m // 2], idx[: m // 2], torch.zeros(B, dtype=tdt, device=dev),
                            ws=ws_sc)
        torch.cuda.synchronize()
        reset()
        graph.replay()
        got = snapshot()
        for k, (g, d) in enumerate(zip(got, direct)):
            assert bits_equal(g, d), ("replay", rep, k, first_mismatch(g, d))


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_streams_do_not_change_bits(dev, dtype):
    # the same calls on the default stream and on two other streams running at the same time
    # (each with its own workspace, as the interface requires of overlapping calls)
    tdt = torch.float32 if dtype == np.float32 else torch.float64
    n = 3 * 256 * TILE + 777
    x = torch.from_numpy(rounding(n, dtype, 5)).to(dev)
    rng = np.random.default_rng(6)
    idx = torch.from_numpy(rng.integers(0, 5000, n).astype(np.int32)).to(dev)

    def run(ws_sum, ws_scan, ws_sc):
        s = det.det_sum(x, ws=ws_sum)
        h = torch.full((), -1, dtype=torch.int32, device=dev)   # the scan's health word
        y = det.det_scan(x, exclusive=True, reverse=True, ws=ws_scan, health=h)
        o = torch.zeros(5000, dtype=tdt, device=dev)
        det.det_scatter_add(x, idx, o, ws=ws_sc)
        healths.append(h)
        return s, y, o

    healths = []

    code = 0 if dtype == np.float32 else 1

    def workspaces():
        return (ws_for(det.det_sum_workspace_size(n, code), dev),
                ws_for(det.det_scan_workspace_size(n, code, 3, 0), dev),
                ws_for(det.det_scatter_add_workspace_size(n, 5000, 1, code), dev))

    ref = [t.cpu().numpy() for t in run(*workspaces())]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    w1, w2 = workspaces(), workspaces()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            r1 = run(*w1)
        with torch.cuda.stream(s2):
            r2 = run(*w2)
        outs.append((r1, r2))
    torch.cuda.synchronize()
    # 0: no look-back wait of any scan hit its time bound
    assert [int(h.item()) for h in healths] == [0] * len(healths)
    for it, (r1, r2) in enumerate(outs):
        for si, got in enumerate((r1, r2)):
            for name, g, w in zip(("sum", "scan", "scatter"), got, ref):
                g = g.cpu().numpy().reshape(w.shape)
                assert bits_equal(g, w), (name, "round", it, "stream", si + 1,
                                          first_mismatch(g.reshape(-1), w.reshape(-1)))
