"""Benchmark of the reproducible add-reductions on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic f32 input at
n = 2^28: det_sum (uniform [0,1) values), det_scan (inclusive forward, normal x 10^U(-4,4)
values with random signs) and det_scatter_add (normal values into 65,536 uniform int32 bins).
Inputs are resident in HBM before the timed region.  `value` is the step's algorithmic bytes
(sum 4n, scan 8n, scatter 8n + 8*bins) divided by the step time.

Prints ONE JSON line.  Besides the contract fields it carries:
  roofline      the kernel with the largest share of the step (by the library's own per-launch
                HIP events, recorded on the launching stream over a timed pass of K steps): its
                algorithmic bytes per launch over its average launch time, against 8 TB/s; and
                `traffic`, the HBM bytes per launch that rocprofv3 counters measured for the same
                kernel source (read from profiles/, null when that source has changed since);
  kernels       every library kernel of the step: launches per step, average ms;
  ops           per operation: time, GB/s, Gelem/s, fraction of 8 TB/s, the non-deterministic
                baseline's time on the same input (atomic-tail sum, per-element atomic
                scatter, the ROCm library scan), the deterministic-mode overhead, and the number
                of distinct results over repeated runs of each;
  cpu_baseline  the CPU oracle (single thread) on the same workload, timed on the host.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "scan_fixed_order_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--log2n", type=int, default=28)
    ap.add_argument("--bins", type=int, default=65536)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-baselines", action="store_true")
    ap.add_argument("--only", default="", help="comma list of sum,scan,scatter (profiling)")
    ap.add_argument("--repeat-runs", type=int, default=100,
                    help="runs whose distinct results are counted (library and baselines)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other configurations (parity cases) of the spec")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain device copy of 2^log2n f32 (1 GiB each way at 2^28): "
                         "the known-size kernel that scales rocprofv3 byte counters")
    return ap.parse_args()


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def kernel_bytes_per_step(n, B):
    """Algorithmic HBM bytes each library kernel must move in one step (f32, row_len 1).

    The scatter's two radix passes move key and value in and out.  When every destination fits
    16 bits, every pass writes 16-bit keys and the later passes read them: the first pass reads
    4 + 4 and writes 2 + 4 bytes per element, the second reads and writes 2 + 4 (else 4-byte
    keys throughout).  The segment reduction reads the sorted keys and values, and reads and
    writes each destination once."""
    parts = -(-n // (1 << 14))
    kb = 2.0 if B <= 65536 else 4.0
    return {
        "k_sum_chunks<f32>": 4.0 * n + 4.0 * parts,       # values, then the partials' level
        "k_scan<f32>": 8.0 * n,                           # read x, write y
        "k_radix_hist": 4.0 * n + kb * n,                 # keys, one pass per 8-bit digit
        "k_radix_scatter": (12.0 + kb) * n + (8.0 + 2 * kb) * n,   # first pass, second pass
        "k_segred_scalar": (kb + 4.0) * n + 8.0 * B,      # sorted keys + values, out r/w
    }


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch from a committed counter summary for `kernel`, or None when there is
    none or the kernel's source has changed since the counters were taken."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    for fn in sorted(os.listdir(pdir)):
        if not fn.endswith(".md"):
            continue
        text = open(os.path.join(pdir, fn)).read()
        m_k = re.search(r"^traffic-kernel: (\S+)\s*$", text, re.M)
        if not m_k or m_k.group(1) != kernel:
            continue
        m_s = re.search(r"^traffic-source: (\S+) sha256 ([0-9a-f]{64})\s*$", text, re.M)
        m_b = re.search(r"^traffic-bytes-per-launch: (\d+)\s*$", text, re.M)
        if not m_s or not m_b:
            continue
        src = os.path.join(ROOT, m_s.group(1))
        if not os.path.exists(src) or source_hash(src) != m_s.group(2):
            return None
        return int(m_b.group(1))
    return None


def time_configs(det, workloads, dev, log, base_lib=None):
    """Times every configuration of the workload spec besides the headline step (one GPU,
    inputs resident): median over repetitions of one call, bracketed by events on the current
    stream.  Returns {case: {ms, GB_s, frac_hbm, Gelem_s}} with algorithmic bytes as in the
    headline step; the large f64 case also reports the distinct results over launch grids of
    1x, 2x and 4x the compute-unit count."""
    import hashlib as _h

    import numpy as np
    import torch

    stream = torch.cuda.current_stream(dev)
    res = {}

    def med(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    def put(name, fn, nbytes, nelem, reps):
        ms = med(fn, reps)
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "GB_s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_GBS, 4),
                     "Gelem_s": round(nelem / (ms * 1e-3) / 1e9, 3)}

    def dev_t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def ws_of(nbytes):
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)

    # sum, n = 2^20 uniform and n = 4096 ones
    x = dev_t(workloads.uniform01(1 << 20, seed=0))
    w = ws_of(det.det_sum_workspace_size(1 << 20, 0))
    o = torch.empty((), dtype=torch.float32, device=dev)
    put("sum f32 n=2^20 U[0,1)", lambda: det.det_sum(x, out=o, ws=w), 4 << 20, 1 << 20, 50)
    if base_lib is not None:
        import ctypes as _ct0
        sp0 = _ct0.c_void_p(stream.cuda_stream)
        tmp = torch.empty((), dtype=torch.float32, device=dev)
        bms = med(lambda: base_lib.detbase_atomic_sum(_ct0.c_void_p(x.data_ptr()),
                                                      _ct0.c_int64(1 << 20), 0,
                                                      _ct0.c_void_p(tmp.data_ptr()), sp0), 50)
        res["sum f32 n=2^20 U[0,1)"]["nondet_baseline_ms"] = round(bms, 4)
        res["sum f32 n=2^20 U[0,1)"]["det_overhead"] = round(res["sum f32 n=2^20 U[0,1)"]["ms"] / bms - 1.0, 4)
    ones = torch.ones(4096, dtype=torch.float32, device=dev)
    put("sum f32 n=4096 ones", lambda: det.det_sum(ones, out=o, ws=w), 4 * 4096, 4096, 50)
    # scatter, n = 2^24: uniform over 65,536 bins, and every value into bin 0
    n = 1 << 24
    v = dev_t(workloads.normal(n, seed=1))
    for label, bins, B in (("65536 uniform bins", workloads.bins_uniform(n, 65536, seed=1), 65536),
                           ("bin 0 (contended)", np.zeros(n, np.int32), 65536)):
        bi = dev_t(bins)
        out = torch.zeros(B, dtype=torch.float32, device=dev)
        w = ws_of(det.det_scatter_add_workspace_size(n, B, 1, 0))
        put(f"scatter f32 n=2^24 into {label}",
            lambda: det.det_scatter_add(v, bi, out, ws=w), 8.0 * n + 8.0 * B, n, 20)
        if B == 65536 and label.startswith("65536"):
            # the same with prev as the running value (values, index read; prev written)
            pv = torch.empty_like(v)
            w2 = ws_of(det.det_scatter_add_running_workspace_size(n, B, 1, 0))
            put(f"scatter f32 n=2^24 into {label}, running prev",
                lambda: det.det_scatter_add_running(v, bi, out, prev=pv, ws=w2),
                12.0 * n + 8.0 * B, n, 10)
            del pv, w2
    del v
    # scan: f32 and f64, inclusive/exclusive x forward/reverse; the inclusive forward scan
    # beside the ROCm library's (hipCUB DeviceScan::InclusiveSum) on the same input, for the
    # deterministic-mode overhead at the sizes the drjit page measures
    import ctypes as _ct
    modes = ((False, False, "incl"), (True, False, "excl"), (False, True, "incl rev"),
             (True, True, "excl rev"))
    sp = _ct.c_void_p(stream.cuda_stream)
    for dt, tdt, code in ((np.float32, torch.float32, 0), (np.float64, torch.float64, 1)):
        for n in (16384, 164738, 1048577, 1 << 28):
            xs = dev_t(workloads.scan_values(n, dt, seed=2))
            ys = torch.empty_like(xs)
            w = ws_of(det.det_scan_workspace_size(n, code, 3, 0))
            reps = 20 if n < (1 << 28) else 10
            name0 = None
            for ex, rv, tag in modes:
                name = f"scan {np.dtype(dt).name} n={n if n < (1 << 28) else '2^28'} {tag}"
                name0 = name0 or name
                put(name, lambda: det.det_scan(xs, y=ys, exclusive=ex, reverse=rv, ws=w),
                    2.0 * n * xs.element_size(), n, reps)
            if base_lib is not None:
                f64 = code == 1
                wsz = (base_lib.detbase_lib_scan64_workspace_size if f64
                       else base_lib.detbase_lib_scan_workspace_size)(_ct.c_int64(n))
                wb = ws_of(wsz)
                fn = base_lib.detbase_lib_scan64 if f64 else base_lib.detbase_lib_scan
                args = (_ct.c_void_p(xs.data_ptr()), _ct.c_void_p(ys.data_ptr()), _ct.c_int64(n),
                        _ct.c_void_p(wb.data_ptr()), _ct.c_size_t(wsz), sp)
                bms = med(lambda: fn(*args), reps)
                res[name0]["nondet_baseline_ms"] = round(bms, 4)
                res[name0]["det_overhead"] = round(res[name0]["ms"] / bms - 1.0, 4)
            del xs, ys
    # the small latency-bound calls replayed from a captured HIP graph (launch gaps removed)
    xg = dev_t(workloads.uniform01(1 << 20, seed=0))
    wg = ws_of(det.det_sum_workspace_size(1 << 20, 0))
    og = torch.empty((), dtype=torch.float32, device=dev)
    xs = dev_t(workloads.scan_values(16384, np.float32, seed=2))
    ys = torch.empty_like(xs)
    wsg = ws_of(det.det_scan_workspace_size(16384, 0, 0, 0))
    for name, fn, nb, ne in (("sum f32 n=2^20 U[0,1), graph replay",
                              lambda: det.det_sum(xg, out=og, ws=wg), 4 << 20, 1 << 20),
                             ("scan float32 n=16384 incl, graph replay",
                              lambda: det.det_scan(xs, y=ys, ws=wsg), 8 * 16384, 16384)):
        fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.graph(graph, stream=side):
            fn()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        put(name, graph.replay, nb, ne, 50)
    log("configs: sum, scatter, scan timed")
    # segmented scan f32 2^26 (geometric segments, mean 100) and the row accumulate
    n = 1 << 26
    xs = dev_t(workloads.scan_values(n, np.float32, seed=3))
    offs_h = workloads.segment_offsets(n, 100.0, seed=3)
    offs = dev_t(offs_h)
    ys = torch.empty_like(xs)
    w = ws_of(det.det_scan_workspace_size(n, 0, 3, offs_h.size - 1))
    for ex, rv, tag in modes:
        put(f"segmented scan f32 n=2^26 mean 100 {tag}",
            lambda: det.det_scan(xs, y=ys, exclusive=ex, reverse=rv, offsets=offs, ws=w),
            8.0 * n + 8.0 * offs_h.size, n, 10)
    del xs, ys
    src, rows, out0 = workloads.rows_case()
    st, rt, ot0 = dev_t(src), dev_t(rows), dev_t(out0)
    ot = ot0.clone()
    w = ws_of(det.det_scatter_add_workspace_size(src.shape[0], out0.shape[0], src.shape[1], 0))
    put("rows f32 2^16x256 into 2^14 rows", lambda: det.det_scatter_add(st, rt, ot, ws=w),
        4.0 * src.size + 4.0 * rows.size + 8.0 * out0.size, src.size, 20)
    pr = torch.empty_like(st)
    w = ws_of(det.det_scatter_add_running_workspace_size(src.shape[0], out0.shape[0],
                                                         src.shape[1], 0))
    put("rows f32 2^16x256 into 2^14 rows, running prev",
        lambda: det.det_scatter_add_running(st, rt, ot, prev=pr, ws=w),
        8.0 * src.size + 4.0 * rows.size + 8.0 * out0.size, src.size, 20)
    del pr
    log("configs: segmented scan and rows timed")
    # large mixed-magnitude f64, n = 2^29: sum, scan, scatter into 2^20 Zipf(1.1) bins
    n = 1 << 29
    xm = dev_t(workloads.mixed_f64(n, seed=4))
    o64 = torch.empty((), dtype=torch.float64, device=dev)
    w = ws_of(max(det.det_sum_workspace_size(n, 1), det.det_scan_workspace_size(n, 1, 0, 0)))
    put("sum f64 n=2^29 mixed", lambda: det.det_sum(xm, out=o64, ws=w), 8.0 * n, n, 10)
    ym = torch.empty_like(xm)
    put("scan f64 n=2^29 mixed incl", lambda: det.det_scan(xm, y=ym, ws=w), 16.0 * n, n, 5)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    hs = {"sum": set(), "scan": set()}
    for g in (cus, 2 * cus, 4 * cus):
        det.det_debug_set_launch(g, 0)
        det.det_sum(xm, out=o64, ws=w)
        det.det_scan(xm, y=ym, ws=w)
        torch.cuda.synchronize()
        hs["sum"].add(_h.sha256(o64.cpu().numpy().tobytes()).hexdigest())
        hs["scan"].add(_h.sha256(ym.cpu().numpy().tobytes()).hexdigest())
    det.det_debug_set_launch(0, 0)
    res["sum f64 n=2^29 mixed"]["distinct_over_grids_1x_2x_4x_CUs"] = len(hs["sum"])
    res["scan f64 n=2^29 mixed incl"]["distinct_over_grids_1x_2x_4x_CUs"] = len(hs["scan"])
    del ym
    bi = dev_t(workloads.zipf_bins(n, 1 << 20, 1.1, seed=4))
    out = torch.zeros(1 << 20, dtype=torch.float64, device=dev)
    w = ws_of(det.det_scatter_add_workspace_size(n, 1 << 20, 1, 1))
    put("scatter f64 n=2^29 mixed into 2^20 Zipf(1.1) bins",
        lambda: det.det_scatter_add(xm, bi, out, ws=w), 12.0 * n + 16.0 * (1 << 20), n, 5)
    del xm, bi, w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log("configs: f64 2^29 timed")
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import ctypes

    import numpy as np
    import torch

    from scan_fixed_order_amd import det, workloads

    dev = torch.device("cuda:0")
    n = 1 << args.log2n
    B = args.bins
    only = set(filter(None, args.only.split(","))) or {"sum", "scan", "scatter"}

    # ---------------------------------------------------------------- inputs (host -> HBM)
    t0 = time.time()
    host = {}
    if "sum" in only:
        host["x_sum"] = workloads.uniform01(n, seed=0)
    if "scan" in only:
        host["x_scan"] = workloads.scan_values(n, np.float32, seed=2)
    if "scatter" in only:
        host["v_sc"] = workloads.normal(n, seed=1)
        host["b_sc"] = workloads.bins_uniform(n, B, seed=1)
    log(f"inputs generated in {time.time() - t0:.1f}s")
    g = {k: torch.from_numpy(v).to(dev) for k, v in host.items()}
    y_scan = torch.empty(n, dtype=torch.float32, device=dev) if "scan" in only else None
    out_sc = torch.zeros(B, dtype=torch.float32, device=dev) if "scatter" in only else None
    s_out = torch.empty((), dtype=torch.float32, device=dev)
    ws = torch.empty(max(det.det_sum_workspace_size(n, 0), det.det_scan_workspace_size(n, 0, 0, 0),
                         det.det_scatter_add_workspace_size(n, B, 1, 0)),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    ops = []
    if "sum" in only:
        ops.append(("sum", lambda: det.det_sum(g["x_sum"], out=s_out, ws=ws), 4.0 * n))
    if "scan" in only:
        ops.append(("scan", lambda: det.det_scan(g["x_scan"], y=y_scan, ws=ws), 8.0 * n))
    if "scatter" in only:
        ops.append(("scatter", lambda: det.det_scatter_add(g["v_sc"], g["b_sc"], out_sc, ws=ws),
                    8.0 * n + 8.0 * B))

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        for _, fn, _ in ops:
            fn()
    torch.cuda.synchronize()
    log("warmup done")

    # ---------------------------------------------------------------- timed steps
    # Three passes of K steps each, so that no pass carries another's markers: the whole step
    # bracketed by one event pair (ms_per_step, value); one event pair around each operation
    # (per-operation times); the library's own per-launch events on its stream (the kernel
    # table and the roofline).  Each marker adds a few microseconds of stream time.
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        for _, fn, _ in ops:
            fn()
    stop.record(stream)
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(stop) / args.steps
    log(f"timed {args.steps} steps: {step_ms:.3f} ms/step")

    ev = {name: [] for name, _, _ in ops}
    for _ in range(args.steps):
        for name, fn, _ in ops:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev[name].append((a, b))
    torch.cuda.synchronize()
    op_ms = {name: float(np.mean([a.elapsed_time(b) for a, b in ev[name]])) for name in ev}

    det.det_debug_kernel_timing(True)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        for _, fn, _ in ops:
            fn()
    torch.cuda.synchronize()
    kernels = det.det_debug_kernel_report()
    det.det_debug_kernel_timing(False)
    log(f"per-operation and per-kernel passes done")

    step_bytes = sum(bts for _, _, bts in ops)
    value = step_bytes / (step_ms * 1e-3) / 1e9

    if args.calibrate_copy:
        src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} f32 elements, 3 times")

    # ---------------------------------------------------------------- non-deterministic baselines
    base_ms = {}
    distinct = {}
    if not args.no_baselines:
        bl = ctypes.CDLL(os.path.join(ROOT, "scan_fixed_order_amd", "libdet_baselines.so"))
        sp = ctypes.c_void_p(stream.cuda_stream)
        vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        tmp = torch.empty((), dtype=torch.float32, device=dev)
        out_b = torch.zeros(B, dtype=torch.float32, device=dev)
        bl.detbase_lib_scan_workspace_size.restype = ctypes.c_size_t
        wsb_bytes = bl.detbase_lib_scan_workspace_size(ctypes.c_int64(n))
        wsb = torch.empty(max(wsb_bytes, 256), dtype=torch.uint8, device=dev)
        calls = {
            "sum": lambda: bl.detbase_atomic_sum(vp(g["x_sum"]), ctypes.c_int64(n), 0, vp(tmp), sp),
            "scan": lambda: bl.detbase_lib_scan(vp(g["x_scan"]), vp(y_scan), ctypes.c_int64(n),
                                                vp(wsb), ctypes.c_size_t(wsb_bytes), sp),
            "scatter": lambda: bl.detbase_atomic_scatter(vp(g["v_sc"]), vp(g["b_sc"]),
                                                         ctypes.c_int64(n), 0, vp(out_b),
                                                         ctypes.c_int64(B), sp),
        }
        for name, _, _ in ops:
            fn = calls[name]
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(args.steps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            base_ms[name] = a.elapsed_time(b) / args.steps
        log("baselines timed")

        # distinct results over repeated runs: the library and the baselines on the same input
        # (the scan's output compared on its last 2^20 elements, which depend on every input)
        import hashlib as _h

        def digest(t):
            return _h.sha256(t.cpu().numpy().tobytes()).hexdigest()

        tail = min(n, 1 << 20)
        probes = {
            "sum": (lambda: (det.det_sum(g["x_sum"], out=s_out, ws=ws), s_out)[1],
                    lambda: (calls["sum"](), tmp)[1]),
            "scan": (lambda: det.det_scan(g["x_scan"], y=y_scan, ws=ws)[-tail:],
                     lambda: (calls["scan"](), y_scan)[1][-tail:]),
            "scatter": (lambda: (out_sc.zero_(), det.det_scatter_add(g["v_sc"], g["b_sc"], out_sc,
                                                                      ws=ws))[1],
                        lambda: (out_b.zero_(), calls["scatter"](), out_b)[2]),
        }
        for name, _, _ in ops:
            dfn, bfn = probes[name]
            hashes_det = {digest(dfn()) for _ in range(args.repeat_runs)}
            hashes_base = {digest(bfn()) for _ in range(args.repeat_runs)}
            distinct[name] = {"det": len(hashes_det), "nondet_baseline": len(hashes_base)}
        log(f"repeatability over {args.repeat_runs} runs: {distinct}")

    # ---------------------------------------------------------------- per-op report
    op_rep = {}
    for name, _, bts in ops:
        ms = op_ms[name]
        gbs = bts / (ms * 1e-3) / 1e9
        r = {"ms": round(ms, 4), "GB_s": round(gbs, 1), "Gelem_s": round(n / (ms * 1e-3) / 1e9, 2),
             "frac_hbm": round(gbs / PEAK_GBS, 4), "algorithmic_bytes": int(bts)}
        if name in base_ms:
            r["nondet_baseline_ms"] = round(base_ms[name], 4)
            r["det_overhead"] = round(ms / base_ms[name] - 1.0, 4)
        if name in distinct:
            r["distinct_results"] = dict(distinct[name], runs=args.repeat_runs)
        op_rep[name] = r

    # ---------------------------------------------------------------- dominant kernel
    kern_rep = {k: {"launches_per_step": round(c / args.steps, 3), "avg_ms": round(avg, 5),
                    "ms_per_step": round(tot / args.steps, 5)}
                for k, (c, tot, avg) in kernels.items()}
    roofline = None
    if kernels:
        dom = max(kernels, key=lambda k: kernels[k][1])
        c, tot, avg = kernels[dom]
        per_step = kernel_bytes_per_step(n, B).get(dom)
        if per_step is not None:
            per_launch = per_step / (c / args.steps)
            achieved = per_launch / (avg * 1e-3) / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                        "traffic": measured_traffic(dom), "kernel": dom,
                        "algorithmic_bytes_per_launch": int(per_launch),
                        "avg_launch_ms": round(avg, 5)}

    # ---------------------------------------------------------------- the other configurations
    configs = None
    if not args.no_configs:
        blib = None
        if not args.no_baselines:
            blib = ctypes.CDLL(os.path.join(ROOT, "scan_fixed_order_amd", "libdet_baselines.so"))
            for nm in ("detbase_lib_scan_workspace_size", "detbase_lib_scan64_workspace_size"):
                getattr(blib, nm).restype = ctypes.c_size_t
        configs = time_configs(det, workloads, dev, log, blib)

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        xs = host.get("x_sum")
        xc = host.get("x_scan")
        vs, bs = host.get("v_sc"), host.get("b_sc")
        reps, dt, cpu_bytes = 0, 0.0, 0.0
        while reps < 3 and dt < 10.0:
            t = time.perf_counter()
            if xs is not None:
                oracle.det_sum(xs)
            if xc is not None:
                oracle.scan(xc)
            if vs is not None:
                oracle.scatter_add(vs, bs, np.zeros(B, np.float32))
            dt += time.perf_counter() - t
            cpu_bytes += step_bytes
            reps += 1
        cpu = {"value": round(cpu_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"the whole step's workload ({', '.join(sorted(only))} at n=2^{args.log2n}, "
                         f"{B} bins) run {reps} time(s) through the single-threaded C oracle: "
                         f"{dt:.1f} s on {os.cpu_count()} visible host cores"}
        log(f"cpu oracle: {reps} pass(es), {dt:.1f}s")

    line = {
        "metric": "GB/s & % HBM peak for bit-reproducible f32 sum/scatter-add/scan at 2^28, 1 GPU",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"f32 n=2^{args.log2n}: sum (U[0,1)), inclusive scan "
                               f"(N(0,1)*10^U(-4,4), random signs), scatter-add "
                               f"(N(0,1) into {B} uniform bins)",
                   "n": n, "bins": B, "ops": sorted(only)},
        "frac_hbm": round(value / PEAK_GBS, 4),
        "roofline": roofline,
        "kernels": kern_rep,
        "ops": op_rep,
        "cpu_baseline": cpu,
        "configs": configs,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
