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
  attainable    what a plain streaming read and a plain copy reach on the same GPU in the same run;
  kernels       every library kernel of the step: launches per step, average ms;
  ops           per operation: time (mean, median, p10, p90), GB/s, Gelem/s, fraction of 8 TB/s,
                the non-deterministic baselines on the same input and the deterministic-mode
                overhead, distinct results over repeated runs (every output element of every
                run compared with the first run on the device, and 64-bit fingerprints of the
                baselines' outputs), the error against a double-precision reference next to the
                baselines' errors, and the SHA-256 digest of the output bytes;
  configs       every other configuration of the workload spec (see time_configs);
  cpu_baseline  the CPU oracle (single thread) on the same workload, timed on the host; its
                `parallel` entry: the OpenMP driver of the same oracle functions on the usable
                cores, with a check that it gives the single-threaded bits.
"""
import argparse
import ctypes
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
    ap.add_argument("--no-accuracy", action="store_true",
                    help="skip the host-side error and digest computations")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain device copy of 2^log2n f32 (1 GiB each way at 2^28): "
                         "the known-size kernel that scales rocprofv3 byte counters")
    return ap.parse_args()


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def kernel_bytes_per_step(n, B):
    """Algorithmic HBM bytes each library kernel must move in one step (f32, row_len 1).

    With 256 < B <= 65536 the scatter sorts in two radix passes on byte keys: the first reads
    the 4-byte destination and the value and writes the destination's high byte and the value
    (8 + 5 bytes per element); the second reads those and writes the value (5 + 4); the two
    histogram passes read the destinations (4) and the bytes (1); the destination offsets come
    from the histograms, so the reduction reads only the sorted values (4) and reads and writes
    each destination once."""
    parts = -(-n // (1 << 14))
    rows = {"k_sum_chunks<f32>": 4.0 * n + 4.0 * parts,  # values, then the partials' level
            "k_scan<f32>": 8.0 * n}                      # read x, write y
    if 256 < B <= 65536:
        rows.update({"k_radix_hist": 4.0 * n + 1.0 * n,          # destinations, then key bytes
                     "k_radix_scatter": 13.0 * n + 9.0 * n,      # first pass, second pass
                     "k_segred_scalar": 4.0 * n + 8.0 * B})      # sorted values, out r/w
    return rows


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


def host_info():
    model, mem = "unknown", None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                mem = round(int(line.split()[1]) / (1 << 20), 1)
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "mem_total_GiB": mem, "visible_cores": os.cpu_count(),
            "usable_cores": usable}


# ---------------------------------------------------------------- device helpers

def ibits(t):
    import torch
    return t.view(torch.int64 if t.dtype == torch.float64 else torch.int32)


def fingerprint(t):
    """64-bit weighted sum (mod 2^64) of the output's bit patterns, computed on the device with
    integer arithmetic (any order gives the same value); distinct outputs collide with
    probability about 2^-64."""
    import torch
    b = ibits(t).reshape(-1).to(torch.int64)
    w = torch.arange(1, b.numel() + 1, device=t.device, dtype=torch.int64)
    w = w * 0x5851F42D4C957F2D + 0x14057B7EF767814F
    return int((b * (w | 1)).sum().item())


def distinct_runs(fn, runs):
    """(distinct results, first output): every run's output compared, element by element on the
    device, with the first run's, and fingerprinted."""
    import torch
    first = fn().clone()
    fps = {fingerprint(first)}
    same = 0
    for _ in range(runs - 1):
        o = fn()
        fps.add(fingerprint(o))
        same += int(torch.equal(ibits(o), ibits(first)))
    # every run equal to the first means one result; else count fingerprints
    return (1 if same == runs - 1 else max(2, len(fps))), first


def stats(ts):
    import numpy as np
    a = np.asarray(ts, dtype=np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)),
            "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90))}


# ---------------------------------------------------------------- accuracy (host)

def sum_error(got, x):
    import numpy as np
    ref = float(np.sum(x, dtype=np.float64))
    return abs(float(got) - ref) / abs(ref) if ref else abs(float(got))


def scan_error(got, x):
    """max_i |y_i - r_i| / sum_{k<=i} |x_k|: the normwise error against a double-precision
    prefix sum (its own error is at most n * 2^-53 relative to the same norm)."""
    import numpy as np
    r = np.cumsum(x, dtype=np.float64)
    d = np.abs(got.astype(np.float64) - r)
    del r
    a = np.cumsum(np.abs(x), dtype=np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        q = np.where(a > 0, d / np.where(a > 0, a, 1.0), d)
    return float(q.max())


def scatter_error(got, v, b, B, init):
    """max over destinations of |out - ref| / (|init| + sum |v|), ref in double precision."""
    import numpy as np
    ok = (b >= 0) & (b < B)
    ref = np.bincount(b[ok], weights=v[ok].astype(np.float64), minlength=B) + init
    den = np.bincount(b[ok], weights=np.abs(v[ok]).astype(np.float64), minlength=B) + np.abs(init)
    d = np.abs(got.astype(np.float64) - ref)
    q = np.where(den > 0, d / np.where(den > 0, den, 1.0), d)
    return float(q.max())


def sha256_of(t):
    return hashlib.sha256(t.detach().cpu().numpy().tobytes()).hexdigest()


# ---------------------------------------------------------------- the other configurations

def time_configs(det, workloads, dev, log, base_lib=None):
    """Times every configuration of the workload spec besides the headline step (one GPU,
    inputs resident): median (and p10/p90) over repetitions of one call, bracketed by events on
    the current stream.  Returns {case: {...}} with algorithmic bytes as in the headline step.

    Besides the spec's cases: the scan beside the same kernel with the adaptive look-back and
    beside the ROCm library scan, with distinct results over 100 runs of each; the segmented
    scan of 200,000 elements in blocks of 65,537 (drjit-core pull request, "Microbenchmark");
    Warp's accumulation grid (writes 65,536 / 262,144 / 1,048,576 into 1 or 65,536 outputs,
    a graph replay of zero + launch, "Performance"); the small calls 20 to a graph; and the
    f64 2^29 sum and scan over launch grids of 1x, 2x and 4x the CU count at two occupancies."""
    import numpy as np
    import torch

    stream = torch.cuda.current_stream(dev)
    res = {}
    sp = ctypes.c_void_p(stream.cuda_stream)
    vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def times(fn, reps, warm=2):
        for _ in range(warm):
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
        return stats(ts)

    def put(name, fn, nbytes, nelem, reps, per_call=1):
        st = times(fn, reps)
        ms = st["median"] / per_call
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "p10_ms": round(st["p10"] / per_call, 4),
                     "p90_ms": round(st["p90"] / per_call, 4), "GB_s": round(gbs, 1),
                     "frac_hbm": round(gbs / PEAK_GBS, 4),
                     "Gelem_s": round(nelem / (ms * 1e-3) / 1e9, 3)}
        return res[name]

    def dev_t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def ws_of(nbytes):
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)

    def graph_of(fn, k):
        """A HIP graph holding k calls of fn, captured on a side stream."""
        fn()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.graph(gr, stream=side):
            for _ in range(k):
                fn()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        return gr

    # sum, n = 2^20 uniform and n = 4096 ones
    x = dev_t(workloads.uniform01(1 << 20, seed=0))
    w = ws_of(det.det_sum_workspace_size(1 << 20, 0))
    o = torch.empty((), dtype=torch.float32, device=dev)
    put("sum f32 n=2^20 U[0,1)", lambda: det.det_sum(x, out=o, ws=w), 4 << 20, 1 << 20, 50)
    if base_lib is not None:
        tmp = torch.empty((), dtype=torch.float32, device=dev)
        bms = times(lambda: base_lib.detbase_atomic_sum(vp(x), ctypes.c_int64(1 << 20), 0,
                                                        vp(tmp), sp), 50)["median"]
        r = res["sum f32 n=2^20 U[0,1)"]
        r["nondet_baseline_ms"] = round(bms, 4)
        r["det_overhead"] = round(r["ms"] / bms - 1.0, 4)
    ones = torch.ones(4096, dtype=torch.float32, device=dev)
    put("sum f32 n=4096 ones", lambda: det.det_sum(ones, out=o, ws=w), 4 * 4096, 4096, 50)
    # the small latency-bound calls, 20 to a captured graph: the per-call cost without launch
    # gaps (one call per replay mostly measures the graph launch itself)
    gr = graph_of(lambda: det.det_sum(x, out=o, ws=w), 20)
    put("sum f32 n=2^20 U[0,1), per call in a graph of 20", gr.replay, 4 << 20, 1 << 20, 30,
        per_call=20)
    gr1 = graph_of(lambda: det.det_sum(x, out=o, ws=w), 1)
    put("sum f32 n=2^20 U[0,1), graph of 1 call", gr1.replay, 4 << 20, 1 << 20, 30)
    del gr, gr1
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
    # Warp's accumulation grid: graph replay of (zero the outputs + the scatter), f32 values,
    # all writes into one output or uniform over 65,536; det_scatter_add beside per-element
    # float atomics
    for writes in (65536, 262144, 1048576):
        vv = dev_t(workloads.normal(writes, seed=31))
        for B in (1, 65536):
            bi = dev_t(np.zeros(writes, np.int32) if B == 1
                       else workloads.bins_uniform(writes, B, seed=31))
            out = torch.zeros(B, dtype=torch.float32, device=dev)
            w = ws_of(det.det_scatter_add_workspace_size(writes, B, 1, 0))

            def det_call():
                out.zero_()
                det.det_scatter_add(vv, bi, out, ws=w)

            name = f"pattern A: {writes} writes into {B} output(s), graph replay of zero + launch"
            r = put(name, graph_of(det_call, 1).replay, 8.0 * writes + 8.0 * B, writes, 50)
            r20 = times(graph_of(det_call, 20).replay, 20)["median"] / 20
            r["ms_per_call_in_graph_of_20"] = round(r20, 4)
            if base_lib is not None:
                def nd_call():
                    out.zero_()
                    base_lib.detbase_atomic_scatter(vp(vv), vp(bi), ctypes.c_int64(writes), 0,
                                                    vp(out), ctypes.c_int64(B), sp)

                nd = times(graph_of(nd_call, 1).replay, 50)["median"]
                nd20 = times(graph_of(nd_call, 20).replay, 20)["median"] / 20
                r["nondet_baseline_ms"] = round(nd, 4)
                r["nondet_baseline_ms_per_call_in_graph_of_20"] = round(nd20, 4)
                r["det_overhead"] = round(r["ms"] / nd - 1.0, 4)
    log("configs: sum, scatter, pattern A timed")
    # scan: f32 and f64, inclusive/exclusive x forward/reverse; beside the same kernel with the
    # adaptive look-back (every mode) and the ROCm library's inclusive scan
    modes = ((False, False, "incl"), (True, False, "excl"), (False, True, "incl rev"),
             (True, True, "excl rev"))
    for dt, code in ((np.float32, 0), (np.float64, 1)):
        for n in (16384, 164738, 1048577, 1 << 28):
            xs = dev_t(workloads.scan_values(n, dt, seed=2))
            ys = torch.empty_like(xs)
            w = ws_of(det.det_scan_workspace_size(n, code, 3, 0))
            reps = 20 if n < (1 << 28) else 10
            wa = None
            if base_lib is not None:
                wa = ws_of(base_lib.detbase_adaptive_scan_workspace_size(ctypes.c_int64(n), code,
                                                                         ctypes.c_int64(0)))
            for ex, rv, tag in modes:
                name = f"scan {np.dtype(dt).name} n={n if n < (1 << 28) else '2^28'} {tag}"
                r = put(name, lambda: det.det_scan(xs, y=ys, exclusive=ex, reverse=rv, ws=w),
                        2.0 * n * xs.element_size(), n, reps)
                if wa is not None:
                    flags = (1 if ex else 0) | (2 if rv else 0)

                    def ad(flags=flags):
                        base_lib.detbase_adaptive_scan(vp(xs), vp(ys), ctypes.c_int64(n), code,
                                                       flags, None, ctypes.c_int64(0), vp(wa),
                                                       ctypes.c_size_t(wa.numel()), sp)
                        return ys

                    ams = times(ad, reps)["median"]
                    r["adaptive_lookback_ms"] = round(ams, 4)
                    r["det_overhead_vs_adaptive"] = round(r["ms"] / ams - 1.0, 4)
                    if tag == "incl":
                        runs = 100
                        r["distinct_results_100_runs"] = {
                            "det": distinct_runs(lambda: det.det_scan(xs, y=ys, ws=w), runs)[0],
                            "adaptive_lookback": distinct_runs(ad, runs)[0]}
            if base_lib is not None:
                f64 = code == 1
                wsz = (base_lib.detbase_lib_scan64_workspace_size if f64
                       else base_lib.detbase_lib_scan_workspace_size)(ctypes.c_int64(n))
                wb = ws_of(wsz)
                fn = base_lib.detbase_lib_scan64 if f64 else base_lib.detbase_lib_scan
                args = (vp(xs), vp(ys), ctypes.c_int64(n), vp(wb), ctypes.c_size_t(wsz), sp)
                name0 = f"scan {np.dtype(dt).name} n={n if n < (1 << 28) else '2^28'} incl"
                bms = times(lambda: fn(*args), reps)["median"]
                res[name0]["rocm_library_scan_ms"] = round(bms, 4)
                res[name0]["det_overhead_vs_library"] = round(res[name0]["ms"] / bms - 1.0, 4)
            del xs, ys, w, wa
    xs = dev_t(workloads.scan_values(16384, np.float32, seed=2))
    ys = torch.empty_like(xs)
    wsg = ws_of(det.det_scan_workspace_size(16384, 0, 0, 0))
    gr = graph_of(lambda: det.det_scan(xs, y=ys, ws=wsg), 20)
    put("scan float32 n=16384 incl, per call in a graph of 20", gr.replay, 8 * 16384, 16384, 30,
        per_call=20)
    del gr
    log("configs: scans timed")
    # the drjit microbenchmark's segmented case: 200,000 elements in blocks of 65,537
    n = 200000
    offs = dev_t(np.array([0, 65537, 131074, 196611, 200000], np.int64))
    for dt, code in ((np.float32, 0), (np.float64, 1)):
        xs = dev_t(workloads.scan_values(n, dt, seed=2))
        ys = torch.empty_like(xs)
        w = ws_of(det.det_scan_workspace_size(n, code, 3, 4))
        wa = None if base_lib is None else ws_of(base_lib.detbase_adaptive_scan_workspace_size(
            ctypes.c_int64(n), code, ctypes.c_int64(4)))
        for ex, rv, tag in modes:
            name = f"segmented scan {np.dtype(dt).name} n=200000 blocks of 65537 {tag}"
            r = put(name, lambda: det.det_scan(xs, y=ys, exclusive=ex, reverse=rv, offsets=offs,
                                               ws=w), 2.0 * n * xs.element_size(), n, 20)
            if wa is not None:
                flags = (1 if ex else 0) | (2 if rv else 0)
                ams = times(lambda: base_lib.detbase_adaptive_scan(
                    vp(xs), vp(ys), ctypes.c_int64(n), code, flags, vp(offs), ctypes.c_int64(4),
                    vp(wa), ctypes.c_size_t(wa.numel()), sp), 20)["median"]
                r["adaptive_lookback_ms"] = round(ams, 4)
                r["det_overhead_vs_adaptive"] = round(r["ms"] / ams - 1.0, 4)
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
    log("configs: segmented scans and rows timed")
    # large mixed-magnitude f64, n = 2^29: sum, scan, scatter into 2^20 Zipf(1.1) bins
    n = 1 << 29
    xm = dev_t(workloads.mixed_f64(n, seed=4))
    o64 = torch.empty((), dtype=torch.float64, device=dev)
    w = ws_of(max(det.det_sum_workspace_size(n, 1), det.det_scan_workspace_size(n, 1, 0, 0)))
    put("sum f64 n=2^29 mixed", lambda: det.det_sum(xm, out=o64, ws=w), 8.0 * n, n, 10)
    ym = torch.empty_like(xm)
    put("scan f64 n=2^29 mixed incl", lambda: det.det_scan(xm, y=ym, ws=w), 16.0 * n, n, 5)
    # launch grids of 1x, 2x, 4x the CU count, each at the default occupancy and with 24 KiB
    # more LDS per workgroup (one f64 scan workgroup per CU instead of two); the shapes that
    # actually ran are read back from the library
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    ref_scan = ref_sum = None
    shapes, same_sum, same_scan = [], True, True
    for grid, lds in ((cus, 0), (2 * cus, 0), (4 * cus, 0), (cus, 24576), (2 * cus, 24576),
                      (4 * cus, 24576)):
        det.det_debug_set_launch(grid, lds)
        det.det_sum(xm, out=o64, ws=w)
        det.det_scan(xm, y=ym, ws=w)
        torch.cuda.synchronize()
        last = det.det_debug_last_launch()
        shapes.append({"requested_grid": grid, "extra_lds": lds, **last})
        if ref_scan is None:
            ref_scan, ref_sum = ym.clone(), o64.clone()
        else:
            same_scan &= torch.equal(ibits(ym), ibits(ref_scan))
            same_sum &= torch.equal(ibits(o64), ibits(ref_sum))
    det.det_debug_set_launch(0, 0)
    res["sum f64 n=2^29 mixed"]["distinct_over_launch_shapes"] = 1 if same_sum else 2
    res["scan f64 n=2^29 mixed incl"]["distinct_over_launch_shapes"] = 1 if same_scan else 2
    res["scan f64 n=2^29 mixed incl"]["launch_shapes"] = shapes
    del ym, ref_scan
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
        print(json.dumps({"error": "this benchmark runs on one GPU only (nothing here uses a "
                                   "second one); run it with --gpus 1", "n_gpus": args.gpus}))
        sys.exit(2)

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
    health = torch.zeros((), dtype=torch.int32, device=dev)
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
    if "scan" in only:
        # the scans' bounded waits all ended normally (the workspace's health word)
        det.det_scan(g["x_scan"], y=y_scan, ws=ws, health=health)
        if int(health.item()) != 0:
            raise SystemExit("det_scan health word set: a look-back wait gave up")

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
    op_st = {name: stats([a.elapsed_time(b) for a, b in ev[name]]) for name in ev}

    det.det_debug_kernel_timing(True)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        for _, fn, _ in ops:
            fn()
    torch.cuda.synchronize()
    kernels = det.det_debug_kernel_report()
    det.det_debug_kernel_timing(False)
    log("per-operation and per-kernel passes done")

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
    base_ms, distinct, outs_base = {}, {}, {}
    attainable = None
    bl = None
    if not args.no_baselines:
        bl = ctypes.CDLL(os.path.join(ROOT, "scan_fixed_order_amd", "libdet_baselines.so"))
        for nm in ("detbase_lib_scan_workspace_size", "detbase_lib_scan64_workspace_size",
                   "detbase_adaptive_scan_workspace_size"):
            getattr(bl, nm).restype = ctypes.c_size_t
        sp = ctypes.c_void_p(stream.cuda_stream)
        vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        tmp = torch.empty((), dtype=torch.float32, device=dev)
        out_b = torch.zeros(B, dtype=torch.float32, device=dev)
        y_b = torch.empty(n, dtype=torch.float32, device=dev) if "scan" in only else None
        wsb_bytes = bl.detbase_lib_scan_workspace_size(ctypes.c_int64(n))
        wsb = torch.empty(max(wsb_bytes, 256), dtype=torch.uint8, device=dev)
        wsa_bytes = bl.detbase_adaptive_scan_workspace_size(ctypes.c_int64(n), 0,
                                                            ctypes.c_int64(0))
        wsa = torch.empty(max(wsa_bytes, 256), dtype=torch.uint8, device=dev)
        calls = {
            "sum": lambda: (bl.detbase_atomic_sum(vp(g["x_sum"]), ctypes.c_int64(n), 0, vp(tmp),
                                                  sp), tmp)[1],
            "scan": lambda: (bl.detbase_adaptive_scan(vp(g["x_scan"]), vp(y_b), ctypes.c_int64(n),
                                                      0, 0, None, ctypes.c_int64(0), vp(wsa),
                                                      ctypes.c_size_t(wsa_bytes), sp), y_b)[1],
            "scatter": lambda: (out_b.zero_(),
                                bl.detbase_atomic_scatter(vp(g["v_sc"]), vp(g["b_sc"]),
                                                          ctypes.c_int64(n), 0, vp(out_b),
                                                          ctypes.c_int64(B), sp), out_b)[2],
        }

        def lib_scan():
            bl.detbase_lib_scan(vp(g["x_scan"]), vp(y_b), ctypes.c_int64(n), vp(wsb),
                                ctypes.c_size_t(wsb_bytes), sp)
            return y_b

        def timed_loop(fn):
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
            return a.elapsed_time(b) / args.steps

        for name, _, _ in ops:
            base_ms[name] = timed_loop(calls[name])
        if "scan" in only:
            base_ms["scan_library"] = timed_loop(lib_scan)
        log("baselines timed")

        # what this GPU's HBM gives a plain kernel, in the same run: a streaming read of 2^log2n
        # f32 (16-byte non-temporal loads), and a copy of as many
        xr = g.get("x_sum", g.get("x_scan", g.get("v_sc")))
        sink = torch.zeros(4096, dtype=torch.float32, device=dev)
        yr = torch.empty_like(xr)
        nb = xr.numel() * 4
        rd = timed_loop(lambda: bl.detbase_stream_read(vp(xr), ctypes.c_int64(nb), vp(sink), sp))
        cp = timed_loop(lambda: bl.detbase_copy(vp(xr), vp(yr), ctypes.c_int64(nb), sp))
        attainable = {"stream_read_GB_s": round(nb / (rd * 1e-3) / 1e9, 1),
                      "copy_GB_s": round(2 * nb / (cp * 1e-3) / 1e9, 1),
                      "bytes_read": nb, "note": "16-byte non-temporal accesses, 4096 workgroups"}
        del yr
        log(f"attainable: read {attainable['stream_read_GB_s']} GB/s, "
            f"copy {attainable['copy_GB_s']} GB/s")

        # distinct results over repeated runs: the library and the baselines on the same input,
        # every output element of every run compared with the first run's on the device
        probes = {
            "sum": lambda: det.det_sum(g["x_sum"], out=s_out, ws=ws),
            "scan": lambda: det.det_scan(g["x_scan"], y=y_scan, ws=ws),
            "scatter": lambda: (out_sc.zero_(), det.det_scatter_add(g["v_sc"], g["b_sc"], out_sc,
                                                                     ws=ws))[1],
        }
        for name, _, _ in ops:
            dn, _ = distinct_runs(probes[name], args.repeat_runs)
            bn, first_b = distinct_runs(calls[name], args.repeat_runs)
            outs_base[name] = first_b
            distinct[name] = {"det": dn, "nondet_baseline": bn, "runs": args.repeat_runs,
                              "compared": "every output element of every run, on the device"}
            if name == "scan":
                distinct[name]["rocm_library_scan"] = distinct_runs(lib_scan,
                                                                    args.repeat_runs)[0]
        log(f"repeatability over {args.repeat_runs} runs: {distinct}")

    # ---------------------------------------------------------------- accuracy and digests
    accuracy = {}
    if not args.no_accuracy:
        for name, fn, _ in ops:
            if name == "scatter":
                out_sc.zero_()
            o = fn()
            torch.cuda.synchronize()
            r = {"sha256": sha256_of(o)}
            if name == "sum":
                r["det_rel_err"] = sum_error(o.item(), host["x_sum"])
                if "sum" in outs_base:
                    r["nondet_baseline_rel_err"] = sum_error(outs_base["sum"].item(),
                                                             host["x_sum"])
                r["measure"] = "|s - ref| / |ref|, ref the float64 sum"
            elif name == "scan":
                r["det_rel_err"] = scan_error(o.cpu().numpy(), host["x_scan"])
                if "scan" in outs_base:
                    r["nondet_baseline_rel_err"] = scan_error(outs_base["scan"].cpu().numpy(),
                                                              host["x_scan"])
                r["measure"] = "max_i |y_i - r_i| / sum_{k<=i} |x_k|, r the float64 prefix sum"
            else:
                r["det_rel_err"] = scatter_error(o.cpu().numpy(), host["v_sc"], host["b_sc"], B,
                                                 np.zeros(B))
                if "scatter" in outs_base:
                    r["nondet_baseline_rel_err"] = scatter_error(
                        outs_base["scatter"].cpu().numpy(), host["v_sc"], host["b_sc"], B,
                        np.zeros(B))
                r["measure"] = "max_b |out_b - r_b| / sum_{i in b} |v_i|, r in float64"
            accuracy[name] = r
        log("accuracy and digests done")

    # ---------------------------------------------------------------- per-op report
    op_rep = {}
    for name, _, bts in ops:
        st = op_st[name]
        ms = st["mean"]
        gbs = bts / (ms * 1e-3) / 1e9
        r = {"ms": round(ms, 4), "median_ms": round(st["median"], 4),
             "p10_ms": round(st["p10"], 4), "p90_ms": round(st["p90"], 4),
             "GB_s": round(gbs, 1), "Gelem_s": round(n / (ms * 1e-3) / 1e9, 2),
             "frac_hbm": round(gbs / PEAK_GBS, 4), "algorithmic_bytes": int(bts)}
        if name in base_ms:
            r["nondet_baseline_ms"] = round(base_ms[name], 4)
            r["det_overhead"] = round(ms / base_ms[name] - 1.0, 4)
            r["nondet_baseline"] = {"sum": "atomic tail (one float atomic per workgroup)",
                                    "scan": "the same scan kernel with the adaptive look-back",
                                    "scatter": "one float atomic per element"}[name]
        if name == "scan" and "scan_library" in base_ms:
            r["rocm_library_scan_ms"] = round(base_ms["scan_library"], 4)
            r["det_overhead_vs_library"] = round(ms / base_ms["scan_library"] - 1.0, 4)
        if name in distinct:
            r["distinct_results"] = distinct[name]
        if name in accuracy:
            r["accuracy"] = accuracy[name]
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
        configs = time_configs(det, workloads, dev, log, bl)

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        xs = host.get("x_sum")
        xc = host.get("x_scan")
        vs, bs = host.get("v_sc"), host.get("b_sc")
        reps, dt, cpu_bytes = 0, 0.0, 0.0
        ref = {}
        while reps < 3 and dt < 10.0:
            t = time.perf_counter()
            if xs is not None:
                ref["sum"] = oracle.det_sum(xs)
            if xc is not None:
                ref["scan"] = oracle.scan(xc)
            if vs is not None:
                ref["scatter"] = oracle.scatter_add(vs, bs, np.zeros(B, np.float32))[0]
            dt += time.perf_counter() - t
            cpu_bytes += step_bytes
            reps += 1
        hi = host_info()
        cpu = {"value": round(cpu_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"the whole step's workload ({', '.join(sorted(only))} at n=2^{args.log2n}, "
                         f"{B} bins) run {reps} time(s) through the single-threaded C oracle: "
                         f"{dt:.1f} s on one of {hi['usable_cores']} usable host cores",
               "host": hi}
        log(f"cpu oracle: {reps} pass(es), {dt:.1f}s")
        # the same oracle functions over independent units on OpenMP threads (same bits)
        preps, pdt, pbytes, same = 0, 0.0, 0.0, True
        while preps < 5 and pdt < 5.0:
            t = time.perf_counter()
            got = {}
            if xs is not None:
                got["sum"] = oracle.par_det_sum(xs)
            if xc is not None:
                got["scan"] = oracle.par_scan(xc)
            if vs is not None:
                got["scatter"] = oracle.par_scatter_add(vs, bs, np.zeros(B, np.float32))[0]
            pdt += time.perf_counter() - t
            pbytes += step_bytes
            preps += 1
            for k, v in got.items():
                same = same and np.asarray(v).tobytes() == np.asarray(ref[k]).tobytes()
        cpu["parallel"] = {"value": round(pbytes / pdt / 1e9, 3), "unit": "GB/s",
                           "cores": oracle.par_threads(), "kind": "oracle, OpenMP driver",
                           "same_bits_as_single_thread": bool(same),
                           "sample": f"the same workload run {preps} time(s) with aligned sum "
                                     f"chunks, destinations and scan tiles on "
                                     f"{oracle.par_threads()} threads: {pdt:.1f} s"}
        log(f"cpu oracle, {oracle.par_threads()} threads: {preps} pass(es), {pdt:.1f}s, "
            f"same bits: {same}")

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
        "attainable": attainable,
        "kernels": kern_rep,
        "ops": op_rep,
        "cpu_baseline": cpu,
        "configs": configs,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
