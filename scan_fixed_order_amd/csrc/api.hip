// api.hip -- the library's C interface: argument checks, workspace sizing, dispatch.
//
// Every check that needs no device data happens here, before anything is enqueued; the
// kernels never see an argument this file rejected.
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "det_internal.h"

namespace det {

static_assert(DET_SUM_NOALLOC_SCRATCH_BYTES == kSumNoAllocBytes,
              "the header and the library disagree on the no-allocation array's size");

static LaunchOverride g_override = {0, 0, 0, 0, 0, 0u, 0u};

const LaunchOverride& launch_override() { return g_override; }

static std::atomic<int64_t> g_last_sum_grid{0}, g_last_scan_grid{0}, g_last_scan_per_cu{0};

void note_sum_grid(int64_t grid) { g_last_sum_grid.store(grid, std::memory_order_relaxed); }

void note_scan_grid(int64_t grid, int64_t per_cu) {
    g_last_scan_grid.store(grid, std::memory_order_relaxed);
    g_last_scan_per_cu.store(per_cu, std::memory_order_relaxed);
}

int64_t resident_wgs(const void* fn, int block, int dyn_lds, int* per_cu_out) {
    struct Entry {
        int dev;
        const void* fn;
        int block, lds, per_cu;
        int64_t wgs;
    };
    static std::mutex mu;
    static Entry cache[128];
    static int used = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].dev == dev && cache[i].fn == fn && cache[i].block == block &&
            cache[i].lds == dyn_lds) {
            if (per_cu_out) *per_cu_out = cache[i].per_cu;
            return cache[i].wgs;
        }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, (size_t)dyn_lds) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (per_cu < 1) per_cu = 1;
    const int64_t wgs = (int64_t)per_cu * cus;
    if (used < 128) cache[used++] = Entry{dev, fn, block, dyn_lds, per_cu, wgs};
    if (per_cu_out) *per_cu_out = per_cu;
    return wgs;
}

int cu_count() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cache[dev] = cus;
    }
    return cache[dev];
}

// ---------------------------------------------------------------- kernel timing hook

namespace {
struct TimedLaunch {
    const char* name;
    hipEvent_t a, b;
};
std::mutex g_tm;
std::atomic<bool> g_timing{false};
unsigned g_gen = 0;                    // bumped whenever the records are dropped
std::vector<TimedLaunch> g_launches;
std::vector<hipEvent_t> g_events;      // idle events for reuse

hipEvent_t take_event() {
    if (!g_events.empty()) {
        hipEvent_t e = g_events.back();
        g_events.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

void drop_launches() {
    for (const TimedLaunch& t : g_launches) {
        if (t.a) g_events.push_back(t.a);
        if (t.b) g_events.push_back(t.b);
    }
    g_launches.clear();
    ++g_gen;
}
}  // namespace

KernelTimer::KernelTimer(const char* name, hipStream_t s) : s_(s), slot_(-1), gen_(0) {
    if (!g_timing.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lock(g_tm);
    TimedLaunch t{name, take_event(), take_event()};
    if (!t.a || !t.b || hipEventRecord(t.a, s) != hipSuccess) {
        if (t.a) g_events.push_back(t.a);
        if (t.b) g_events.push_back(t.b);
        return;
    }
    g_launches.push_back(t);
    slot_ = (long)g_launches.size() - 1;
    gen_ = g_gen;
}

KernelTimer::~KernelTimer() {
    if (slot_ < 0) return;
    std::lock_guard<std::mutex> lock(g_tm);
    if (gen_ != g_gen || slot_ >= (long)g_launches.size()) return;
    if (hipEventRecord(g_launches[slot_].b, s_) != hipSuccess) g_launches[slot_].name = nullptr;
}

static bool valid_dtype(det_dtype d) { return d == DET_F32 || d == DET_F64; }
// det_scan also takes int32 (wrapping sums: the order cannot change them)
static bool valid_scan_dtype(det_dtype d) { return valid_dtype(d) || d == DET_I32; }

static bool ranges_overlap(const void* a, const void* b, size_t bytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a);
    const uintptr_t y = reinterpret_cast<uintptr_t>(b);
    return x < y + bytes && y < x + bytes;
}

}  // namespace det

using namespace det;

namespace {
// The workspace must be 256-byte aligned (status words and counters sit on their own lines).
bool ws_aligned(const void* ws) { return (reinterpret_cast<uintptr_t>(ws) & 255u) == 0; }
// Data pointers must be aligned to their element size.
bool elem_aligned(const void* p, size_t es) { return (reinterpret_cast<uintptr_t>(p) % es) == 0; }
}  // namespace

extern "C" {

size_t det_sum_workspace_size(int64_t n, det_dtype dtype) {
    if (n < 0 || n > DET_MAX_N || !valid_dtype(dtype)) return 0;
    return sum_workspace(n, dtype);
}

det_status det_sum(const void* x, int64_t n, det_dtype dtype, void* out, void* ws,
                   size_t ws_bytes, void* stream) {
    if (!valid_dtype(dtype)) return DET_ERROR_UNSUPPORTED;
    if (n < 0) return DET_ERROR_INVALID_VALUE;
    if (n > DET_MAX_N) return DET_ERROR_TOO_LARGE;
    if (!out || (n > 0 && !x)) return DET_ERROR_INVALID_VALUE;
    if (!elem_aligned(out, dtype_size(dtype)) || !elem_aligned(x, dtype_size(dtype)))
        return DET_ERROR_INVALID_VALUE;
    if (!ws || !ws_aligned(ws) || ws_bytes < sum_workspace(n, dtype)) return DET_ERROR_WORKSPACE;
    return sum_launch(x, n, dtype, out, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

det_status det_sum_noalloc(const void* x, int64_t n, det_dtype dtype, void* out, void* stream) {
    if (!valid_dtype(dtype)) return DET_ERROR_UNSUPPORTED;
    if (n < 0) return DET_ERROR_INVALID_VALUE;
    if (n > DET_MAX_N) return DET_ERROR_TOO_LARGE;
    if (!out || (n > 0 && !x)) return DET_ERROR_INVALID_VALUE;
    if (!elem_aligned(out, dtype_size(dtype)) || !elem_aligned(x, dtype_size(dtype)))
        return DET_ERROR_INVALID_VALUE;
    return sum_noalloc_launch(x, n, dtype, out, static_cast<hipStream_t>(stream));
}

size_t det_scan_workspace_size(int64_t n, det_dtype dtype, unsigned flags, int64_t num_segments) {
    if (n < 0 || n > DET_MAX_N || !valid_scan_dtype(dtype) || num_segments < 0) return 0;
    if (flags & ~(DET_SCAN_EXCLUSIVE | DET_SCAN_REVERSE)) return 0;
    return scan_workspace(n, dtype, flags, num_segments);
}

det_status det_scan(const void* x, void* y, int64_t n, det_dtype dtype, unsigned flags,
                    const int64_t* seg_offsets, int64_t num_segments, void* ws, size_t ws_bytes,
                    void* stream) {
    if (!valid_scan_dtype(dtype)) return DET_ERROR_UNSUPPORTED;
    if (n < 0 || num_segments < 0) return DET_ERROR_INVALID_VALUE;
    if (n > DET_MAX_N || num_segments > DET_MAX_N) return DET_ERROR_TOO_LARGE;
    if (flags & ~(DET_SCAN_EXCLUSIVE | DET_SCAN_REVERSE)) return DET_ERROR_INVALID_VALUE;
    if (n > 0 && (!x || !y)) return DET_ERROR_INVALID_VALUE;
    if (seg_offsets && n > 0 && num_segments < 1) return DET_ERROR_INVALID_VALUE;
    if (!elem_aligned(x, dtype_size(dtype)) || !elem_aligned(y, dtype_size(dtype)) ||
        !elem_aligned(seg_offsets, sizeof(int64_t)))
        return DET_ERROR_INVALID_VALUE;
    const size_t bytes = (size_t)n * dtype_size(dtype);
    if ((flags & DET_SCAN_EXCLUSIVE) && n > 0 && ranges_overlap(x, y, bytes))
        return DET_ERROR_INVALID_VALUE;
    if (n > 0 && x != y && ranges_overlap(x, y, bytes)) return DET_ERROR_INVALID_VALUE;
    if (!ws || !ws_aligned(ws) || ws_bytes < scan_workspace(n, dtype, flags, num_segments))
        return DET_ERROR_WORKSPACE;
    return scan_launch(x, y, n, dtype, flags, seg_offsets, num_segments, ws, ws_bytes,
                       static_cast<hipStream_t>(stream));
}

det_status det_scan_error(const void* ws, int32_t* out, void* stream) {
    if (!ws || !out) return DET_ERROR_INVALID_VALUE;
    return scan_error(ws, out, static_cast<hipStream_t>(stream));
}

size_t det_scatter_add_workspace_size(int64_t n, int64_t num_out, int64_t row_len,
                                      det_dtype dtype) {
    if (n < 0 || n > DET_MAX_N || num_out < 0 || num_out > DET_MAX_N || row_len < 1 ||
        !valid_dtype(dtype))
        return 0;
    return scatter_workspace(n, num_out, row_len, dtype);
}

// columns of the running scatter: 32 per workgroup along the grid's y dimension (65535 at most)
constexpr int64_t kRunningMaxRowLen = 65535LL * 32;

size_t det_scatter_add_running_workspace_size(int64_t n, int64_t num_out, int64_t row_len,
                                              det_dtype dtype) {
    if (n < 0 || n > DET_MAX_N || num_out < 0 || num_out > DET_MAX_N || row_len < 1 ||
        !valid_dtype(dtype))
        return 0;
    if (row_len > kRunningMaxRowLen) return 0;
    return scatter_running_workspace(n, num_out, row_len, dtype);
}

}  // extern "C"

namespace {
bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return abytes > 0 && bbytes > 0 && a0 < b0 + bbytes && b0 < a0 + abytes;
}

det_status scatter_checked(const void* values, const int32_t* index, int64_t n, int64_t row_len,
                           det_dtype dtype, void* out, int64_t num_out, void* prev,
                           int64_t* n_skipped, void* ws, size_t ws_bytes, bool negate,
                           void* stream) {
    if (!valid_dtype(dtype)) return DET_ERROR_UNSUPPORTED;
    if (n < 0 || num_out < 0 || row_len < 1) return DET_ERROR_INVALID_VALUE;
    if (n > DET_MAX_N || num_out > DET_MAX_N) return DET_ERROR_TOO_LARGE;
    if ((double)n * (double)row_len > 9.0e18 || (double)num_out * (double)row_len > 9.0e18)
        return DET_ERROR_TOO_LARGE;
    if (n > 0 && (!values || !index)) return DET_ERROR_INVALID_VALUE;
    if (num_out > 0 && !out) return DET_ERROR_INVALID_VALUE;
    const size_t es = dtype_size(dtype);
    if (!elem_aligned(values, es) || !elem_aligned(out, es) || !elem_aligned(prev, es) ||
        !elem_aligned(index, sizeof(int32_t)) || !elem_aligned(n_skipped, sizeof(int64_t)))
        return DET_ERROR_INVALID_VALUE;
    if (n > 0 && num_out > 0) {
        const uintptr_t v0 = reinterpret_cast<uintptr_t>(values);
        const uintptr_t v1 = v0 + (size_t)n * row_len * es;
        const uintptr_t o0 = reinterpret_cast<uintptr_t>(out);
        const uintptr_t o1 = o0 + (size_t)num_out * row_len * es;
        if (v0 < o1 && o0 < v1) return DET_ERROR_INVALID_VALUE;
    }
    if (!ws || !ws_aligned(ws) || ws_bytes < scatter_workspace(n, num_out, row_len, dtype))
        return DET_ERROR_WORKSPACE;
    return scatter_launch(values, index, n, row_len, dtype, out, num_out, prev, n_skipped, ws,
                          ws_bytes, negate, static_cast<hipStream_t>(stream));
}
}  // namespace

extern "C" {

det_status det_scatter_add(const void* values, const int32_t* index, int64_t n, int64_t row_len,
                           det_dtype dtype, void* out, int64_t num_out, void* prev,
                           int64_t* n_skipped, void* ws, size_t ws_bytes, void* stream) {
    return scatter_checked(values, index, n, row_len, dtype, out, num_out, prev, n_skipped, ws,
                           ws_bytes, false, stream);
}

det_status det_scatter_sub(const void* values, const int32_t* index, int64_t n, int64_t row_len,
                           det_dtype dtype, void* out, int64_t num_out, void* prev,
                           int64_t* n_skipped, void* ws, size_t ws_bytes, void* stream) {
    return scatter_checked(values, index, n, row_len, dtype, out, num_out, prev, n_skipped, ws,
                           ws_bytes, true, stream);
}

det_status det_scatter_add_running(const void* values, const int32_t* index, int64_t n,
                                   int64_t row_len, det_dtype dtype, void* out, int64_t num_out,
                                   void* prev, int64_t* n_skipped, void* ws, size_t ws_bytes,
                                   void* stream) {
    if (!valid_dtype(dtype)) return DET_ERROR_UNSUPPORTED;
    if (n < 0 || num_out < 0 || row_len < 1) return DET_ERROR_INVALID_VALUE;
    if (n > DET_MAX_N || num_out > DET_MAX_N) return DET_ERROR_TOO_LARGE;
    if (row_len > kRunningMaxRowLen) return DET_ERROR_TOO_LARGE;
    if ((double)n * (double)row_len > 9.0e18 || (double)num_out * (double)row_len > 9.0e18)
        return DET_ERROR_TOO_LARGE;
    if (n > 0 && (!values || !index || !prev)) return DET_ERROR_INVALID_VALUE;
    if (num_out > 0 && !out) return DET_ERROR_INVALID_VALUE;
    const size_t es = dtype_size(dtype);
    if (!elem_aligned(values, es) || !elem_aligned(out, es) || !elem_aligned(prev, es) ||
        !elem_aligned(index, sizeof(int32_t)) || !elem_aligned(n_skipped, sizeof(int64_t)))
        return DET_ERROR_INVALID_VALUE;
    const size_t vbytes = (size_t)n * row_len * es, obytes = (size_t)num_out * row_len * es;
    if (overlaps(values, vbytes, out, obytes) || overlaps(prev, vbytes, out, obytes) ||
        overlaps(prev, vbytes, values, vbytes))
        return DET_ERROR_INVALID_VALUE;
    if (!ws || !ws_aligned(ws) ||
        ws_bytes < scatter_running_workspace(n, num_out, row_len, dtype))
        return DET_ERROR_WORKSPACE;
    return scatter_running_launch(values, index, n, row_len, dtype, out, num_out, prev, n_skipped,
                                  ws, static_cast<hipStream_t>(stream));
}

int det_spec_version(void) { return 1; }

void det_spec_constants(int64_t* V, int64_t* L, int64_t* A, int64_t* A2) {
    if (V) *V = kScanV;
    if (L) *L = kScanL;
    if (A) *A = kScanA;
    if (A2) *A2 = kScanA2;
}

const char* det_status_string(det_status s) {
    switch (s) {
        case DET_SUCCESS: return "DET_SUCCESS";
        case DET_ERROR_INVALID_VALUE: return "DET_ERROR_INVALID_VALUE";
        case DET_ERROR_UNSUPPORTED: return "DET_ERROR_UNSUPPORTED";
        case DET_ERROR_TOO_LARGE: return "DET_ERROR_TOO_LARGE";
        case DET_ERROR_WORKSPACE: return "DET_ERROR_WORKSPACE";
        case DET_ERROR_LAUNCH: return "DET_ERROR_LAUNCH";
    }
    return "DET_UNKNOWN_STATUS";
}

det_status det_debug_set_launch(int grid_wgs, int extra_lds_bytes) {
    if (grid_wgs < 0 || extra_lds_bytes < 0 || extra_lds_bytes > kMaxExtraLds)
        return DET_ERROR_INVALID_VALUE;
    g_override.grid_wgs = grid_wgs;
    g_override.extra_lds = extra_lds_bytes;
    return DET_SUCCESS;
}

det_status det_debug_set_sum_chunk(int chunk_log2) {
    if (chunk_log2 != 0 && (chunk_log2 < 14 || chunk_log2 > 24)) return DET_ERROR_INVALID_VALUE;
    g_override.sum_chunk_log2 = chunk_log2;
    return DET_SUCCESS;
}

void det_debug_last_launch(int64_t* sum_grid, int64_t* scan_grid, int64_t* scan_per_cu) {
    if (sum_grid) *sum_grid = g_last_sum_grid.load(std::memory_order_relaxed);
    if (scan_grid) *scan_grid = g_last_scan_grid.load(std::memory_order_relaxed);
    if (scan_per_cu) *scan_per_cu = g_last_scan_per_cu.load(std::memory_order_relaxed);
}

det_status det_debug_set_scan_delay(unsigned seed, int max_us) {
    if (max_us < 0 || max_us > 1000) return DET_ERROR_INVALID_VALUE;
    g_override.delay_seed = seed;
    g_override.delay_us = (uint32_t)max_us;
    return DET_SUCCESS;
}

det_status det_debug_set_scan_anchors(int A, int A2) {
    if (A < 0 || A > kScanA || A2 < 0 || A2 > kScanA2) return DET_ERROR_INVALID_VALUE;
    g_override.scan_A = A;
    g_override.scan_A2 = A2;
    return DET_SUCCESS;
}

det_status det_debug_kernel_timing(int enable) {
    if (enable != 0 && enable != 1) return DET_ERROR_INVALID_VALUE;
    std::lock_guard<std::mutex> lock(g_tm);
    drop_launches();
    g_timing.store(enable == 1, std::memory_order_relaxed);
    return DET_SUCCESS;
}

size_t det_debug_kernel_report(char* buf, size_t len) {
    std::map<std::string, std::pair<long, double>> agg;   // name -> launches, total ms
    std::string out;
    long failed = 0;
    hipError_t last = hipSuccess;
    {
        std::lock_guard<std::mutex> lock(g_tm);
        for (const TimedLaunch& t : g_launches) {
            float ms = 0.f;
            hipError_t e1 = t.name ? hipEventSynchronize(t.b) : hipErrorInvalidValue;
            hipError_t e2 = e1 == hipSuccess ? hipEventElapsedTime(&ms, t.a, t.b) : e1;
            if (e2 != hipSuccess) {
                ++failed;
                last = e2;
                continue;
            }
            auto& e = agg[t.name];
            e.first += 1;
            e.second += ms;
        }
    }
    if (failed) {
        char line[256];
        snprintf(line, sizeof line, "# %ld launch(es) not timed: %s\n", failed,
                 hipGetErrorString(last));
        out += line;
    }
    for (const auto& kv : agg) {
        char line[256];
        snprintf(line, sizeof line, "%s %ld %.6f %.6f\n", kv.first.c_str(), kv.second.first,
                 kv.second.second, kv.second.second / (double)kv.second.first);
        out += line;
    }
    if (buf && len > 0) {
        const size_t m = out.size() < len - 1 ? out.size() : len - 1;
        memcpy(buf, out.data(), m);
        buf[m] = '\0';
    }
    return out.size() + 1;
}

}  // extern "C"
