// det_internal.h -- host-side declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "det.h"

namespace det {

// Launch overrides for the shape-invariance tests (0 = default).
struct LaunchOverride {
    int grid_wgs;        // workgroups of the sum and look-back scan kernels
    int extra_lds;       // dynamic LDS bytes added to k_scan, k_sum_chunks and the radix kernels
    int sum_chunk_log2;
    int scan_A;          // test-only scan anchor constants (0 = the spec's)
    int scan_A2;
    uint32_t delay_seed; // test-only: seeded delays before the scan's status publications
    uint32_t delay_us;   //   (at most this many microseconds each; 0 = none)
};
const LaunchOverride& launch_override();
constexpr int kMaxExtraLds = 65536;   // largest extra_lds the test hook accepts

// What the most recent launches used (for the tests that show the launch shape changed).
void note_sum_grid(int64_t grid);
void note_scan_grid(int64_t grid, int64_t per_cu);

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline size_t dtype_size(det_dtype d) { return d == DET_F64 ? 8 : 4; }   // f32, i32: 4

// ---- sum
size_t sum_workspace(int64_t n, det_dtype dt);
det_status sum_launch(const void* x, int64_t n, det_dtype dt, void* out, void* ws, size_t ws_bytes,
                      hipStream_t s);
// det_sum with the partials in the library's own per-GPU array (no workspace argument)
constexpr size_t kSumNoAllocBytes = ((size_t)1 << 20) + ((size_t)1 << 14) + 256;
constexpr int kMaxDevices = 64;
det_status sum_noalloc_launch(const void* x, int64_t n, det_dtype dt, void* out, hipStream_t s);

// ---- scan
constexpr int kScanV = 32;       // elements per lane
constexpr int kScanW = 64;       // lanes per wave
constexpr int kScanWaves = 4;    // waves per tile
constexpr int kScanL = kScanW * kScanWaves;   // lanes per tile
constexpr int kScanT = kScanV * kScanL;       // elements per tile
constexpr int kScanA = 256;      // tiles per anchor interval
constexpr int kScanA2 = 256;     // anchor intervals per super-interval

size_t scan_workspace(int64_t n, det_dtype dt, unsigned flags, int64_t num_segments);
det_status scan_error(const void* ws, int32_t* out, hipStream_t s);
det_status scan_launch(const void* x, void* y, int64_t n, det_dtype dt, unsigned flags,
                       const int64_t* offs, int64_t nseg, void* ws, size_t ws_bytes,
                       hipStream_t s);

// ncols scans of n elements each (column c: x + c * n -> y + c * n) sharing flags and offsets,
// with the bits of ncols separate scan_launch calls; ws: the workspace of one n-element scan;
// cagg: scan_columns_agg_bytes(n, ncols) more bytes (tile totals of every column), 256-aligned.
det_status scan_columns_launch(const void* x, void* y, int64_t n, int64_t ncols, det_dtype dt,
                               unsigned flags, const int64_t* offs, int64_t nseg, void* ws,
                               void* cagg, hipStream_t s);
size_t scan_columns_agg_bytes(int64_t n, int64_t ncols);

// ---- scatter-add
size_t scatter_workspace(int64_t n, int64_t num_out, int64_t row_len, det_dtype dt);
// negate: every value enters negated (scatter-subtract)
det_status scatter_launch(const void* values, const int32_t* index, int64_t n, int64_t row_len,
                          det_dtype dt, void* out, int64_t num_out, void* prev, int64_t* n_skipped,
                          void* ws, size_t ws_bytes, bool negate, hipStream_t s);

// scatter-add whose prev is the running value (prev required; arguments checked by the caller)
size_t scatter_running_workspace(int64_t n, int64_t num_out, int64_t row_len, det_dtype dt);
det_status scatter_running_launch(const void* values, const int32_t* index, int64_t n,
                                  int64_t row_len, det_dtype dt, void* out, int64_t num_out,
                                  void* prev, int64_t* n_skipped, void* ws, hipStream_t s);

// Workgroups of `block` threads of kernel `fn` with `dyn_lds` bytes of dynamic LDS that are
// resident on the current device at once (occupancy x compute units), cached per device,
// kernel and LDS size; 0 if the runtime cannot tell.  *per_cu (optional) receives the
// occupancy per compute unit.
int64_t resident_wgs(const void* fn, int block, int dyn_lds = 0, int* per_cu = nullptr);

// Compute units of the current device (cached per device); 0 if the runtime cannot tell.
int cu_count();

// Kernel timing (a test hook): while it is switched on, a KernelTimer brackets one launch with
// two HIP events on the launch's stream; det_debug_kernel_report reads them.  Off, it costs one
// relaxed load.
class KernelTimer {
  public:
    KernelTimer(const char* name, hipStream_t s);
    ~KernelTimer();
    KernelTimer(const KernelTimer&) = delete;
    KernelTimer& operator=(const KernelTimer&) = delete;

  private:
    hipStream_t s_;
    long slot_;
    unsigned gen_;
};

inline det_status launch_status() {
    return hipGetLastError() == hipSuccess ? DET_SUCCESS : DET_ERROR_LAUNCH;
}

}  // namespace det
