/*
 * det.h -- reproducible floating-point add-reductions on AMD Instinct MI355X (gfx950).
 *
 * Three operations whose result bits depend only on (op, flags, dtype, input): never on the
 * grid, occupancy, CU count, stream, run or device.  Every addition is one IEEE-754
 * round-to-nearest-even addition in the input dtype (no contraction, subnormals kept); the
 * association order is fixed by the problem size alone:
 *
 *  PW(v)   adjacent-pair tree: pad v with -0.0 to a power of two, then replace the list by
 *          v0+v1, v2+v3, ... until one value remains (course page "Floating point and
 *          reproducibility", section "Fix the order of every addition": a fixed bracket over
 *          pairs instead of an atomic tail).
 *
 * Conventions for every entry point:
 *  - Data pointers are DEVICE pointers owned by the caller.  Any element-aligned address is
 *    accepted (tensor views); alignment never changes the bits.  A data pointer that is not
 *    aligned to its element size is rejected with DET_ERROR_INVALID_VALUE.
 *  - The library never allocates and never synchronises.  Scratch memory is a caller-provided
 *    device workspace of at least *_workspace_size(...) bytes, 256-byte aligned (else
 *    DET_ERROR_WORKSPACE; torch's and hipMalloc's allocations are); its contents
 *    on entry do not matter and are undefined on return.  Calls that overlap in time must not
 *    share a workspace.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the call
 *    returns without waiting for it.
 *  - Host-checkable problems return a status and enqueue nothing.  Data-dependent conditions
 *    never fail: out-of-range scatter indices are skipped and counted.
 *  - Sizes: 0 <= n <= DET_MAX_N (2^31 - 1), as scatter record slots are signed 32-bit
 *    (Warp "Deterministic Execution", section "Limitations", large launches).
 *  - No C++ exception crosses this interface.
 */
#ifndef DET_H
#define DET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* DET_I32 is accepted by det_scan only (Warp "Deterministic Execution", section "Pattern 2:
 * Slot Allocation": the count-scan-write workflow's prefix scan over int32 slot counts); its
 * sums wrap modulo 2^32 as two's complement, which no association order can change. */
typedef enum { DET_F32 = 0, DET_F64 = 1, DET_I32 = 2 } det_dtype;

typedef enum {
    DET_SUCCESS = 0,
    DET_ERROR_INVALID_VALUE = 1, /* bad argument (negative size, NULL pointer, bad flags...) */
    DET_ERROR_UNSUPPORTED = 2,   /* unknown dtype */
    DET_ERROR_TOO_LARGE = 3,     /* n or a derived size beyond DET_MAX_N */
    DET_ERROR_WORKSPACE = 4,     /* ws NULL, not 256-byte aligned, or smaller than the
                                    matching *_workspace_size */
    DET_ERROR_LAUNCH = 5         /* the HIP runtime refused a launch */
} det_status;

#define DET_MAX_N 2147483647LL

/* det_scan flags (inclusive and forward when 0) */
#define DET_SCAN_EXCLUSIVE 1u
#define DET_SCAN_REVERSE 2u

/* ------------------------------------------------------------------ sum */

/* Bytes of workspace det_sum needs for n elements (0 when the arguments are invalid). */
size_t det_sum_workspace_size(int64_t n, det_dtype dtype);

/* *out = PW(x[0..n)) for n >= 1, +0.0 for n == 0.
 * x:   device, n elements of dtype (read only).
 * out: device, one element of dtype (written).
 * The fixed tree replaces the atomic tail of a block-partials reduction (course page
 * "Floating point and reproducibility", sections "Twenty answers, none of them wrong" and
 * "Fix the order of every addition").  Any aligned power-of-two chunk of x is a subtree of
 * PW, so the kernels may split x into chunks of any power-of-two size without moving a bit.
 * ws: device, at least det_sum_workspace_size(n, dtype) bytes, 256-byte aligned, any initial
 * contents; the call leaves it holding partial values.  Sums of 2 to 1024 chunks of 2^14
 * elements (up to 2^24 elements) finish in one launch: the grid's last workgroup waits for
 * the chunk values tagged for the call, a wait bounded at 2 seconds of the GPU's 100 MHz
 * clock after which *out receives a NaN instead of the sum (a failure of the GPU's forward
 * progress, not of the data).  Calls that share a workspace must be ordered on one stream. */
det_status det_sum(const void* x, int64_t n, det_dtype dtype, void* out, void* ws,
                   size_t ws_bytes, void* stream);

/* det_sum for callers that cannot allocate device memory (code under HIP graph capture that
 * must not call hipMalloc, tight serving loops, harnesses that forbid allocation): no
 * workspace argument and no allocation; the result bits are det_sum's.
 * x, out, n, dtype, stream and the errors are det_sum's (n up to DET_MAX_N, beyond it
 * DET_ERROR_TOO_LARGE); DET_ERROR_LAUNCH if the runtime cannot give the array's address.
 * The partial sums live in a static device array of DET_SUM_NOALLOC_SCRATCH_BYTES bytes, one
 * per GPU the library runs on, loaded with the library's code and held until the process
 * ends; that size covers every n up to DET_MAX_N in f32 and f64.  Every call on one GPU uses
 * that GPU's single array, which keeps the last call's partials: calls that overlap in time
 * on one GPU (different streams or host threads without ordering) race and give unspecified
 * results.  Calls ordered on one stream are safe. */
#define DET_SUM_NOALLOC_SCRATCH_BYTES (1048576 + 16384 + 256)
det_status det_sum_noalloc(const void* x, int64_t n, det_dtype dtype, void* out, void* stream);

/* ------------------------------------------------------------------ scan */

/* Bytes of workspace det_scan needs. */
size_t det_scan_workspace_size(int64_t n, det_dtype dtype, unsigned flags, int64_t num_segments);

/* Prefix sum with look-back through fixed anchor intervals (drjit-core pull request "Make
 * CUDA floating-point prefix sums deterministic", sections "Root cause" and
 * "Implementation"; inclusive/exclusive, forward/reverse, full/segmented per "Validation").
 *
 * Order (constants from det_spec_constants: V = 32 elements per lane, W = 64 lanes per wave,
 * 4 waves per tile, T = 8192 elements per tile, A = 256 tiles per anchor interval, A2 = 256
 * intervals per super-interval):
 *   lane-serial prefix s over each lane's run of V elements; Kogge-Stone over the lane totals
 *   inside each wave (p = lane-exclusive prefix); Kogge-Stone over the 4 wave totals
 *   (P = wave-exclusive prefix; the last value is the tile total Agg_j); for tile j in anchor
 *   interval q of super-interval Q: W_j = PW(Agg_{qA..j-1}); interval totals
 *   G_q = PW(all Agg of q); WG = PW(G_{Q*A2..q-1}); super-interval carries CC_0 = -0.0,
 *   CC_{Q+1} = CC_Q + PW(all G of Q); y = ((((CC_Q + WG) + W_j) + P) + p) + s.  Only fixed
 *   anchors publish totals and carries, so the bits do not depend on which predecessors a tile
 *   saw as finished.
 *
 * dtype DET_I32: int32 elements, sums wrapping modulo 2^32 (the same dataflow; every order
 *         gives the same integers), the exclusive scan's first value 0.
 * x, y:   device, n elements of dtype.  Inclusive scans may run in place (y == x); exclusive
 *         scans must not overlap x and y (DET_ERROR_INVALID_VALUE if the ranges overlap).
 * flags:  DET_SCAN_EXCLUSIVE (y[0] = +0.0, y[i] = inclusive[i-1]) and/or DET_SCAN_REVERSE
 *         (scan of the flipped array, flipped back).
 * seg_offsets: NULL for one segment, else device int64 [num_segments + 1] with
 *         0 = o_0 <= o_1 <= ... <= o_S = n (precondition, not checked on the device).  Each
 *         segment restarts the scan: the head-flag operator (f1|f2, f2 ? b : a + b) runs
 *         through the same order; exclusive scans write +0.0 at every segment head (for
 *         reverse: at every segment's last element).  num_segments >= 1 when n > 0. */
det_status det_scan(const void* x, void* y, int64_t n, det_dtype dtype, unsigned flags,
                    const int64_t* seg_offsets, int64_t num_segments, void* ws, size_t ws_bytes,
                    void* stream);

/* Health word of the last det_scan run in workspace ws, for callers that want to verify it.
 * A scan of more than one anchor interval (more than 256 * 8192 elements) waits on status words
 * that earlier tiles publish.  Each such wait is bounded: after 2 seconds of the GPU's constant
 * 100 MHz clock it gives up, sets this word and leaves y unspecified while det_scan has already
 * returned DET_SUCCESS.  Any failure of the kernel's forward progress (a broken offsets
 * precondition, a hardware fault, a scheduler that never runs a workgroup holding a claimed
 * tile) ends that way, never in a hang; a silent wrong result is possible only if a status
 * word arrives corrupted yet tagged ready.  Shorter and empty scans never wait and leave the
 * word at 0.
 * Enqueues on `stream` a copy of the word into *out (device int32: 0 = every wait ended
 * normally, 1 = some wait gave up); returns without waiting.  ws: the workspace the scan used
 * (device); out: device int32 (written).  DET_ERROR_INVALID_VALUE for NULL. */
det_status det_scan_error(const void* ws, int32_t* out, void* stream);

/* ------------------------------------------------------------------ scatter-add */

/* Bytes of workspace det_scatter_add needs. */
size_t det_scatter_add_workspace_size(int64_t n, int64_t num_out, int64_t row_len,
                                      det_dtype dtype);

/* Keyed scatter-add along axis 0, the reproducible form of atomic_add(out, index[i],
 * values[i]) (Warp "Deterministic Execution", sections "Pattern 1: Accumulation" and
 * "Writing Manual Deterministic Code") and, for row_len > 1, of the row-indexed tile
 * accumulate (Warp reference "warp.tile_atomic_add_indexed").
 *
 * For destination r and column c: M = [values[i*row_len + c] for ascending i with
 * index[i] == r]; if M is non-empty, out[r*row_len + c] = out[r*row_len + c] + PW(M), else
 * out is left untouched.
 *
 * values:  device, [n * row_len] of dtype, row-major (read only; must not alias out).
 * index:   device int32 [n].  Entries outside [0, num_out) are skipped, never an error.
 * out:     device, [num_out * row_len] of dtype, updated in place.
 * prev:    NULL, or device [n * row_len]: for every valid i, the destination row as it was
 *          before this call (rows of skipped i are not written).
 * n_skipped: NULL, or device int64: set (not accumulated) to the number of skipped i.
 * row_len: >= 1. */
det_status det_scatter_add(const void* values, const int32_t* index, int64_t n, int64_t row_len,
                           det_dtype dtype, void* out, int64_t num_out, void* prev,
                           int64_t* n_skipped, void* ws, size_t ws_bytes, void* stream);

/* Keyed scatter-subtract, the reproducible form of atomic_sub(out, index[i], values[i]): the
 * values are negated and then added in the order of det_scatter_add (Warp "Deterministic
 * Execution", section "Pattern 1: Accumulation", its table of atomics).  So for destination r
 * and column c, out = out + PW(-M) with every element of M negated on its own; this is not
 * out - PW(M) where a destination's contributions cancel to zero (the zero's sign differs).
 * Arguments, workspace (det_scatter_add_workspace_size), ownership and errors as for
 * det_scatter_add; prev receives the destination rows before the call. */
det_status det_scatter_sub(const void* values, const int32_t* index, int64_t n, int64_t row_len,
                           det_dtype dtype, void* out, int64_t num_out, void* prev,
                           int64_t* n_skipped, void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace det_scatter_add_running needs (0 when the arguments are invalid). */
size_t det_scatter_add_running_workspace_size(int64_t n, int64_t num_out, int64_t row_len,
                                              det_dtype dtype);

/* det_scatter_add whose prev is the running value: what a loop of atomic adds in ascending
 * source index would hand back to each source, with the sum of the earlier contributions
 * formed in a fixed order.  The Warp reference "warp.tile_atomic_add_indexed" returns the
 * destination rows as they were before the accumulate and leaves them unspecified under
 * repeated indices; this entry point fixes them.
 *
 * Order: lay the members of every destination (ascending source index, as in
 * det_scatter_add) end to end in destination order, one segment per destination, and take
 * E = the forward exclusive segmented det_scan of each column of that array.  The member at
 * position g of that array, source row i, destination r, gets
 *   prev[i*row_len + c] = out[r*row_len + c]          at r's first position,
 *   prev[i*row_len + c] = out[r*row_len + c] + E[g]   elsewhere
 * (out as before the call).  out receives exactly what det_scatter_add gives it.
 *
 * values, index, out, n_skipped, row_len: as for det_scatter_add.
 * prev:    device [n * row_len] of dtype, required when n > 0 (rows of skipped i are not
 *          written); must not overlap values or out (DET_ERROR_INVALID_VALUE).
 * row_len: 1 .. 65535 * 32 (DET_ERROR_TOO_LARGE beyond).
 * Workspace: det_scatter_add_running_workspace_size bytes, about 2 * n * row_len elements
 * more than det_scatter_add's (f32 with row_len 1 and more than 2^21 members, whose values
 * travel through the sort beside their source indices and whose prev goes out through windows
 * of the source index: about 7 * n 4-byte words more).  The columns are scanned in one launch
 * when each fits one anchor interval of tiles, else one scan per column. */
det_status det_scatter_add_running(const void* values, const int32_t* index, int64_t n,
                                   int64_t row_len, det_dtype dtype, void* out, int64_t num_out,
                                   void* prev, int64_t* n_skipped, void* ws, size_t ws_bytes,
                                   void* stream);

/* ------------------------------------------------------------------ introspection */

/* Version of the association order; results of one version never change. */
int det_spec_version(void);

/* Scan constants of this version: elements per lane, lanes per tile, tiles per anchor
 * interval, anchor intervals per super-interval (any pointer may be NULL). */
void det_spec_constants(int64_t* V, int64_t* L, int64_t* A, int64_t* A2);

/* Static string naming a status code. */
const char* det_status_string(det_status s);

/* ------------------------------------------------------------------ test hooks */

/* Not part of the stable interface.  Overrides how the work is spread over the GPU, for the
 * tests that show the bits depend on neither the block count nor the occupancy:
 *   grid_wgs > 0 sets the number of workgroups of the sum kernel and of the look-back scan
 *     kernel, also beyond the number that fit on the GPU at once (workgroups that start late
 *     claim their tiles when they start); 0 = the default;
 *   extra_lds_bytes in [0, 65536] adds that much dynamic LDS to every workgroup of the sum,
 *     look-back scan and radix-sort kernels, which lowers how many fit per compute unit.
 * Process-wide; DET_ERROR_INVALID_VALUE when out of range. */
det_status det_debug_set_launch(int grid_wgs, int extra_lds_bytes);

/* Not part of the stable interface.  chunk_log2 in [14, 24] sets the elements per partial of
 * the sum's first level (0 = default, 14).  Process-wide; DET_ERROR_INVALID_VALUE when out of
 * range. */
det_status det_debug_set_sum_chunk(int chunk_log2);

/* Not part of the stable interface.  The launch shape the library last used: the grid of the
 * sum kernel's first level, the grid of the look-back scan kernel and the scan workgroups the
 * runtime reported resident per compute unit for that launch (with its extra LDS).  Any
 * pointer may be NULL; values are 0 before the first such launch. */
void det_debug_last_launch(int64_t* sum_grid, int64_t* scan_grid, int64_t* scan_per_cu);

/* Not part of the stable interface.  Seeded pauses in the look-back scan: with max_us > 0,
 * the publishing thread of one status publication in four (tile totals, interval totals,
 * super-interval carries) first pauses for a time in [0, max_us] microseconds chosen by a
 * hash of seed, tile and publication kind, so successors find predecessors' status words
 * ready or not at different moments (drjit-core pull request "Make CUDA floating-point prefix
 * sums deterministic", section "Root cause": results must not depend on the states a tile
 * observes).  max_us in [0, 1000], 0 = off.  Process-wide; DET_ERROR_INVALID_VALUE when out
 * of range. */
det_status det_debug_set_scan_delay(unsigned seed, int max_us);

/* Not part of the stable interface.  Replaces the scan's anchor constants (tiles per anchor
 * interval A, intervals per super-interval A2; each in [1, 256], 0 = the spec's 256) so tests
 * can exercise many intervals and super-interval carries at small n against the oracle run
 * with the same constants.  Results then follow that variant's order, not SPEC v1.
 * Process-wide; DET_ERROR_INVALID_VALUE when out of range. */
det_status det_debug_set_scan_anchors(int A, int A2);

/* Not part of the stable interface.  Kernel timing for benchmarks: while enabled, every kernel
 * the library enqueues is bracketed by two HIP events recorded on the call's stream.
 * enable = 1 drops earlier records and starts recording, 0 drops them and stops; anything else
 * is DET_ERROR_INVALID_VALUE.  Recording adds an event pair per launch. */
det_status det_debug_kernel_timing(int enable);

/* Not part of the stable interface.  Waits for every recorded event pair, then writes one line
 * per kernel name, "name launches total_ms average_ms", into buf (at most len bytes including
 * the terminating NUL; buf may be NULL).  The records stay until det_debug_kernel_timing is
 * called again.  Launches whose events failed are counted in a last line starting with '#'.
 * Returns the bytes the full report needs, NUL included. */
size_t det_debug_kernel_report(char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* DET_H */
