// scan.hip -- det_scan: single-pass prefix sum with look-back through fixed anchor intervals.
//
// Order (drjit-core pull request "Make CUDA floating-point prefix sums deterministic",
// sections "Root cause" and "Implementation"; the in-tile order is this library's own):
//   tile j = 8192 elements = 4 waves x 64 lanes x 32 elements; lane t owns 32 consecutive
//   elements.
//   s      lane-serial inclusive prefix of the lane's run;
//   p      Kogge-Stone over the lane totals inside the wave (offsets 1..32), shifted one lane;
//   P      Kogge-Stone over the 4 wave totals (offsets 1, 2), shifted one wave;
//   Agg_j  the tile total (last wave-level value), published at once;
//   W_j    PW(Agg_{qA} .. Agg_{j-1}) over the earlier tiles of the same anchor interval
//          q = j / 256 (each of 256 threads reads one predecessor's status slot);
//   G_q    PW(all 256 Agg of interval q), published by the interval's last tile (its anchor),
//          which needs nothing from earlier intervals;
//   WG     PW(G_{Q*256} .. G_{q-1}) over the earlier intervals of super-interval Q = q / 256;
//   CC_Q   carry into super-interval Q: CC_0 = -0.0, CC_{Q+1} = CC_Q + PW(all 256 G of Q),
//          published by the super-interval's last tile; the only serial chain, one link per
//          2^29 elements;
//   y      ((((CC_Q + WG) + W_j) + P) + p) + s.
// A tile never reads an inclusive prefix of a non-anchor predecessor, so whether a
// predecessor was seen as finished or not cannot change the association order.
//
// Status slots are 64-bit words (tag << 32 | payload): tag bit 0 = ready, bit 1 = segment
// head seen; f64 payloads take two words, each carrying the tag.  Every word validates itself,
// so relaxed agent-scope atomics suffice and no fence is needed.  The slots and the tile
// counters are cleared by a small kernel before each scan.
//
// Segmented scans run the pair operator (f1 | f2, f2 ? b : a + b) through the same dataflow;
// the head flags come from a bitmap marked before the scan (k_mark_heads), each tile loading
// its 257 words with its data (a scan of at most 3 tiles searches the offsets instead).
// Reverse scans read and write through mirrored indices (n - 1 - f); exclusive scans store
// each inclusive value one position later (and +0.0 at position 0 and at segment heads).
// Tiles are loaded coalesced and turned into lane runs through LDS; every output is written
// with 16-byte non-temporal stores.
#include "scan_kernels.h"

namespace det {
namespace {

// Workspace header: the tile counters, the error word and the dummy load line, each on lines
// of their own.
constexpr size_t kErrOff = (size_t)(kCounters * kCounterStride * 4);
constexpr size_t kDummyOff = kErrOff + 256;
constexpr size_t kHeader = kDummyOff + 256;

struct Layout {
    int64_t ntiles, nq, nQ;
    size_t agg_off, g_off, carry_off, used, hb_off, hb_words, clear, total;
};

// Slots for tile totals, interval totals and super-interval carries.  The reservation assumes
// the smallest anchors (A = A2 = 1) so the test hook never needs a larger workspace; only the
// part the current constants use is cleared.
// seg: room for the head bitmap (256 words per tile and one more), right after the status
// slots in use, so one clear covers both
Layout layout(int64_t n, det_dtype dt, int A, int A2, bool seg) {
    Layout L;
    const size_t sw = dt == DET_F64 ? 2 : 1;
    L.ntiles = (n + kT - 1) / kT;
    L.nq = (L.ntiles + A - 1) / A;
    L.nQ = (L.nq + A2 - 1) / A2;
    const size_t tile_bytes = round_up((size_t)L.ntiles * sw * 8, 256);
    const size_t worst = round_up((size_t)(L.ntiles + 1) * sw * 8, 256);
    L.agg_off = kHeader;
    L.g_off = L.agg_off + tile_bytes;
    L.carry_off = L.g_off + tile_bytes;
    L.used = L.carry_off + round_up((size_t)(L.nQ + 1) * sw * 8, 256);
    L.hb_off = L.used;
    L.hb_words = seg ? (size_t)L.ntiles * (kHeadWords - 1) + 1 : 0;
    L.clear = L.hb_off + round_up(L.hb_words * 4, 256);
    L.total = L.clear > L.carry_off + worst ? L.clear : L.carry_off + worst;
    return L;
}

// Clears words [from, to) of the workspace (bytes, multiples of 8), then, for a segmented scan,
// marks the heads into the bitmap of L.
det_status clear_and_mark(char* ws, size_t from, size_t to, const Layout& L,
                          const int64_t* offs, int64_t nseg, int64_t n, bool rev, hipStream_t s) {
    const int64_t words = (int64_t)((to - from) / 8);
    if (words > 0) {
        int zg = (int)((words + 255) / 256);
        if (zg > 1024) zg = 1024;
        KernelTimer kt("k_zero_words", s);
        k_zero_words<<<zg, 256, 0, s>>>(reinterpret_cast<uint64_t*>(ws + from), words);
    }
    det_status st = launch_status();
    if (st != DET_SUCCESS || !offs) return st;
    int64_t g = (nseg + 1 + 255) / 256;
    if (g > 16384) g = 16384;
    {
        KernelTimer kt("k_mark_heads", s);
        k_mark_heads<<<(unsigned)g, 256, 0, s>>>(offs, nseg, n, rev ? 1 : 0,
                                                 reinterpret_cast<uint32_t*>(ws + L.hb_off));
    }
    return launch_status();
}

// One k_scan_small launch over ncols columns (workgroup b: x + b * stride, y + b * stride).
template <typename T>
det_status scan_small(const T* x, T* y, int64_t n, int64_t ncols, int64_t stride, int mode0,
                      const int64_t* offs, int64_t nseg, char* ws, const Layout& L, int A, int A2,
                      hipStream_t s) {
    ScanArgs<T> a{};
    a.x = x;
    a.y = y;
    a.n = n;
    a.offs = offs;
    a.nseg = nseg;
    a.dummy = reinterpret_cast<const T*>(ws + kDummyOff);
    a.err = reinterpret_cast<uint32_t*>(ws + kErrOff);
    a.ntiles = (int)L.ntiles;
    a.rev = (mode0 & 2) ? 1 : 0;
    a.excl = mode0 & 1;
    a.A = A;
    a.A2 = A2;
    a.col_stride = stride;
    if (offs && ncols > 1) {
        // every column has the same heads: one bitmap, loaded with each tile's data
        const det_status st = clear_and_mark(ws, L.hb_off, L.clear, L, offs, nseg, n,
                                             (mode0 & 2) != 0, s);
        if (st != DET_SUCCESS) return st;
        a.hbits = reinterpret_cast<const uint32_t*>(ws + L.hb_off);
    }
    const void* fn = nullptr;
    switch (mode0) {
        case 0: fn = (const void*)k_scan_small<T, false, false, false>; break;
        case 1: fn = (const void*)k_scan_small<T, false, false, true>; break;
        case 2: fn = (const void*)k_scan_small<T, false, true, false>; break;
        case 3: fn = (const void*)k_scan_small<T, false, true, true>; break;
        case 4: fn = (const void*)k_scan_small<T, true, false, false>; break;
        case 5: fn = (const void*)k_scan_small<T, true, false, true>; break;
        case 6: fn = (const void*)k_scan_small<T, true, true, false>; break;
        default: fn = (const void*)k_scan_small<T, true, true, true>; break;
    }
    void* args[] = {&a};
    KernelTimer kt("k_scan_small", s);
    if (hipLaunchKernel(fn, dim3((unsigned)ncols), dim3(256), args, 0, s) != hipSuccess)
        return DET_ERROR_LAUNCH;
    return launch_status();
}

// The two launches of k_scan_two over L.ntiles tiles (at most A) of ncols columns, stride
// elements apart; agg: ncols * L.ntiles slots (null: the workspace's tile slots, one column).
// hbits: the head bitmap when already marked, else null (each tile searches the offsets).
template <typename T>
det_status scan_two(const T* x, T* y, int64_t n, int64_t ncols, int64_t stride, uint64_t* agg,
                    const uint32_t* hbits, int mode0, const int64_t* offs, int64_t nseg,
                    char* ws, const Layout& L, int A, int A2, hipStream_t s) {
    ScanArgs<T> a{};
    a.x = x;
    a.y = y;
    a.n = n;
    a.offs = offs;
    a.nseg = nseg;
    a.agg = agg ? agg : reinterpret_cast<uint64_t*>(ws + L.agg_off);
    a.hbits = hbits;
    a.col_stride = stride;
    a.dummy = reinterpret_cast<const T*>(ws + kDummyOff);
    a.err = reinterpret_cast<uint32_t*>(ws + kErrOff);
    a.ntiles = (int)L.ntiles;
    a.rev = (mode0 & 2) ? 1 : 0;
    a.excl = mode0 & 1;
    a.A = A;
    a.A2 = A2;
    const void* f1 = nullptr;
    const void* f2 = nullptr;
#define DET_TWO(M, SG, RV, EX)                                          \
    case M:                                                             \
        f1 = (const void*)k_scan_two<T, SG, RV, EX, false>;             \
        f2 = (const void*)k_scan_two<T, SG, RV, EX, true>;              \
        break;
    switch (mode0) {
        DET_TWO(0, false, false, false)
        DET_TWO(1, false, false, true)
        DET_TWO(2, false, true, false)
        DET_TWO(3, false, true, true)
        DET_TWO(4, true, false, false)
        DET_TWO(5, true, false, true)
        DET_TWO(6, true, true, false)
        default:
        DET_TWO(7, true, true, true)
    }
#undef DET_TWO
    void* args[] = {&a};
    {
        KernelTimer kt("k_scan_two", s);
        const dim3 g((unsigned)L.ntiles, (unsigned)ncols);
        if (hipLaunchKernel(f1, g, dim3(256), args, 0, s) != hipSuccess) return DET_ERROR_LAUNCH;
        if (hipLaunchKernel(f2, g, dim3(256), args, 0, s) != hipSuccess) return DET_ERROR_LAUNCH;
    }
    return launch_status();
}

template <typename T, bool NT>
const void* k_scan_fn(int mode) {
    switch (mode) {
        case 0: return (const void*)k_scan<T, false, false, false, NT>;
        case 1: return (const void*)k_scan<T, false, false, true, NT>;
        case 2: return (const void*)k_scan<T, false, true, false, NT>;
        case 3: return (const void*)k_scan<T, false, true, true, NT>;
        case 4: return (const void*)k_scan<T, true, false, false, NT>;
        case 5: return (const void*)k_scan<T, true, false, true, NT>;
        case 6: return (const void*)k_scan<T, true, true, false, NT>;
        default: return (const void*)k_scan<T, true, true, true, NT>;
    }
}

template <typename T>
det_status scan_impl(const T* x, T* y, int64_t n, unsigned flags, const int64_t* offs,
                     int64_t nseg, char* ws, hipStream_t s) {
    if (n == 0) {   // nothing to scan; the health word still reports this call: no wait
        k_zero_words<<<1, 64, 0, s>>>(reinterpret_cast<uint64_t*>(ws + kErrOff), 1);
        return launch_status();
    }
    const LaunchOverride& ov = launch_override();
    const int A = ov.scan_A ? ov.scan_A : kScanA;
    const int A2 = ov.scan_A2 ? ov.scan_A2 : kScanA2;
    const Layout L = layout(n, sizeof(T) == 8 ? DET_F64 : DET_F32, A, A2, offs != nullptr);
    const int mode0 = (offs ? 4 : 0) | ((flags & DET_SCAN_REVERSE) ? 2 : 0) |
                      ((flags & DET_SCAN_EXCLUSIVE) ? 1 : 0);
    // one tile: one workgroup, one launch; up to an anchor interval: two launches that never
    // wait (on MI355X at 24,577 to 2^21 elements f32: 10-11 us against 15-17 us for the
    // look-back kernel and its clearing launch); beyond: the look-back kernel
    if (L.ntiles <= kSmallTiles && L.ntiles <= A)
        return scan_small<T>(x, y, n, 1, 0, mode0, offs, nseg, ws, L, A, A2, s);
    if (L.ntiles <= A)
        return scan_two<T>(x, y, n, 1, 0, nullptr, nullptr, mode0, offs, nseg, ws, L, A, A2, s);
    // status slots and counters (and the head bitmap) cleared, heads marked
    det_status st = clear_and_mark(ws, 0, L.clear, L, offs, nseg, n,
                                   (flags & DET_SCAN_REVERSE) != 0, s);
    if (st != DET_SUCCESS) return st;
    ScanArgs<T> a;
    a.x = x;
    a.y = y;
    a.n = n;
    a.offs = offs;
    a.nseg = nseg;
    a.agg = reinterpret_cast<uint64_t*>(ws + L.agg_off);
    a.gtot = reinterpret_cast<uint64_t*>(ws + L.g_off);
    a.carry = reinterpret_cast<uint64_t*>(ws + L.carry_off);
    a.ticket = reinterpret_cast<uint32_t*>(ws);
    a.err = reinterpret_cast<uint32_t*>(ws + kErrOff);
    a.dummy = reinterpret_cast<const T*>(ws + kDummyOff);
    a.hbits = offs ? reinterpret_cast<const uint32_t*>(ws + L.hb_off) : nullptr;
    a.col_stride = 0;
    a.ntiles = (int)L.ntiles;
    a.rev = (flags & DET_SCAN_REVERSE) ? 1 : 0;
    a.excl = (flags & DET_SCAN_EXCLUSIVE) ? 1 : 0;
    a.A = A;
    a.A2 = A2;
    const int mode = (offs ? 4 : 0) | (a.rev ? 2 : 0) | (a.excl ? 1 : 0);
    // Inputs of 512 MiB and more are read with non-temporal loads: on MI355X at 2^28 (1 GiB)
    // f32 inclusive 390 -> 384 us, exclusive 409 -> 402 us, f64 inclusive 727 -> 711 us, and
    // f64 at 2^26 (512 MiB) 197 -> 193 us; at 2^26 and 2^26 + 1 f32 (256 MiB, the size of the
    // last-level cache) repeated calls that found part of their input in that cache lost it
    // (92 -> 104 us), so smaller inputs keep ordinary loads.
    const bool nt = (uint64_t)n * sizeof(T) >= (512ull << 20);
    const void* fn = nt ? k_scan_fn<T, true>(mode) : k_scan_fn<T, false>(mode);
    // Persistent grid: as many workgroups as are resident at once.  More would only queue
    // behind them, and a workgroup that starts late has lost its pipeline's overlap.
    const int extra = ov.extra_lds;
    int per_cu = 0;
    const int64_t resident = resident_wgs(fn, 256, extra, &per_cu);
    if (resident <= 0) return DET_ERROR_LAUNCH;
    int64_t grid = resident;
    // at most 3 workgroups per CU: for f32, 4 resident per CU measured 1-3% slower on MI355X
    // (more tiles in flight than the memory system turns into bandwidth); f64 fits 2
    const int64_t cap = 3 * (int64_t)cu_count();
    if (cap > 0 && grid > cap) grid = cap;
    if (grid > L.ntiles) grid = L.ntiles;
    // the test hook sets the grid, also beyond the resident count: workgroups that start late
    // claim their tiles when they start, and those past the last tile return at once
    if (ov.grid_wgs > 0) grid = ov.grid_wgs;
    note_scan_grid(grid, per_cu);
    // one counter per workgroup that surely runs: never more counters than resident
    // workgroups, or a counter could be left with none running while others wait on its tiles
    int64_t nctr = grid < kCounters ? grid : kCounters;
    if (nctr > resident) nctr = resident;
    a.nctr = (int)nctr;
    a.delay_seed = ov.delay_seed;
    a.delay_us = ov.delay_us;
    void* args[] = {&a};
    KernelTimer kt(sizeof(T) == 8 ? "k_scan<f64>" : __is_same(T, float) ? "k_scan<f32>"
                                                                        : "k_scan<i32>", s);
    if (hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, (size_t)extra, s) !=
        hipSuccess)
        return DET_ERROR_LAUNCH;
    return launch_status();
}

}  // namespace

det_status scan_error(const void* ws, int32_t* out, hipStream_t s) {
    const uint32_t* err =
        reinterpret_cast<const uint32_t*>(static_cast<const char*>(ws) + kErrOff);
    k_copy_error<<<1, 1, 0, s>>>(err, out);
    return launch_status();
}

// ncols scans of n elements that share the flags and segment offsets: column c reads
// x + c * n and writes y + c * n.  Columns that fit in one anchor interval go in one launch,
// a workgroup per column; longer ones are scanned one launch after another.
template <typename T>
det_status scan_cols_impl(const T* x, T* y, int64_t n, int64_t ncols, unsigned flags,
                          const int64_t* offs, int64_t nseg, char* ws, uint64_t* cagg,
                          hipStream_t s) {
    if (n == 0 || ncols == 0) return DET_SUCCESS;
    const LaunchOverride& ov = launch_override();
    const int A = ov.scan_A ? ov.scan_A : kScanA;
    const int A2 = ov.scan_A2 ? ov.scan_A2 : kScanA2;
    const Layout L = layout(n, sizeof(T) == 8 ? DET_F64 : DET_F32, A, A2, offs != nullptr);
    const int mode0 = (offs ? 4 : 0) | ((flags & DET_SCAN_REVERSE) ? 2 : 0) |
                      ((flags & DET_SCAN_EXCLUSIVE) ? 1 : 0);
    if (ncols > 1 && L.ntiles <= A) {
        // every column has the same heads: one bitmap, loaded with each tile's data
        const uint32_t* hb = nullptr;
        if (offs) {
            const det_status st = clear_and_mark(ws, L.hb_off, L.clear, L, offs, nseg, n,
                                                 (mode0 & 2) != 0, s);
            if (st != DET_SUCCESS) return st;
            hb = reinterpret_cast<const uint32_t*>(ws + L.hb_off);
        }
        if (L.ntiles == 1)
            return scan_small<T>(x, y, n, ncols, n, mode0, offs, nseg, ws, L, A, A2, s);
        if (ncols <= 65535)   // columns along the grid's y dimension
            return scan_two<T>(x, y, n, ncols, n, cagg, hb, mode0, offs, nseg, ws, L, A, A2, s);
    }
    for (int64_t c = 0; c < ncols; ++c) {
        const det_status st = scan_impl<T>(x + c * n, y + c * n, n, flags, offs, nseg, ws, s);
        if (st != DET_SUCCESS) return st;
    }
    return DET_SUCCESS;
}

size_t scan_workspace(int64_t n, det_dtype dt, unsigned flags, int64_t num_segments) {
    (void)flags;
    return layout(n, dt, 1, 1, num_segments > 0).total;
}

det_status scan_launch(const void* x, void* y, int64_t n, det_dtype dt, unsigned flags,
                       const int64_t* offs, int64_t nseg, void* ws, size_t ws_bytes,
                       hipStream_t s) {
    (void)ws_bytes;
    if (dt == DET_F32)
        return scan_impl<float>(static_cast<const float*>(x), static_cast<float*>(y), n, flags,
                                offs, nseg, static_cast<char*>(ws), s);
    if (dt == DET_I32)   // two's-complement wrapping sums: computed on the unsigned bits
        return scan_impl<uint32_t>(static_cast<const uint32_t*>(x), static_cast<uint32_t*>(y), n,
                                   flags, offs, nseg, static_cast<char*>(ws), s);
    return scan_impl<double>(static_cast<const double*>(x), static_cast<double*>(y), n, flags,
                             offs, nseg, static_cast<char*>(ws), s);
}

}  // namespace det

namespace det {

det_status scan_columns_launch(const void* x, void* y, int64_t n, int64_t ncols, det_dtype dt,
                               unsigned flags, const int64_t* offs, int64_t nseg, void* ws,
                               void* cagg, hipStream_t s) {
    char* w = static_cast<char*>(ws);
    uint64_t* ca = static_cast<uint64_t*>(cagg);
    if (dt == DET_F32)
        return scan_cols_impl<float>(static_cast<const float*>(x), static_cast<float*>(y), n,
                                     ncols, flags, offs, nseg, w, ca, s);
    if (dt == DET_F64)
        return scan_cols_impl<double>(static_cast<const double*>(x), static_cast<double*>(y), n,
                                      ncols, flags, offs, nseg, w, ca, s);
    return DET_ERROR_UNSUPPORTED;
}

size_t scan_columns_agg_bytes(int64_t n, int64_t ncols) {
    // 16 bytes per tile total (f64 value and flag), one set per column
    return (size_t)((n + kT - 1) / kT) * (size_t)ncols * 16;
}

}  // namespace det
