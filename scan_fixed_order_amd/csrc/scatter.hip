// scatter.hip -- det_scatter_add: keyed scatter-add with a fixed per-destination order.
//
// Order (Warp "Deterministic Execution", sections "Pattern 1: Accumulation", "Writing Manual
// Deterministic Code" and "Picking the Right Mode"; rows per "warp.tile_atomic_add_indexed"):
// the contributions to destination r are taken in ascending source index and combined by the
// adjacent-pair tree PW over their local rank 0, 1, 2, ...; the destination's old value is
// added last: out[r] = out[r] + PW(M_r).  Empty destinations are untouched; out-of-range
// indices are skipped and counted.
//
// Pipeline on gfx950 (every step integer-exact or a fixed tree, so no atomics touch a value):
//   prev   optional snapshot prev[i] = out[index[i]] before anything changes;
//   sort   stable LSD radix sort of (key, payload) with 8-bit digits; the first pass also
//          splits off out-of-range keys into a 257th bucket at the end, and later passes only
//          see the valid prefix.  Payload = the value (row_len 1) or the source row (rows and
//          the running prev).  Per pass: per-chunk digit histogram, integer exclusive scan,
//          then each workgroup ranks its chunk stably (wave ballots + per-wave digit
//          counters), stages it in LDS in digit order and writes contiguous runs.  Scalar
//          values into 257..2^24 destinations take the byte paths: each pass writes only the
//          key bytes the later passes sort on (2 or 3 passes: 4 -> 1 -> 0 or 4 -> 2 -> 1 -> 0
//          bytes), and no sorted key is ever read again.  Otherwise keys travel as 16 bits
//          when every destination fits;
//   bins   off[b] = first sorted position with key >= b: on the byte paths from the passes'
//          bucket offsets and a count of key bytes inside one chunk, otherwise by binary
//          search per bin;
//   reduce a destination's members are cut at local ranks that are multiples of D (D = 8192
//          values, or 64 rows).  Each block is a subtree of PW; one pass reduces every block
//          (a lane per block of at most 32 values, a wave per larger block) and applies
//          destinations with one block; a second pass combines the block values of longer
//          destinations by the same tree and applies them.  Without sorted keys (byte paths)
//          each range of D positions starts from the destination holding its first position
//          (a 64-way search per range) and walks the offsets.
// The running prev (det_scatter_add_running) adds, between sort and reduce: the grouped values
// gathered column by column, the exclusive segmented det_scan of each column (one segment per
// destination), and prev written from it and the old values.
#include "det_device.h"
#include "det_internal.h"
#include <type_traits>

namespace det {
namespace {

constexpr int kSegD = 8192;     // scalar: ranks per block
constexpr int kRowD = 64;       // rows: member rows per block
constexpr int kBuckets0 = 257;  // first pass: 256 digits + the out-of-range bucket

// Key output of a radix pass: uint32_t / uint16_t keys as they are; KeyHi8 / KeyHi16, the
// key shifted down by the byte this pass sorted on, as one or two bytes (the later passes'
// digits: the byte paths, whose keys shrink pass by pass); NoKey, none (the last pass of a
// byte path, whose destination offsets come from the histograms).
struct NoKey {};
struct KeyHi8 {};
struct KeyHi16 {};
template <typename KO>
__device__ __forceinline__ void put_key(KO* keys_out, int64_t g, uint32_t kk) {
    if constexpr (__is_same(KO, NoKey)) {
        (void)keys_out, (void)g, (void)kk;
    } else if constexpr (__is_same(KO, KeyHi8)) {
        reinterpret_cast<uint8_t*>(keys_out)[g] = (uint8_t)(kk >> 8);
    } else if constexpr (__is_same(KO, KeyHi16)) {
        reinterpret_cast<uint16_t*>(keys_out)[g] = (uint16_t)(kk >> 8);
    } else {
        keys_out[g] = (KO)kk;
    }
}

// Keys of a radix chunk (one workgroup's share of a pass): 8192 for 4-byte payloads, 4096 for
// 8-byte ones.  Long chunks give long runs per bucket (32 keys on average for 256 buckets), so
// the scattered writes leave mostly whole lines.  Inputs of at most kSmallN keys take chunks of
// 1024, so a pass has more workgroups than a handful (f32 into 65,536 bins on MI355X: 2^16
// values 128 -> 115 us, 2^18 99 -> 81 us, 2^20 96 -> 82 us, 2^21 111 -> 96 us per call; f32 2^22
// into 2^20 bins 258 -> 173 us; above 2^22 the long chunks are faster: 2^24 into 65,536 bins
// 203 against 289 us).
template <typename P>
constexpr int kChunkBig = sizeof(P) == 4 ? 8192 : 4096;
constexpr int kChunkSmall = 1024;
constexpr int64_t kSmallN = int64_t(1) << 22;
// Waves per radix-scatter workgroup: for 4-byte payloads 8 waves of 16 items need about 112
// VGPRs, so a CU holds two such workgroups (16 waves) where 4 waves of 32 items needed about
// 190 and held 8 waves (f32 2^28 into 65,536 bins on MI355X: 0.80 -> 0.74 ms per pass, same
// ranks); 8-byte payloads keep 4 waves of 16 (8 waves: f64 2^29 into 2^20 Zipf bins 2.50 ->
// 2.65 ms per pass).
template <typename P>
constexpr int kRadixNW = sizeof(P) == 4 ? 8 : 4;
template <typename P>
constexpr int kRadixNT = 64 * kRadixNW<P>;
template <typename P, int CH>
constexpr int kRadixIPT = CH / kRadixNT<P>;   // items per thread for chunks of CH keys

// Workgroup b runs on XCD b mod 8 (round-robin dispatch); give each XCD a contiguous range of
// chunks, so the writes of consecutive chunks into a bucket's region meet in one L2 and leave
// it as whole lines.  Any bijection is correct; this one only changes where the work runs.
__device__ __forceinline__ int64_t xcd_chunk(int64_t b, int64_t nchunks) {
    const int64_t x = b & 7, j = b >> 3;
    const int64_t q = nchunks >> 3, r = nchunks & 7;
    return x * q + (x < r ? x : r) + j;
}

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- integer block helpers

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, uint32_t* s4) {
    v = wave_sum_u32(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) s4[wave] = v;
    __syncthreads();
    const uint32_t t = s4[0] + s4[1] + s4[2] + s4[3];
    __syncthreads();
    return t;
}

// exclusive prefix over the NW * 64 threads (integers: exact in any order); *total = sum
template <int NW = 4>
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t* s4, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t inc = v;
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = shfl_up(inc, d, lane);
        if (lane >= d) inc += o;
    }
    if (lane == 63) s4[wave] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        if (w < wave) before += s4[w];
        all += s4[w];
    }
    *total = all;
    __syncthreads();
    return before + inc - v;
}

// One count per active lane into the LDS counters cnt[d] (integers, so any order is exact).
// When at least 8 lanes share the first active lane's digit (a wave-uniform test), those lanes
// add theirs as one addition by the lowest of them: skewed digits (a contended destination, a
// heavy Zipf head, the few values of a key's top bits) otherwise put most lanes of one atomic
// on one counter.  Other rows, the usual case for uniform keys, take one atomic per lane.
// Returns (uniformly) whether the row was aggregated.
__device__ __forceinline__ bool count_digit(uint32_t* cnt, int d) {
    const int d0 = __builtin_amdgcn_readfirstlane(d);
    const uint64_t m0 = __ballot(d == d0);
    if (__popcll(m0) >= 8) {
        if (d == d0) {
            if (__builtin_amdgcn_mbcnt_hi((uint32_t)(m0 >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m0, 0u)) == 0u)
                atomicAdd(&cnt[d0], (uint32_t)__popcll(m0));
        } else {
            atomicAdd(&cnt[d], 1u);
        }
        return true;
    }
    atomicAdd(&cnt[d], 1u);
    return false;
}

// ---------------------------------------------------------------- histogram offsets

// The digit counts of a pass are row-major, cnt[c * nb + d] = keys of chunk c with digit d (16
// bits: a chunk holds at most 8192 keys), so each chunk's counts are written contiguously.  The
// scatter needs, for chunk c and digit d, off[c][d] = (keys with a digit below d) + (keys with
// digit d in chunks before c): an exclusive scan in digit-major order, done in three launches
// over blocks of rb rows: column sums per row block (stored column-major), an exclusive
// scan of each column's block sums, then each row block scans the digit totals and writes its
// 32-bit offsets, off[c * nb + d].  Integers, so exact in any order.  (32-bit counts rewritten
// in place moved more bytes: f64 2^29 into 2^20 Zipf bins on MI355X, 0.25 -> 0.18 ms for the
// three passes' offsets.)
// Row blocks: 128 rows, or 16 when there are at most 4096 rows, so that few rows still make
// many short workgroups (2^22 f32 values into 65,536 bins, 512 rows, on MI355X: the call 275 ->
// 138 us; the single-workgroup kernel below walked 512 rows in 103 us per pass).
constexpr int kRowBlk = 64;
constexpr int kRowBlkFew = 16;
constexpr int kRowBatch = 16;   // rows whose loads are in flight together

// csum[d * nrb + rb] = sum over the rows of block rb of column d (thread t: column t; column
// 256, when nb = 257, a row per thread and a block sum).  Whole batches of rows load without a
// per-row test.
__global__ __launch_bounds__(256) void k_hist_colsums(const uint16_t* __restrict__ hist,
                                                      int64_t nrows, int nb, int64_t nrb, int rb,
                                                      uint32_t* __restrict__ csum) {
    static_assert(kRowBlk <= 256 && kRowBlkFew <= 256, "column 256: a row per thread");
    __shared__ uint32_t s4[4];
    const int t = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * rb;
    const int64_t r1 = (r0 + rb < nrows) ? r0 + rb : nrows;
    uint32_t s0 = 0;
    const uint16_t* hp = hist + r0 * nb + t;
    for (int64_t r = r0; r < r1; r += kRowBatch, hp += (int64_t)kRowBatch * nb) {
        uint32_t v[kRowBatch];
        if (r + kRowBatch <= r1) {
#pragma unroll
            for (int k = 0; k < kRowBatch; ++k) v[k] = hp[(int64_t)k * nb];
        } else {
#pragma unroll
            for (int k = 0; k < kRowBatch; ++k) v[k] = r + k < r1 ? hp[(int64_t)k * nb] : 0u;
        }
#pragma unroll
        for (int k = 0; k < kRowBatch; ++k) s0 += v[k];
    }
    csum[(int64_t)t * nrb + blockIdx.x] = s0;
    if (nb > 256) {
        const uint32_t w = t < r1 - r0 ? (uint32_t)hist[(r0 + t) * nb + 256] : 0u;
        const uint32_t s1 = block_sum_u32(w, s4);
        if (t == 0) csum[(int64_t)256 * nrb + blockIdx.x] = s1;
    }
}

// column d = blockIdx.x: exclusive scan of its block sums in place; tot[d] = the column total
__global__ __launch_bounds__(256) void k_hist_colscan(uint32_t* __restrict__ csum, int64_t nrb,
                                                      uint32_t* __restrict__ tot) {
    __shared__ uint32_t s4[4];
    uint32_t* col = csum + (int64_t)blockIdx.x * nrb;
    uint32_t carry = 0;
    for (int64_t base = 0; base < nrb; base += 256) {
        const int64_t k = base + threadIdx.x;
        const uint32_t v = k < nrb ? col[k] : 0u;
        uint32_t total;
        const uint32_t ex = block_excl_scan_u32(v, s4, &total);
        if (k < nrb) col[k] = carry + ex;
        carry += total;
    }
    if (threadIdx.x == 0) tot[blockIdx.x] = carry;
}

// tot[d] = the keys of digit d (column totals).  Each workgroup turns them into the digit
// bases (keys with a digit below d; d = 256, the out-of-range bucket, after every digit) and
// writes its row block's offsets (column 256: a row per thread, a block scan).  Workgroup 0
// also sets *ident = 1 when one bucket holds every key (the pass is then the identity
// permutation), else 0, and *valid (if given) = the keys in range (the base of bucket 256).
__global__ __launch_bounds__(256) void k_hist_apply(const uint16_t* __restrict__ hist,
                                                    uint32_t* __restrict__ off, int64_t nrows,
                                                    int nb, int64_t nrb, int rb,
                                                    const uint32_t* __restrict__ csum,
                                                    const uint32_t* __restrict__ tot,
                                                    uint32_t* __restrict__ ident,
                                                    uint32_t* __restrict__ valid) {
    __shared__ uint32_t s4[4];
    const int t = threadIdx.x;
    const uint32_t v = tot[t];
    const uint32_t v256 = nb > 256 ? tot[256] : 0u;
    uint32_t total;
    const uint32_t base = block_excl_scan_u32(v, s4, &total);
    const int one = __syncthreads_or(v == total + v256 || v256 == total + v256);
    if (blockIdx.x == 0 && t == 0) {
        *ident = one ? 1u : 0u;
        if (valid) {
            valid[0] = total;
            valid[1] = v256 == 0u ? 1u : 0u;   // no key out of range
        }
    }
    const int64_t r0 = (int64_t)blockIdx.x * rb;
    const int64_t r1 = (r0 + rb < nrows) ? r0 + rb : nrows;
    if (nb > 256) {
        const bool in = t < r1 - r0;
        const uint32_t w = in ? (uint32_t)hist[(r0 + t) * nb + 256] : 0u;
        uint32_t wt;
        const uint32_t ex = block_excl_scan_u32(w, s4, &wt);
        if (in) off[(r0 + t) * nb + 256] = total + csum[(int64_t)256 * nrb + blockIdx.x] + ex;
    }
    uint32_t run0 = base + csum[(int64_t)t * nrb + blockIdx.x];
    const uint16_t* hp = hist + r0 * nb + t;
    uint32_t* op = off + r0 * nb + t;
    for (int64_t r = r0; r < r1;
         r += kRowBatch, hp += (int64_t)kRowBatch * nb, op += (int64_t)kRowBatch * nb) {
        uint32_t v[kRowBatch];
        if (r + kRowBatch <= r1) {
#pragma unroll
            for (int k = 0; k < kRowBatch; ++k) v[k] = hp[(int64_t)k * nb];
#pragma unroll
            for (int k = 0; k < kRowBatch; ++k) {
                op[(int64_t)k * nb] = run0;
                run0 += v[k];
            }
        } else {
#pragma unroll
            for (int k = 0; k < kRowBatch; ++k) v[k] = r + k < r1 ? hp[(int64_t)k * nb] : 0u;
#pragma unroll
            for (int k = 0; k < kRowBatch; ++k) {
                if (r + k < r1) op[(int64_t)k * nb] = run0;
                run0 += v[k];
            }
        }
    }
}

// The same offsets for at most 64 rows, in one launch of one workgroup: thread d loads column
// d of every row at once (one round trip), an exclusive scan over the digit totals gives each
// digit's base, and thread d writes its column's running offsets from the values it holds.
// *valid (if given) receives the base of digit 256 (the keys in range) and valid[1] whether no
// key is out of range.  (Walking the rows 8 at a time took 20 us for 64 rows on MI355X.)
constexpr int64_t kSmallHistRows = 64;

__global__ __launch_bounds__(256) void k_hist_offsets_small(const uint16_t* __restrict__ hist,
                                                            uint32_t* __restrict__ off,
                                                            int64_t nrows, int nb,
                                                            uint32_t* __restrict__ valid,
                                                            uint32_t* __restrict__ ident) {
    constexpr int R = (int)kSmallHistRows;
    static_assert(R == 64, "the out-of-range column takes one row per lane of a wave");
    __shared__ uint32_t s4[4];
    __shared__ uint32_t s_c256;
    const int t = threadIdx.x, lane = t & 63;
    const int nr = (int)nrows;   // 1 .. R
    // column t; rows past nr load row nr - 1 (in bounds, no branch) and count as zero
    uint32_t v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t x = hist[(int64_t)(r < nr ? r : nr - 1) * nb + t];
        v[r] = r < nr ? x : 0u;
    }
    // the out-of-range column (nb = 257): row lane of wave 0, an inclusive scan over the rows
    const bool extra = nb > 256 && t < 64;
    uint32_t w = 0u, winc = 0u;
    if (extra) {
        w = lane < nr ? (uint32_t)hist[(int64_t)lane * nb + 256] : 0u;
        winc = w;
        for (int dd = 1; dd < 64; dd <<= 1) {
            const uint32_t o = shfl_up(winc, dd, lane);
            if (lane >= dd) winc += o;
        }
        if (lane == 63) s_c256 = winc;
    } else if (t == 0) {
        s_c256 = 0u;
    }
    uint32_t c0 = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) c0 += v[r];
    uint32_t total;
    uint32_t run0 = block_excl_scan_u32(c0, s4, &total);   // its barriers publish s_c256
    const uint32_t c256 = s_c256;
    const uint32_t grand = total + c256;
    const int one = __syncthreads_or(c0 == grand || c256 == grand);
    if (t == 0) *ident = one ? 1u : 0u;
    uint32_t* po = off + t;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r < nr) po[0] = run0;
        po += nb;
        run0 += v[r];
    }
    if (extra && lane < nr) off[(int64_t)lane * nb + 256] = total + winc - w;
    if (valid && t == 0) {
        valid[0] = total;
        valid[1] = c256 == 0u ? 1u : 0u;   // no key out of range
    }
}

// The same for 65 to 256 rows in one launch of one workgroup of 1024 threads: thread (q, d)
// holds rows 64 q .. 64 q + 63 of column d in registers; the column totals are the four
// quarters' sums, and quarter q starts its running offsets after the quarters before it.  The
// out-of-range column goes a row per lane to the first wave of each quarter.
constexpr int64_t kMidHistRows = 256;

__global__ __launch_bounds__(1024) void k_hist_offsets_mid(const uint16_t* __restrict__ hist,
                                                           uint32_t* __restrict__ off,
                                                           int64_t nrows, int nb,
                                                           uint32_t* __restrict__ valid,
                                                           uint32_t* __restrict__ ident) {
    __shared__ uint32_t s_part[4][256];
    __shared__ uint32_t s_base[256];
    __shared__ uint32_t s4[4];
    __shared__ uint32_t s_oor[4];
    __shared__ uint32_t s_total;
    const int t = threadIdx.x, d = t & 255, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6), q = wave >> 2;   // uniform per wave
    const int nr = (int)nrows;   // 65 .. 256
    const int r0 = 64 * q;
    // rows past nr load row nr - 1 (in bounds, no branch); they are a suffix, left out of the
    // sum and written nowhere
    uint32_t v[64];
#pragma unroll
    for (int r = 0; r < 64; ++r) {
        const int rr = r0 + r;
        v[r] = hist[(int64_t)(rr < nr ? rr : nr - 1) * nb + d];
    }
    uint32_t cq = 0;
#pragma unroll
    for (int r = 0; r < 64; ++r) cq += r0 + r < nr ? v[r] : 0u;
    s_part[q][d] = cq;
    const bool extra = nb > 256 && d < 64;   // the first wave of each quarter
    uint32_t w = 0u, winc = 0u;
    if (extra) {
        const int rr = r0 + lane;
        w = rr < nr ? (uint32_t)hist[(int64_t)rr * nb + 256] : 0u;
        winc = w;
        for (int dd = 1; dd < 64; dd <<= 1) {
            const uint32_t o = shfl_up(winc, dd, lane);
            if (lane >= dd) winc += o;
        }
        if (lane == 63) s_oor[q] = winc;
    } else if (nb <= 256 && t < 4) {
        s_oor[t] = 0u;
    }
    __syncthreads();
    // column totals, and their exclusive scan over the 256 digits (the first four waves)
    uint32_t tot = 0u, inc = 0u;
    if (t < 256) {
        tot = s_part[0][d] + s_part[1][d] + s_part[2][d] + s_part[3][d];
        inc = tot;
        for (int dd = 1; dd < 64; dd <<= 1) {
            const uint32_t o = shfl_up(inc, dd, lane);
            if (lane >= dd) inc += o;
        }
        if (lane == 63) s4[wave] = inc;
    }
    __syncthreads();
    if (t < 256) {
        uint32_t before = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (k < wave) before += s4[k];
        s_base[d] = before + inc - tot;
        if (t == 0) s_total = s4[0] + s4[1] + s4[2] + s4[3];
    }
    __syncthreads();
    const uint32_t total = s_total;
    const uint32_t c256 = s_oor[0] + s_oor[1] + s_oor[2] + s_oor[3];
    const uint32_t grand = total + c256;
    const int one = __syncthreads_or((t < 256 && tot == grand) || c256 == grand);
    if (t == 0) *ident = one ? 1u : 0u;
    uint32_t run0 = s_base[d];
#pragma unroll
    for (int k = 0; k < 3; ++k)
        if (k < q) run0 += s_part[k][d];
    uint32_t* po = off + (int64_t)r0 * nb + d;
#pragma unroll
    for (int r = 0; r < 64; ++r) {
        if (r0 + r < nr) po[0] = run0;
        po += nb;
        run0 += v[r];
    }
    if (extra && r0 + lane < nr) {
        uint32_t ob = total;
#pragma unroll
        for (int k = 0; k < 3; ++k)
            if (k < q) ob += s_oor[k];
        off[(int64_t)(r0 + lane) * nb + 256] = ob + winc - w;
    }
    if (valid && t == 0) {
        valid[0] = total;
        valid[1] = c256 == 0u ? 1u : 0u;   // no key out of range
    }
}

// csum needs nb * nrb words, tot nb words (nb <= 257).  valid (first pass only): receives the
// number of keys in range (the offset of the out-of-range bucket in chunk 0).  ident: 1 when
// one bucket holds every key, else 0.
det_status hist_offsets(const uint16_t* hist, uint32_t* off, int64_t nrows, int nb,
                        uint32_t* csum, uint32_t* tot, uint32_t* valid, uint32_t* ident,
                        hipStream_t s) {
    KernelTimer kt("k_hist_offsets", s);
    if (nrows <= kSmallHistRows) {
        k_hist_offsets_small<<<1, 256, 0, s>>>(hist, off, nrows, nb, valid, ident);
        return launch_status();
    }
    if (nrows <= kMidHistRows) {
        k_hist_offsets_mid<<<1, 1024, 0, s>>>(hist, off, nrows, nb, valid, ident);
        return launch_status();
    }
    const int rb = nrows <= 4096 ? kRowBlkFew : kRowBlk;
    const int64_t nrb = cdiv(nrows, rb);
    k_hist_colsums<<<dim3((unsigned)nrb), dim3(256), 0, s>>>(hist, nrows, nb, nrb, rb, csum);
    k_hist_colscan<<<dim3((unsigned)nb), dim3(256), 0, s>>>(csum, nrb, tot);
    k_hist_apply<<<dim3((unsigned)nrb), dim3(256), 0, s>>>(hist, off, nrows, nb, nrb, rb, csum,
                                                          tot, ident, valid);
    return launch_status();
}

// ---------------------------------------------------------------- 10-bit digits

// f64 values into more than 65,536 and at most 2^20 destinations (chunks of 4096 keys) sort in
// two passes of 10-bit digits instead of three of 8: the first on the low 10 bits (bucket 1024
// for keys out of range), writing the high 10 bits as 16-bit keys, the second on those, writing
// no key.  The kernels below are the 8-bit ones widened to kWideB buckets (plus one); every
// count and offset is an integer, so the order of additions changes nothing.
constexpr int kWideBits = 10;
constexpr int kWideB = 1 << kWideBits;   // 1024 digits
constexpr int kWideCols = kWideB + 1;    // and the out-of-range bucket of the first pass
constexpr int kWideRowBatch = 8;         // rows whose loads are in flight together
constexpr int kWidePer = (kWideCols + 255) / 256;   // columns per thread (5)

template <bool OOR>
__device__ __forceinline__ int wide_digit(uint32_t key, uint32_t B, int shift) {
    if (OOR && key >= B) return kWideB;
    return (int)((key >> shift) & (uint32_t)(kWideB - 1));
}

// Per-chunk digit counts (16-bit), a wave per chunk (four per workgroup), as k_radix_hist:
// a batch whose keys share one digit adds with one atomic, others row by row (count_digit).
template <bool FIRST, typename KI>
__global__ __launch_bounds__(256) void k_radix_hist_w(const KI* __restrict__ keys, int64_t n,
                                                      const uint32_t* __restrict__ nvalid,
                                                      uint32_t B, int nb, int64_t nchunks, int H,
                                                      uint16_t* __restrict__ hist) {
    __shared__ uint32_t cnt[4][kWideCols];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c = (int64_t)blockIdx.x * 4 + wave;
    if (c >= nchunks) return;   // a whole wave; it waits for no other wave
    uint32_t* const wc = cnt[wave];
    for (int d = lane; d < kWideCols; d += 64) wc[d] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t m = FIRST ? n : (int64_t)*nvalid;
    const int64_t base = c * H;
    constexpr int NK = 16;
    constexpr int PER = 64 * NK;
    constexpr int KPW = 4 / (int)sizeof(KI);   // keys per 32-bit word
    // position in the chunk of kk[k]: 4-byte keys i0 + k * 64 + lane; 16-bit keys two to a
    // word, word i0 / 2 + (k / 2) * 64 + lane
    auto pos = [&](int i0, int k) -> int {
        return KPW == 1 ? i0 + k * 64 + lane : i0 + KPW * ((k / KPW) * 64 + lane) + k % KPW;
    };
    for (int i0 = 0; i0 < H; i0 += PER) {
        uint32_t kk[NK];
        if constexpr (KPW == 1) {
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                const int64_t p = base + i0 + k * 64 + lane;
                kk[k] = (i0 + k * 64 + lane < H && p < m)
                            ? (uint32_t)__builtin_nontemporal_load(keys + p) : 0u;
            }
        } else {
            // chunk starts are multiples of 4096 and the keys 256-byte aligned
            const uint32_t* kw = reinterpret_cast<const uint32_t*>(keys) + base / KPW;
#pragma unroll
            for (int k = 0; k < NK / KPW; ++k) {
                const int w = i0 / KPW + k * 64 + lane;
                const uint32_t x = (KPW * w < H && base + KPW * w < m)
                                       ? __builtin_nontemporal_load(kw + w) : 0u;
#pragma unroll
                for (int j = 0; j < KPW; ++j)
                    kk[KPW * k + j] = (x >> (32 / KPW * j)) & (0xffffffffu >> (32 - 32 / KPW));
            }
        }
        const bool full = i0 + PER <= H && base + i0 + PER <= m;   // uniform over the wave
        if (full) {
            const int dref = __builtin_amdgcn_readfirstlane(wide_digit<FIRST>(kk[0], B, 0));
            bool same = true;
#pragma unroll
            for (int k = 0; k < NK; ++k) same = same && wide_digit<FIRST>(kk[k], B, 0) == dref;
            if (__builtin_amdgcn_ballot_w64(!same) == 0ull) {
                if (lane == 0) atomicAdd(&wc[dref], (uint32_t)PER);
            } else {
#pragma unroll
                for (int k = 0; k < NK; ++k) count_digit(wc, wide_digit<FIRST>(kk[k], B, 0));
            }
        } else {
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                const int q = pos(i0, k);
                if (q < H && base + q < m) count_digit(wc, wide_digit<FIRST>(kk[k], B, 0));
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int d = lane; d < nb; d += 64) hist[c * nb + d] = (uint16_t)wc[d];
}

// csum[d * nrb + rb] = sum over the rows of block rb of column d (thread t: columns t + 256 j)
__global__ __launch_bounds__(256) void k_hist_colsums_w(const uint16_t* __restrict__ hist,
                                                        int64_t nrows, int nb, int64_t nrb,
                                                        int rb, uint32_t* __restrict__ csum) {
    const int t = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * rb;
    const int64_t r1 = (r0 + rb < nrows) ? r0 + rb : nrows;
    uint32_t sum[kWidePer];
#pragma unroll
    for (int j = 0; j < kWidePer; ++j) sum[j] = 0u;
    for (int64_t r = r0; r < r1; r += kWideRowBatch) {
        uint32_t v[kWideRowBatch][kWidePer];
#pragma unroll
        for (int k = 0; k < kWideRowBatch; ++k)
#pragma unroll
            for (int j = 0; j < kWidePer; ++j) {
                const int col = t + 256 * j;
                v[k][j] = (r + k < r1 && col < nb) ? hist[(r + k) * nb + col] : 0u;
            }
#pragma unroll
        for (int k = 0; k < kWideRowBatch; ++k)
#pragma unroll
            for (int j = 0; j < kWidePer; ++j) sum[j] += v[k][j];
    }
#pragma unroll
    for (int j = 0; j < kWidePer; ++j) {
        const int col = t + 256 * j;
        if (col < nb) csum[(int64_t)col * nrb + blockIdx.x] = sum[j];
    }
}

// tot[d] = the keys of digit d (column totals, from k_hist_colscan).  Each workgroup turns them
// into the digit bases (keys with a smaller digit; column 1024, the out-of-range bucket, after
// every digit) and writes its row block's offsets.  Workgroup 0 also sets *ident (one bucket
// holds every key) and *valid (if given: the keys in range, and whether none is out of range).
__global__ __launch_bounds__(256) void k_hist_apply_w(const uint16_t* __restrict__ hist,
                                                      uint32_t* __restrict__ off, int64_t nrows,
                                                      int nb, int64_t nrb, int rb,
                                                      const uint32_t* __restrict__ csum,
                                                      const uint32_t* __restrict__ tot,
                                                      uint32_t* __restrict__ ident,
                                                      uint32_t* __restrict__ valid) {
    __shared__ uint32_t s4[4];
    __shared__ uint32_t s_base[kWideCols];
    const int t = threadIdx.x;
    // thread t scans digits 4t .. 4t + 3 (the 1024 regular ones)
    uint32_t v[4], loc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = tot[4 * t + j];
        loc += v[j];
    }
    const uint32_t voor = nb > kWideB ? tot[kWideB] : 0u;
    uint32_t total;
    uint32_t ex = block_excl_scan_u32(loc, s4, &total);
    const uint32_t grand = total + voor;
    bool one = voor == grand;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        s_base[4 * t + j] = ex;
        one = one || v[j] == grand;
        ex += v[j];
    }
    if (t == 0) s_base[kWideB] = total;
    const int anyone = __syncthreads_or(one);   // also publishes s_base
    if (blockIdx.x == 0 && t == 0) {
        *ident = anyone ? 1u : 0u;
        if (valid) {
            valid[0] = total;
            valid[1] = voor == 0u ? 1u : 0u;
        }
    }
    const int64_t r0 = (int64_t)blockIdx.x * rb;
    const int64_t r1 = (r0 + rb < nrows) ? r0 + rb : nrows;
    uint32_t run[kWidePer];
#pragma unroll
    for (int j = 0; j < kWidePer; ++j) {
        const int col = t + 256 * j;
        run[j] = col < nb ? s_base[col] + csum[(int64_t)col * nrb + blockIdx.x] : 0u;
    }
    for (int64_t r = r0; r < r1; r += kWideRowBatch) {
        uint32_t w[kWideRowBatch][kWidePer];
#pragma unroll
        for (int k = 0; k < kWideRowBatch; ++k)
#pragma unroll
            for (int j = 0; j < kWidePer; ++j) {
                const int col = t + 256 * j;
                w[k][j] = (r + k < r1 && col < nb) ? hist[(r + k) * nb + col] : 0u;
            }
#pragma unroll
        for (int k = 0; k < kWideRowBatch; ++k)
#pragma unroll
            for (int j = 0; j < kWidePer; ++j) {
                const int col = t + 256 * j;
                if (r + k < r1 && col < nb) off[(r + k) * nb + col] = run[j];
                run[j] += w[k][j];
            }
    }
}

// Offsets of nb = 1025 or 1024 columns for nrows chunks (three launches, as hist_offsets).
// csum needs nb * nrb words, tot nb words.
det_status hist_offsets_w(const uint16_t* hist, uint32_t* off, int64_t nrows, int nb,
                          uint32_t* csum, uint32_t* tot, uint32_t* valid, uint32_t* ident,
                          hipStream_t s) {
    KernelTimer kt("k_hist_offsets", s);
    const int rb = nrows <= 4096 ? kRowBlkFew : kRowBlk;
    const int64_t nrb = cdiv(nrows, rb);
    k_hist_colsums_w<<<dim3((unsigned)nrb), dim3(256), 0, s>>>(hist, nrows, nb, nrb, rb, csum);
    k_hist_colscan<<<dim3((unsigned)nb), dim3(256), 0, s>>>(csum, nrb, tot);
    k_hist_apply_w<<<dim3((unsigned)nrb), dim3(256), 0, s>>>(hist, off, nrows, nb, nrb, rb, csum,
                                                            tot, ident, valid);
    return launch_status();
}

// ---------------------------------------------------------------- radix sort passes

// digit of a key; in the first pass keys outside [0, B) (as unsigned: also negatives) go to 256
template <bool FIRST>
__device__ __forceinline__ int digit_of(uint32_t key, uint32_t B, int shift) {
    if (FIRST && key >= B) return 256;
    return (int)((key >> shift) & 255u);
}

// Per-chunk digit counts: hist[c * nb + d] = keys of chunk c (positions [c H, c H + H)) with
// digit d.  WPC waves per chunk, each counting into its own LDS histogram.  WPC = 1 (many
// chunks): four chunks per workgroup, each wave writes its own row and no workgroup barrier is
// needed, so a chunk of byte keys (4 or 8 KB) does not cost a whole workgroup's setup (f64 2^29
// into 2^20 Zipf bins on MI355X: 1.21 -> 0.99 ms for the three passes' counts).  WPC = 4 (few
// chunks, so the chunk's waves run side by side): the four histograms are summed.
// KI: the type keys are read in (16-bit or byte keys after a pass that wrote them so).
template <bool FIRST, typename KI, int WPC>
__global__ __launch_bounds__(256) void k_radix_hist(const KI* __restrict__ keys, int64_t n,
                                                    const uint32_t* __restrict__ nvalid, uint32_t B,
                                                    int shift, int nb, int64_t nchunks, int H,
                                                    uint16_t* __restrict__ hist) {
    static_assert(WPC == 1 || WPC == 4, "one wave or the whole workgroup per chunk");
    __shared__ uint32_t cnt[4][kBuckets0];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c = WPC == 1 ? (int64_t)blockIdx.x * 4 + wave : (int64_t)blockIdx.x;
    if (WPC == 1 && c >= nchunks) return;   // a whole wave; it then waits for no other wave
    const int tt = WPC == 1 ? lane : (int)threadIdx.x;   // index in the chunk's team of waves
    constexpr int TS = 64 * WPC;                          // the team's threads
    uint32_t* const wc = cnt[wave];
    for (int d = lane; d < kBuckets0; d += 64) wc[d] = 0u;
    // a wave's LDS instructions run in order: its counts below follow its zeroing
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t m = FIRST ? n : (int64_t)*nvalid;
    const int64_t base = c * H;
    // a batch of NK keys per thread, all loads issued before the first count; a whole batch
    // of a wave whose keys all share the digit of its first lane's first key is added with one
    // atomic (skewed and contended inputs), any other batch row by row (count_digit)
    constexpr int NK = sizeof(KI) < 4 ? 32 : 16;
    constexpr int KPW = 4 / (int)sizeof(KI);      // keys per 32-bit word
    constexpr int PER = TS * NK;                  // keys per batch of the team
    bool skew = true;                             // uniform over the wave
    for (int i0 = 0; i0 < H; i0 += PER) {
        uint32_t kk[NK];
        // thread tt takes keys i0 + k * TS + tt (4-byte keys) or the KPW keys of word
        // i0 / KPW + k * TS + tt (16-bit and byte keys, packed in 32-bit words: H is a multiple
        // of 4 and the keys 256-byte aligned)
        if constexpr (sizeof(KI) < 4) {
            const uint32_t* kw = reinterpret_cast<const uint32_t*>(keys) + base / KPW;
#pragma unroll
            for (int k = 0; k < NK / KPW; ++k) {
                const int w = i0 / KPW + k * TS + tt;
                const uint32_t x = (KPW * w < H && base + KPW * w < m)
                                       ? __builtin_nontemporal_load(kw + w) : 0u;
#pragma unroll
                for (int j = 0; j < KPW; ++j)
                    kk[KPW * k + j] = (x >> (32 / KPW * j)) & (0xffffffffu >> (32 - 32 / KPW));
            }
        } else {
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                const int64_t p = base + i0 + k * TS + tt;
                // non-temporal: each key is read once here (0.21 -> 0.18 ms per pass at 2^28)
                kk[k] = (i0 + k * TS + tt < H && p < m)
                            ? (uint32_t)__builtin_nontemporal_load(keys + p) : 0u;
            }
        }
        auto pos = [&](int k) -> int {   // position of kk[k] in the chunk
            return sizeof(KI) < 4 ? i0 + KPW * ((k / KPW) * TS + tt) + k % KPW
                                  : i0 + k * TS + tt;
        };
        const bool full = i0 + PER <= H && base + i0 + PER <= m;   // uniform over the team
        if (full) {
            const int dref = __builtin_amdgcn_readfirstlane(digit_of<FIRST>(kk[0], B, shift));
            bool same = true;
#pragma unroll
            for (int k = 0; k < NK; ++k) same = same && digit_of<FIRST>(kk[k], B, shift) == dref;
            if (__builtin_amdgcn_ballot_w64(!same) == 0ull) {
                if (lane == 0) atomicAdd(&wc[dref], (uint32_t)(64 * NK));
            } else if (sizeof(KI) == 4 || skew ||
                       __popcll(__builtin_amdgcn_ballot_w64(digit_of<FIRST>(kk[0], B, shift) ==
                                                            dref)) >= 8) {
                // skewed (and always for 4-byte keys, whose pass is bound by its reads, where
                // a moderately skewed low byte made plain atomics slower: f64 2^29 into 2^20
                // Zipf(1.1) bins): row by row, the lanes on the first active lane's digit as
                // one addition; the wave stays in this mode while some row of a batch
                // aggregates
                bool agg = false;
#pragma unroll
                for (int k = 0; k < NK; ++k)
                    agg = count_digit(wc, digit_of<FIRST>(kk[k], B, shift)) || agg;
                skew = agg;
            } else {
                // spread digits in 1- or 2-byte keys (no row of the last batch aggregated, nor
                // this batch's first row): one LDS atomic per key without the per-row test
                // (f32 2^28 into 65,536 bins on MI355X: the two passes' counts 0.31 -> 0.28 ms)
#pragma unroll
                for (int k = 0; k < NK; ++k) atomicAdd(&wc[digit_of<FIRST>(kk[k], B, shift)], 1u);
            }
        } else {
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                const int q = pos(k);
                if (q < H && base + q < m) count_digit(wc, digit_of<FIRST>(kk[k], B, shift));
            }
        }
    }
    if constexpr (WPC == 1) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int d = lane; d < nb; d += 64) hist[c * nb + d] = (uint16_t)wc[d];
    } else {
        __syncthreads();
        for (int d = threadIdx.x; d < nb; d += 256)
            hist[c * nb + d] = (uint16_t)((cnt[0][d] + cnt[1][d]) + (cnt[2][d] + cnt[3][d]));
    }
}

// Launches k_radix_hist with one wave per chunk when there are enough chunks to fill the GPU
// that way (four per compute unit), else with a workgroup per chunk.
template <bool FIRST, typename KI>
void radix_hist(const KI* keys, int64_t n, const uint32_t* nvalid, uint32_t B, int shift, int nb,
                int64_t nchunks, int H, uint16_t* hist, size_t lds, hipStream_t s) {
    KernelTimer kt("k_radix_hist", s);
    if (nchunks >= 4 * (int64_t)cu_count())
        k_radix_hist<FIRST, KI, 1><<<dim3((unsigned)cdiv(nchunks, 4)), dim3(256), lds, s>>>(
            keys, n, nvalid, B, shift, nb, nchunks, H, hist);
    else
        k_radix_hist<FIRST, KI, 4><<<dim3((unsigned)nchunks), dim3(256), lds, s>>>(
            keys, n, nvalid, B, shift, nb, nchunks, H, hist);
}

// P: payload word (uint32_t: f32 value bits or source row; uint64_t: f64 value bits)
// The staged chunk: for 4-byte payloads key and payload share one 64-bit word (kp), so each
// item's scattered LDS write is one instruction; 8-byte payloads keep two arrays.
template <typename P, int CH>
struct RadixSmem {
    static constexpr bool kPacked = sizeof(P) == 4;
    uint64_t kp[kPacked ? CH : 1];
    uint32_t keys[kPacked ? 1 : CH];
    P pay[kPacked ? 1 : CH];
    // per-wave digit counters; then each wave's first position per digit in the staged chunk
    uint32_t cnt[kRadixNW<P>][kBuckets0];
    // global index of staged position 0 for each digit, modulo 2^32 (every index is below 2^31)
    uint32_t gbase[kBuckets0];
    uint32_t s4[kRadixNW<P>];
};

// A chunk's keys and payloads, loaded by thread (wave w, lane l) at positions
// base + w * 64 * IPT + k * 64 + l.  FULL: the whole chunk is in range (no checks, so every
// path issues the same loads).
template <typename P, int CH, bool FIRST, bool ROWS, bool FULL, typename KI>
__device__ __forceinline__ void radix_load(const KI* __restrict__ keys_in,
                                           const P* __restrict__ pay_in, int64_t base, int64_t m,
                                           uint32_t (&key)[kRadixIPT<P, CH>],
                                           P (&pay)[kRadixIPT<P, CH>], int wave, int lane) {
    constexpr int IPT = kRadixIPT<P, CH>;
    const int64_t p0 = base + (int64_t)wave * 64 * IPT + lane;
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
        const int64_t p = p0 + k * 64;
        key[k] = (FULL || p < m) ? (uint32_t)keys_in[p] : 0u;
    }
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
        const int64_t p = p0 + k * 64;
        if constexpr (ROWS && FIRST) {
            pay[k] = (P)((FULL || p < m) ? p : 0);
        } else {
            pay[k] = (FULL || p < m) ? pay_in[p] : (P)0;
        }
    }
}

// Ranks one loaded chunk stably by digit, stages it in LDS in digit order and writes every
// digit's run to its place in the output.  Rank of an item = (items of the chunk with a smaller
// digit) + (items of its digit in earlier waves) + (items of its digit earlier in its wave):
// the last part from the wave's ballots on each digit bit (the lanes that agree on every bit
// are the item's peers), taken in item order k = 0 .. IPT-1 against per-wave counters in LDS:
// every lane reads its digit's counter, then the lowest peer writes it advanced by the peers.
// Integers only, so exact.  Leaves every barrier it passes balanced; ends with the LDS counters
// cleared for the next chunk.
template <typename P, int CH, bool FIRST, bool ROWS, bool FULL, typename KO, bool OOR = FIRST>
__device__ __forceinline__ void radix_rank_write(RadixSmem<P, CH>& sm,
                                                 const uint32_t (&key)[kRadixIPT<P, CH>],
                                                 const P (&pay)[kRadixIPT<P, CH>], int64_t base,
                                                 int64_t m,
                                                 uint32_t B, int shift, uint32_t off0,
                                                 uint32_t off1, KO* __restrict__ keys_out,
                                                 P* __restrict__ pay_out, int tid, int lane,
                                                 int wave) {
    constexpr int IPT = kRadixIPT<P, CH>;
    constexpr int H = CH;
    constexpr int NT = kRadixNT<P>;
    constexpr int NW = kRadixNW<P>;
    // digits up to 256 (the out-of-range bucket) need 9 bits; a first pass whose histogram
    // found no key out of range (OOR false) ranks the low byte alone
    constexpr int BITS = OOR ? 9 : 8;
    constexpr int NB = FIRST ? kBuckets0 : 256;
    uint32_t rk[IPT];
    const int64_t p0 = base + (int64_t)wave * 64 * IPT + lane;
    uint32_t* const wcnt = sm.cnt[wave];
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
        const bool valid = FULL || p0 + k * 64 < m;
        const int d = valid ? digit_of<OOR>(key[k], B, shift) : 0;
        uint32_t plo = FULL ? ~0u : (uint32_t)__ballot(valid);
        uint32_t phi = FULL ? ~0u : (uint32_t)(__ballot(valid) >> 32);
#pragma unroll
        for (int b = 0; b < BITS; ++b) {
            // the lane's bit b as 0 or all ones, kept opaque so the ballot compares it directly
            uint32_t rep = (uint32_t)__builtin_amdgcn_sbfe(d, b, 1);
            asm volatile("" : "+v"(rep));
            const uint64_t mb = __builtin_amdgcn_ballot_w64(rep != 0u);
            // keep the lanes whose bit b agrees with this lane's: mask & ~(rep ^ ballot), one
            // three-input bit operation per 32-lane half (truth table 0x90)
            plo = __builtin_amdgcn_bitop3_b32(plo, rep, (uint32_t)mb, 0x90);
            phi = __builtin_amdgcn_bitop3_b32(phi, rep, (uint32_t)(mb >> 32), 0x90);
        }
        const uint32_t below = __builtin_amdgcn_mbcnt_hi(phi, __builtin_amdgcn_mbcnt_lo(plo, 0u));
        // every lane reads its digit's counter; then the lowest lane of each group of peers
        // adds the group's size.  A wave's LDS instructions run in order and each write waits
        // for its row's read, so the next row reads the advanced counters.
        const uint32_t old = valid ? wcnt[d] : 0u;
        if (valid && below == 0u) wcnt[d] = old + (uint32_t)__popc(plo) + (uint32_t)__popc(phi);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        rk[k] = old + below;
    }
    __syncthreads();
    // per digit: wave offsets (exclusive over waves) and the chunk's count
    uint32_t tot = 0;
    if (tid < 256) {
        uint32_t run = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint32_t cw = sm.cnt[w][tid];
            sm.cnt[w][tid] = run;
            run += cw;
        }
        tot = run;
        if (NB > 256 && tid == 0) {
            uint32_t r2 = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const uint32_t cw = sm.cnt[w][256];
                sm.cnt[w][256] = r2;
                r2 += cw;
            }
        }
    }
    uint32_t total;
    const uint32_t ds = block_excl_scan_u32<NW>(tot, sm.s4, &total);
    // the digit's start in the staged chunk folded into every wave's offset, so staging reads
    // one counter per item
    if (tid < 256) {
#pragma unroll
        for (int w = 0; w < NW; ++w) sm.cnt[w][tid] += ds;
        sm.gbase[tid] = off0 - ds;
    }
    if (NB > 256 && tid == 0) {
#pragma unroll
        for (int w = 0; w < NW; ++w) sm.cnt[w][256] += total;
        sm.gbase[256] = off1 - total;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
        if (FULL || p0 + k * 64 < m) {
            const int d = digit_of<OOR>(key[k], B, shift);
            const uint32_t lp = sm.cnt[wave][d] + rk[k];
            if constexpr (RadixSmem<P, CH>::kPacked) {
                sm.kp[lp] = (uint64_t)key[k] | ((uint64_t)pay[k] << 32);
            } else {
                sm.keys[lp] = key[k];
                sm.pay[lp] = pay[k];
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < NW * kBuckets0; i += NT) (&sm.cnt[0][0])[i] = 0u;
    // staged position i to its global index: gbase[digit] + i (below 2^31, so the 32-bit sum
    // is exact)
    auto emit = [&](int i) {
        uint32_t kk;
        P pp;
        if constexpr (RadixSmem<P, CH>::kPacked) {
            const uint64_t v = sm.kp[i];
            kk = (uint32_t)v;
            pp = (P)(v >> 32);
        } else {
            kk = sm.keys[i];
            pp = sm.pay[i];
        }
        const int64_t g = (int64_t)(sm.gbase[digit_of<OOR>(kk, B, shift)] + (uint32_t)i);
        put_key<KO>(keys_out, g, kk);
        pay_out[g] = pp;
    };
    if constexpr (FULL) {
        // a fixed number of stores, so a later wait on loads issued before them stays partial
#pragma unroll
        for (int k = 0; k < IPT; ++k) emit(k * NT + tid);
    } else {
        const int cntc = (int)((m - base) < H ? (m - base) : H);
        for (int i = tid; i < cntc; i += NT) emit(i);
    }
    __syncthreads();
}

// One chunk per workgroup, chunk xcd_chunk(b) for workgroup b: the dispatcher starts
// workgroups in order, so the chunks an XCD holds at any moment are neighbours and their
// writes into each bucket's region merge in its L2.
// KO: the type keys are written in, KI the type they are read in (uint16_t for passes after
// the first when every valid key fits 16 bits).
template <typename P, int CH, bool FIRST, bool ROWS, typename KO, typename KI>
__global__ __launch_bounds__(kRadixNT<P>) void k_radix_scatter(
    const KI* __restrict__ keys_in, const P* __restrict__ pay_in,
    KO* __restrict__ keys_out, P* __restrict__ pay_out, int64_t n,
    const uint32_t* __restrict__ nvalid, uint32_t B, int shift, int64_t nchunks,
    const uint32_t* __restrict__ hist_ex, const uint32_t* __restrict__ ident) {
    constexpr int IPT = kRadixIPT<P, CH>;
    constexpr int H = CH;
    constexpr int NB = FIRST ? kBuckets0 : 256;
    __shared__ RadixSmem<P, CH> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t m = FIRST ? n : (int64_t)*nvalid;
    const int64_t c = xcd_chunk(blockIdx.x, nchunks);
    const int64_t base = c * H;
    if (base >= m) return;
    if (*ident) {
        // one bucket holds every key: the stable pass leaves every item where it is
        uint32_t key[IPT];
        P pay[IPT];
        radix_load<P, CH, FIRST, ROWS, false, KI>(keys_in, pay_in, base, m, key, pay, wave, lane);
        const int64_t p0 = base + (int64_t)wave * 64 * IPT + lane;
#pragma unroll
        for (int k = 0; k < IPT; ++k) {
            const int64_t p = p0 + k * 64;
            if (p < m) {
                put_key<KO>(keys_out, p, key[k]);
                pay_out[p] = pay[k];
            }
        }
        return;
    }
    // this chunk's bucket offsets, fetched with the keys
    const uint32_t off0 = tid < 256 ? hist_ex[c * NB + tid] : 0u;
    const uint32_t off1 = (NB > 256 && tid == 0) ? hist_ex[c * NB + 256] : 0u;
    for (int i = tid; i < kRadixNW<P> * kBuckets0; i += kRadixNT<P>) (&sm.cnt[0][0])[i] = 0u;
    uint32_t key[IPT];
    P pay[IPT];
    if (base + H <= m) {
        radix_load<P, CH, FIRST, ROWS, true, KI>(keys_in, pay_in, base, m, key, pay, wave, lane);
        __syncthreads();
        if (FIRST && nvalid[1])   // no key out of range: 8-bit ranking
            radix_rank_write<P, CH, FIRST, ROWS, true, KO, false>(
                sm, key, pay, base, m, B, shift, off0, off1, keys_out, pay_out, tid, lane, wave);
        else
            radix_rank_write<P, CH, FIRST, ROWS, true, KO>(sm, key, pay, base, m, B, shift, off0,
                                                           off1, keys_out, pay_out, tid, lane,
                                                           wave);
    } else {
        radix_load<P, CH, FIRST, ROWS, false, KI>(keys_in, pay_in, base, m, key, pay, wave, lane);
        __syncthreads();
        radix_rank_write<P, CH, FIRST, ROWS, false, KO>(sm, key, pay, base, m, B, shift, off0, off1,
                                                keys_out, pay_out, tid, lane, wave);
    }
}

// One radix pass over chunks of H keys (kChunkSmall or kChunkBig<P>, as the layout chose).
template <typename P, bool FIRST, bool ROWS, typename KO, typename KI>
void radix_scatter(int64_t H, unsigned grid, size_t lds, hipStream_t s, const KI* keys_in,
                   const P* pay_in, KO* keys_out, P* pay_out, int64_t n, const uint32_t* nvalid,
                   uint32_t B, int shift, int64_t nchunks, const uint32_t* hist_ex,
                   const uint32_t* ident) {
    if (H == kChunkSmall)
        k_radix_scatter<P, kChunkSmall, FIRST, ROWS, KO, KI><<<grid, kRadixNT<P>, lds, s>>>(
            keys_in, pay_in, keys_out, pay_out, n, nvalid, B, shift, nchunks, hist_ex, ident);
    else
        k_radix_scatter<P, kChunkBig<P>, FIRST, ROWS, KO, KI><<<grid, kRadixNT<P>, lds, s>>>(
            keys_in, pay_in, keys_out, pay_out, n, nvalid, B, shift, nchunks, hist_ex, ident);
}

// ---------------------------------------------------------------- 10-bit radix pass (f64)

// Chunks of 4096 (key, f64 payload), 4 waves of 16 items per thread, as k_radix_scatter with
// 1024 digits (1025 in a first pass that may meet keys out of range).  LDS: keys 16 KB,
// payloads 32 KB, per-wave counters 16 KB, digit bases 4 KB: two workgroups per CU.
constexpr int kWideCH = 4096;
struct RadixSmemW {
    uint32_t keys[kWideCH];
    uint64_t pay[kWideCH];
    uint32_t cnt[4][kWideCols];
    uint32_t gbase[kWideCols];
    uint32_t s4[4];
};
struct KeyW16 {};   // the key's high 10 bits as a 16-bit key

template <typename KO>
__device__ __forceinline__ void put_key_w(KO* keys_out, int64_t g, uint32_t kk) {
    if constexpr (__is_same(KO, KeyW16))
        reinterpret_cast<uint16_t*>(keys_out)[g] = (uint16_t)(kk >> kWideBits);
    else
        (void)keys_out, (void)g, (void)kk;
}

// Rank, stage and write one loaded chunk (as radix_rank_write).  Thread t owns digits 4t ..
// 4t + 3 for the per-digit steps, and thread 0 also digit 1024 in a first pass.
template <bool FIRST, bool FULL, typename KO, bool OOR>
__device__ __forceinline__ void radix_rank_write_w(RadixSmemW& sm, const uint32_t (&key)[16],
                                                   const uint64_t (&pay)[16], int64_t base,
                                                   int64_t m, uint32_t B,
                                                   const uint32_t (&off0)[4], uint32_t off1,
                                                   KO* __restrict__ keys_out,
                                                   uint64_t* __restrict__ pay_out, int tid,
                                                   int lane, int wave) {
    constexpr int IPT = 16, NT = 256, NW = 4;
    constexpr int BITS = OOR ? kWideBits + 1 : kWideBits;
    uint32_t rk[IPT];
    const int64_t p0 = base + (int64_t)wave * 64 * IPT + lane;
    uint32_t* const wcnt = sm.cnt[wave];
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
        const bool valid = FULL || p0 + k * 64 < m;
        const int d = valid ? wide_digit<OOR>(key[k], B, 0) : 0;
        uint32_t plo = FULL ? ~0u : (uint32_t)__ballot(valid);
        uint32_t phi = FULL ? ~0u : (uint32_t)(__ballot(valid) >> 32);
#pragma unroll
        for (int b = 0; b < BITS; ++b) {
            uint32_t rep = (uint32_t)__builtin_amdgcn_sbfe(d, b, 1);
            asm volatile("" : "+v"(rep));
            const uint64_t mb = __builtin_amdgcn_ballot_w64(rep != 0u);
            plo = __builtin_amdgcn_bitop3_b32(plo, rep, (uint32_t)mb, 0x90);
            phi = __builtin_amdgcn_bitop3_b32(phi, rep, (uint32_t)(mb >> 32), 0x90);
        }
        const uint32_t below = __builtin_amdgcn_mbcnt_hi(phi, __builtin_amdgcn_mbcnt_lo(plo, 0u));
        const uint32_t old = valid ? wcnt[d] : 0u;
        if (valid && below == 0u) wcnt[d] = old + (uint32_t)__popc(plo) + (uint32_t)__popc(phi);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        rk[k] = old + below;
    }
    __syncthreads();
    // per digit: the waves' exclusive offsets and the chunk's count
    uint32_t dtot[4], loc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int d = 4 * tid + j;
        uint32_t run = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint32_t cw = sm.cnt[w][d];
            sm.cnt[w][d] = run;
            run += cw;
        }
        dtot[j] = run;
        loc += run;
    }
    if (FIRST && tid == 0) {
        uint32_t r2 = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint32_t cw = sm.cnt[w][kWideB];
            sm.cnt[w][kWideB] = r2;
            r2 += cw;
        }
    }
    uint32_t total;
    uint32_t ds = block_excl_scan_u32<NW>(loc, sm.s4, &total);
    // each digit's start in the staged chunk folded into every wave's offset
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int d = 4 * tid + j;
#pragma unroll
        for (int w = 0; w < NW; ++w) sm.cnt[w][d] += ds;
        sm.gbase[d] = off0[j] - ds;
        ds += dtot[j];
    }
    if (FIRST && tid == 0) {
#pragma unroll
        for (int w = 0; w < NW; ++w) sm.cnt[w][kWideB] += total;
        sm.gbase[kWideB] = off1 - total;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
        if (FULL || p0 + k * 64 < m) {
            const int d = wide_digit<OOR>(key[k], B, 0);
            const uint32_t lp = sm.cnt[wave][d] + rk[k];
            sm.keys[lp] = key[k];
            sm.pay[lp] = pay[k];
        }
    }
    __syncthreads();
    auto emit = [&](int i) {
        const uint32_t kk = sm.keys[i];
        const int64_t g = (int64_t)(sm.gbase[wide_digit<OOR>(kk, B, 0)] + (uint32_t)i);
        put_key_w<KO>(keys_out, g, kk);
        pay_out[g] = sm.pay[i];
    };
    if constexpr (FULL) {
#pragma unroll
        for (int k = 0; k < IPT; ++k) emit(k * NT + tid);
    } else {
        const int cntc = (int)((m - base) < kWideCH ? (m - base) : kWideCH);
        for (int i = tid; i < cntc; i += NT) emit(i);
    }
}

// One chunk per workgroup (xcd_chunk placement), as k_radix_scatter.
template <bool FIRST, typename KO, typename KI>
__global__ __launch_bounds__(256) void k_radix_scatter_w(
    const KI* __restrict__ keys_in, const uint64_t* __restrict__ pay_in,
    KO* __restrict__ keys_out, uint64_t* __restrict__ pay_out, int64_t n,
    const uint32_t* __restrict__ nvalid, uint32_t B, int64_t nchunks,
    const uint32_t* __restrict__ hist_ex, const uint32_t* __restrict__ ident) {
    constexpr int IPT = 16;
    constexpr int NB = FIRST ? kWideCols : kWideB;
    __shared__ RadixSmemW sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t m = FIRST ? n : (int64_t)*nvalid;
    const int64_t c = xcd_chunk(blockIdx.x, nchunks);
    const int64_t base = c * kWideCH;
    if (base >= m) return;
    uint32_t key[IPT];
    uint64_t pay[IPT];
    if (*ident) {
        // one bucket holds every key: the pass leaves every item where it is
        radix_load<uint64_t, kWideCH, FIRST, false, false, KI>(keys_in, pay_in, base, m, key, pay,
                                                                wave, lane);
        const int64_t p0 = base + (int64_t)wave * 64 * IPT + lane;
#pragma unroll
        for (int k = 0; k < IPT; ++k) {
            const int64_t p = p0 + k * 64;
            if (p < m) {
                put_key_w<KO>(keys_out, p, key[k]);
                pay_out[p] = pay[k];
            }
        }
        return;
    }
    uint32_t off0[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) off0[j] = hist_ex[c * NB + 4 * tid + j];
    const uint32_t off1 = (FIRST && tid == 0) ? hist_ex[c * NB + kWideB] : 0u;
    for (int i = tid; i < 4 * kWideCols; i += 256) (&sm.cnt[0][0])[i] = 0u;
    if (base + kWideCH <= m) {
        radix_load<uint64_t, kWideCH, FIRST, false, true, KI>(keys_in, pay_in, base, m, key, pay,
                                                               wave, lane);
        __syncthreads();
        if (FIRST && nvalid[1])   // no key out of range: 10-bit ranking
            radix_rank_write_w<FIRST, true, KO, false>(sm, key, pay, base, m, B, off0, off1,
                                                       keys_out, pay_out, tid, lane, wave);
        else
            radix_rank_write_w<FIRST, true, KO, FIRST>(sm, key, pay, base, m, B, off0, off1,
                                                       keys_out, pay_out, tid, lane, wave);
    } else {
        radix_load<uint64_t, kWideCH, FIRST, false, false, KI>(keys_in, pay_in, base, m, key, pay,
                                                                wave, lane);
        __syncthreads();
        radix_rank_write_w<FIRST, false, KO, FIRST>(sm, key, pay, base, m, B, off0, off1,
                                                    keys_out, pay_out, tid, lane, wave);
    }
}

// ---------------------------------------------------------------- destinations

// off[b] = first sorted position with key >= b, for b in [0, B]; n_skipped = n - valid.
// row0: the last radix pass's bucket starts (row 0 of its offsets), or null.  With one pass
// (destinations below 256: every key is one bucket) they are the answer; with two passes over
// keys below 2^16 (16- or 32-bit) the keys of high byte h lie in that pass's bucket h, so the
// search for b stays inside bucket b >> 8 (f32 2^28 into 65,536 bins on MI355X: 31 -> 18 us);
// with more passes the whole array is searched.
template <typename KT>
__global__ __launch_bounds__(256) void k_bin_offsets(const KT* __restrict__ K,
                                                     const uint32_t* __restrict__ nvalid,
                                                     int64_t B, int64_t n, uint32_t* __restrict__ off,
                                                     int64_t* __restrict__ n_skipped,
                                                     const uint32_t* __restrict__ row0,
                                                     int passes) {
    const int64_t m = *nvalid;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b <= B;
         b += (int64_t)gridDim.x * blockDim.x) {
        if (row0 && passes == 1) {   // b <= B <= 256; row0[256] is the out-of-range bucket's start, m
            off[b] = row0[b];
            continue;
        }
        int64_t lo = 0, hi = m;
        if (row0 && passes == 2) {
            const int64_t h = b >> 8;
            lo = h < 256 ? (int64_t)row0[h] : m;
            hi = h < 255 ? (int64_t)row0[h + 1] : m;
        }
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if ((int64_t)K[mid] < b) lo = mid + 1;
            else hi = mid;
        }
        off[b] = (uint32_t)lo;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0 && n_skipped) *n_skipped = n - m;
}

// The two-pass byte path (destinations below 2^16, scalar values): off[b] for b = 256 h + l
// (high byte h, low byte l) is the number of valid keys below b, i.e. those with a high byte
// below h, plus those with high byte h and a low byte below l.  The first pass sorted by the
// low byte, so the keys with a low byte below l are its output's positions [0, row1[l]) (row1:
// that pass's bucket starts); the second pass's offsets ex2[c][h] count the keys with a high
// byte below h plus those with high byte h in the chunks (of H positions of the first pass's
// output) before c.  With c the chunk holding position row1[l], off[b] = ex2[c][h] + the keys
// of high byte h in [c H, row1[l]), counted here from the first pass's key bytes; when
// row1[l] = m no key has a low byte of l or more, and off[b] = the start of bucket h + 1.
// Integers only.  A workgroup per low byte, a thread per high byte.
// (Three-pass path: the same with KH = uint16_t, the first pass's output keys holding bits
// 8..23, whose low byte is the second digit; it yields the offsets of the 16-bit low part of
// every key, B = 65536, and k_bin_offsets_third takes it from there.)
template <typename KH>
__global__ __launch_bounds__(256) void k_bin_offsets_bytes(
    const uint32_t* __restrict__ row1, const uint32_t* __restrict__ ex2,
    const KH* __restrict__ hb, const uint32_t* __restrict__ nvalid, int64_t B, int64_t n,
    int64_t H, uint32_t* __restrict__ off, int64_t* __restrict__ n_skipped) {
    __shared__ uint32_t cnt[256];
    const int l = blockIdx.x, h = threadIdx.x;
    const int64_t m = *nvalid;
    const int64_t pos = row1[l];
    cnt[h] = 0u;
    __syncthreads();
    const int64_t c = pos / H;
    if (pos < m) {
        // the keys of [c H, pos), four 8-bit or two 16-bit keys to a 32-bit word (chunk starts
        // are multiples of H, so the words are aligned), every word of a thread loaded before
        // any is counted; the last word may reach past pos, inside the key array
        constexpr int KPW = 4 / (int)sizeof(KH);
        constexpr int MAXW = kChunkBig<uint32_t> / KPW / 256;   // H is at most 8192
        const int nk = (int)(pos - c * H);
        const int nw = (nk + KPW - 1) / KPW;
        const uint32_t* hw = reinterpret_cast<const uint32_t*>(hb + c * H);
        uint32_t x[MAXW];
#pragma unroll
        for (int k = 0; k < MAXW; ++k) x[k] = k * 256 + h < nw ? hw[k * 256 + h] : 0u;
#pragma unroll
        for (int k = 0; k < MAXW; ++k)
#pragma unroll
            for (int j = 0; j < KPW; ++j)
                if (KPW * (k * 256 + h) + j < nk)
                    count_digit(cnt, (int)((x[k] >> (32 / KPW * j)) & 255u));
    }
    __syncthreads();
    const int64_t b = (int64_t)h * 256 + l;
    if (b < B) {
        uint32_t o;
        if (pos < m) o = ex2[c * 256 + h] + cnt[h];
        else o = h < 255 ? ex2[h + 1] : (uint32_t)m;   // row 0 of ex2: the bucket starts
        off[b] = o;
    }
    if (l == 0 && h == 0) {
        off[B] = (uint32_t)m;
        if (n_skipped) *n_skipped = n - m;
    }
}

// The 10-bit path: off[b] for b = 1024 h + l (l the low 10 bits, h the high ones) = the keys
// with a high part below h, plus those with high part h and low part below l.  The first pass
// put low part l at positions from pos = row1[l] on; with c the chunk holding pos, the second
// pass's offset of digit h in chunk c counts the first kind and the keys of high part h in
// chunk c before pos, and the keys of [c H, pos) with high part h (counted here from the first
// pass's 16-bit keys) complete it; when pos = m, off[b] = the start of the second pass's bucket
// h + 1.  Workgroup l, thread t takes h = t + 256 j.
__global__ __launch_bounds__(256) void k_bin_offsets_w(const uint32_t* __restrict__ row1,
                                                       const uint32_t* __restrict__ ex2,
                                                       const uint16_t* __restrict__ hb,
                                                       const uint32_t* __restrict__ nvalid,
                                                       int64_t B, int64_t n, int64_t H,
                                                       uint32_t* __restrict__ off,
                                                       int64_t* __restrict__ n_skipped) {
    __shared__ uint32_t cnt[kWideB];
    const int l = blockIdx.x, t = threadIdx.x;
    const int64_t m = *nvalid;
    const int64_t pos = row1[l];
#pragma unroll
    for (int j = 0; j < 4; ++j) cnt[t + 256 * j] = 0u;
    __syncthreads();
    const int64_t c = pos / H;
    if (pos < m) {
        // the 16-bit keys of [c H, pos), two to a 32-bit word, every word of a thread loaded
        // before any is counted (as k_bin_offsets_bytes)
        constexpr int MAXW = kWideCH / 2 / 256;
        const int nk = (int)(pos - c * H);
        const int nw = (nk + 1) / 2;
        const uint32_t* hw = reinterpret_cast<const uint32_t*>(hb + c * H);
        uint32_t x[MAXW];
#pragma unroll
        for (int k = 0; k < MAXW; ++k) x[k] = k * 256 + t < nw ? hw[k * 256 + t] : 0u;
#pragma unroll
        for (int k = 0; k < MAXW; ++k)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (2 * (k * 256 + t) + j < nk)
                    count_digit(cnt, (int)((x[k] >> (16 * j)) & (uint32_t)(kWideB - 1)));
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int h = t + 256 * j;
        const int64_t b = (int64_t)h * kWideB + l;
        if (b < B) {
            uint32_t o;
            if (pos < m) o = ex2[c * kWideB + h] + cnt[h];
            else o = h < kWideB - 1 ? ex2[h + 1] : (uint32_t)m;   // row 0: the bucket starts
            off[b] = o;
        }
    }
    if (l == 0 && t == 0) {
        off[B] = (uint32_t)m;
        if (n_skipped) *n_skipped = n - m;
    }
}

// The three-pass path (scalar destinations in (65536, 2^24]): off[b] for b = 65536 t + p (t the
// key's third byte, p its low 16 bits) = the keys with a third byte below t, plus those with
// third byte t and low part below p.  off2[p] (k_bin_offsets_bytes on the first two passes) is
// where the low parts of p and above start in the second pass's output, which the third pass
// sorted by the third byte; with c the chunk holding position off2[p], off[b] = ex3[c][t] + the
// keys of third byte t in [c H, off2[p]), counted from the second pass's key bytes; when
// off2[p] = m, off[b] = the start of the third pass's bucket t + 1.  A wave per p (f64 2^29
// into 2^20 Zipf bins on MI355X, the whole offsets step: 0.24 ms with a workgroup per p counting
// from the chunk start, 0.11 ms now), a lane per four t.
__global__ __launch_bounds__(256) void k_bin_offsets_third(
    const uint32_t* __restrict__ off2, const uint32_t* __restrict__ ex3,
    const uint8_t* __restrict__ tb, const uint32_t* __restrict__ nvalid, int64_t B, int64_t n,
    int64_t H, uint32_t* __restrict__ off, int64_t* __restrict__ n_skipped) {
    // a wave per low part p (four per workgroup), its own counters; lane l reads the key bytes
    // four to a word (H is a multiple of 4, the bytes 256-byte aligned)
    __shared__ uint32_t cnt[4][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t p = (int64_t)blockIdx.x * 4 + wave;
    if (p >= 65536) return;   // a whole wave; nothing below waits for other waves
    uint32_t* const wc = cnt[wave];
#pragma unroll
    for (int k = 0; k < 4; ++k) wc[lane + 64 * k] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t m = *nvalid;
    const int64_t pos = off2[p];
    const int64_t c = pos / H;
    const int64_t cend = (c + 1) * H < m ? (c + 1) * H : m;   // end of chunk c's keys
    // count the bytes of chunk c before pos, or, when fewer, those from pos to its end and
    // take them from where the chunk's digit t ends (the next chunk's offset, or for the last
    // chunk the end of bucket t)
    const bool after = cend - pos < pos - c * H;
    if (pos < m) {
        const int64_t q0 = after ? pos : c * H, q1 = after ? cend : pos;
        // words from the one holding q0 (H is a multiple of 4, the bytes 256-byte aligned)
        const uint32_t* tw = reinterpret_cast<const uint32_t*>(tb) + q0 / 4;
        const int64_t w0 = q0 & ~int64_t(3);
        for (int64_t w = lane; w0 + 4 * w < q1; w += 64) {
            const uint32_t x = tw[w];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t q = w0 + 4 * w + j;
                if (q >= q0 && q < q1) count_digit(wc, (int)((x >> (8 * j)) & 255u));
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t nch = (n + H - 1) / H;   // rows of ex3
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int t = lane + 64 * k;
        const int64_t b = (int64_t)t * 65536 + p;
        if (b < B) {
            // row 0 of ex3 holds the bucket starts; bucket t ends where t + 1 starts
            const uint32_t bend = t < 255 ? ex3[t + 1] : (uint32_t)m;
            uint32_t o;
            if (pos >= m) o = bend;
            else if (!after) o = ex3[c * 256 + t] + wc[t];
            else o = (c + 1 < nch ? ex3[(c + 1) * 256 + t] : bend) - wc[t];
            off[b] = o;
        }
    }
    if (p == 0 && lane == 0) {
        off[B] = (uint32_t)m;
        if (n_skipped) *n_skipped = n - m;
    }
}

// rbin[r] = the destination holding sorted position p = r * kSegD, for r < nr = ceil(m / kSegD):
// the last b in [0, B) with off[b] <= p (off[0] = 0 <= p and off[B] = m > p, so it exists, and
// off[b + 1] > p).  A wave per range narrows [lo, hi) 64 ways per step (a ballot over 64 probes
// of the non-decreasing offsets).
__global__ __launch_bounds__(256) void k_range_bins(const uint32_t* __restrict__ off, int64_t B,
                                                    int64_t nr, uint32_t* __restrict__ rbin) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= nr) return;
    const int64_t p = r * kSegD;
    int64_t lo = 0, hi = B;
    while (hi - lo > 1) {
        const int64_t step = cdiv(hi - lo, 64);
        const int64_t k = lo + (int64_t)lane * step;
        const uint64_t le = __ballot(k < hi && (int64_t)off[k] <= p);   // lane 0 always
        const int last = 63 - __builtin_clzll(le);
        lo += (int64_t)last * step;
        if (lo + step < hi) hi = lo + step;
    }
    if (lane == 0) rbin[r] = (uint32_t)lo;
}

template <typename T>
__global__ void k_prev_gather(const int32_t* __restrict__ index, int64_t n, int64_t d, int64_t B,
                              const T* __restrict__ out, T* __restrict__ prev) {
    const int64_t total = n * d;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = e / d;
        const int64_t c = e - i * d;
        const int64_t b = index[i];
        if (b >= 0 && b < B) prev[e] = out[b * d + c];
    }
}

template <typename T>
__global__ void k_write_skipped_all(int64_t* n_skipped, int64_t n) {
    *n_skipped = n;
}

// ---------------------------------------------------------------- scalar reduction

// PW over p[0 .. len) (each element negated when NEG; the identity padding is not), len <= 256
// NBLK (element 0 replaced by v0 when use_v0): NBLK blocks
// of 256; lane l of block i holds elements 256 i + 4 l .. + 4 combined as (a0 + a1) + (a2 + a3),
// then the wave butterfly; the block values meet in the log2(NBLK)-level tree (identity for
// blocks past len), built as a binary counter of complete subtrees and folded right-nested at
// the end, which is PW over 256 NBLK padded positions, the same value as over len.  The loads
// of G blocks are in flight together.  Uniform result.
template <typename T, int NBLK = 32, bool NEG = false>
__device__ __forceinline__ T wave_pw_range(const T* __restrict__ p, int64_t len, int lane,
                                           bool use_v0, T v0) {
    // blocks whose loads are in flight together: few enough registers that more workgroups
    // fit per CU (f32 2^28 into 65,536 bins on MI355X: 16 blocks 0.40 ms, 8 0.36, 4 0.34;
    // f64 2^27 into 2^20 bins: 8 blocks 0.68 ms, 4 0.69, 2 0.71)
    constexpr int G0 = sizeof(T) == 4 ? 4 : 8;
    constexpr int G = G0 < NBLK ? G0 : NBLK;
    constexpr int LV = NBLK <= 2 ? 2 : NBLK <= 8 ? 4 : 6;   // stack levels (log2 NBLK + 1)
    // complete subtrees of the block values pushed so far, by level (a binary counter): leaf
    // L merges with the stack's top levels for the trailing ones of L, exactly the pairs of the
    // NBLK-leaf tree
    T stk[LV];
#pragma unroll
    for (int l = 0; l < LV; ++l) stk[l] = ident<T>();
    int nleaf = 0;
#pragma unroll
    for (int g0 = 0; g0 < NBLK; g0 += G) {
        if ((int64_t)g0 * 256 >= len) break;
        T a[G][4];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int blk = (g0 + i) * 256;
            const T* q = p + blk + 4 * lane;
            const int rem = (int)((len - blk) < 256 ? (len - blk) : 256) - 4 * lane;
            if (sizeof(T) == 4 && rem >= 4) {
                // f32: the lane's 4 values by one 16-byte load (element-aligned only: the
                // hardware takes unaligned vector accesses; f32 2^24 into 65,536 bins on MI355X
                // 26.3 -> 18.5 us for the reduction, while f64's two 16-byte loads were no faster)
                typedef T T4 __attribute__((ext_vector_type(4)));
                T4 x;
                __builtin_memcpy(&x, q, sizeof(T4));
                a[i][0] = NEG ? -x.x : x.x;
                a[i][1] = NEG ? -x.y : x.y;
                a[i][2] = NEG ? -x.z : x.z;
                a[i][3] = NEG ? -x.w : x.w;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) a[i][r] = rem > r ? (NEG ? -q[r] : q[r]) : ident<T>();
            }
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int L = g0 + i;
            if ((int64_t)L * 256 < len) {
                if (use_v0 && L == 0 && lane == 0) a[i][0] = v0;
                T v = wave_pw<T>((a[i][0] + a[i][1]) + (a[i][2] + a[i][3]));
                const int tz = __builtin_ctz(~(unsigned)L);   // trailing ones of L
#pragma unroll
                for (int l = 0; l < LV; ++l)
                    if (l < tz) v = stk[l] + v;
#pragma unroll
                for (int l = 0; l < LV; ++l)
                    if (l == tz) stk[l] = v;
                nleaf = L + 1;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // the padded tree's value: the complete subtrees of nleaf's binary expansion folded
    // right-nested (identity leaves change nothing)
    T acc = ident<T>();
    bool have = false;
#pragma unroll
    for (int l = 0; l < LV; ++l) {
        if ((nleaf >> l) & 1) {
            acc = have ? stk[l] + acc : stk[l];
            have = true;
        }
    }
    return acc;
}

// PW over p[0 .. len) for any len (element 0 replaced by v0 when use_v0): blocks of 8192
// by wave_pw_range, merged by a binary counter whose stack lives in LDS (lane 0), then
// folded right-nested.
template <typename T>
__device__ __forceinline__ T wave_pw_long(const T* __restrict__ p, int64_t len, int lane, bool use_v0,
                                       T v0, T* stk) {
    const int64_t nblk = cdiv(len, 8192);
    for (int64_t s = 0; s < nblk; ++s) {
        const int64_t o = s * 8192;
        const int64_t l = (len - o) < 8192 ? (len - o) : 8192;
        // the shortest padded width that holds the block (all give the same value)
        const bool v0s = use_v0 && s == 0;
        T v = l <= 512    ? wave_pw_range<T, 2>(p + o, l, lane, v0s, v0)
              : l <= 2048 ? wave_pw_range<T, 8>(p + o, l, lane, v0s, v0)
                          : wave_pw_range<T>(p + o, l, lane, v0s, v0);
        if (lane == 0) {
            int64_t k = s;
            int lvl = 0;
            while (k & 1) {
                v = stk[lvl] + v;
                k >>= 1;
                ++lvl;
            }
            stk[lvl] = v;
        }
    }
    T acc = ident<T>();
    if (lane == 0) {
        bool have = false;
        for (int lvl = 0; lvl < 40; ++lvl) {
            if ((nblk >> lvl) & 1) {
                acc = have ? stk[lvl] + acc : stk[lvl];
                have = true;
            }
        }
    }
    return readlane(acc, 0);
}

// PW over v[0 .. len) (each element negated when NEG), len <= 32, by one lane: pad to 32 with
// the identity, 5-level tree
template <typename T, bool NEG = false>
__device__ __forceinline__ T lane_pw_32(const T* __restrict__ v, int len) {
    // whole groups of W values by one 16-byte load each (element-aligned only: the hardware
    // takes unaligned vector accesses), the rest one by one
    constexpr int W = 16 / (int)sizeof(T);
    typedef T TW __attribute__((ext_vector_type(W)));
    T a[32];
#pragma unroll
    for (int q = 0; q < 32; q += W) {
        if (q + W <= len) {
            TW x;
            __builtin_memcpy(&x, v + q, 16);
#pragma unroll
            for (int r = 0; r < W; ++r) a[q + r] = NEG ? -x[r] : x[r];
        } else {
#pragma unroll
            for (int r = 0; r < W; ++r)
                a[q + r] = q + r < len ? (NEG ? -v[q + r] : v[q + r]) : ident<T>();
        }
    }
#pragma unroll
    for (int w = 32; w > 1; w /= 2) {
#pragma unroll
        for (int i = 0; i < w / 2; ++i) a[i] = a[2 * i] + a[2 * i + 1];
    }
    return a[0];
}

// Store the value of the block starting at sorted position ps (local rank k*D of bin b).
template <typename T>
__device__ __forceinline__ void emit_scalar(T S, int64_t ps, uint32_t b, int64_t seg_s,
                                            int64_t seg_e, T* __restrict__ out,
                                            T* __restrict__ pF, T* __restrict__ pC) {
    if (seg_e - seg_s <= kSegD) {
        out[b] = out[b] + S;
    } else if (ps == seg_s) {
        pF[ps / kSegD] = S;
    } else {
        pC[ps / kSegD] = S;
    }
}

// Blocks longer than 32 values (s_big: position in the range, destination, the destination's
// first and end positions), reduced by all four waves of the workgroup: each block is cut at
// multiples of 1024 of its positions (aligned subtrees of its tree) and a wave takes one piece at
// a time; then a thread per block combines the block's up to 8 piece values by the 8-leaf tree
// (missing pieces are the identity), which is the block's PW, and stores it.  A range holding
// one or two long blocks so keeps every wave loading, where a wave per block left two of four
// idle for four rounds of loads each.
constexpr int kPiece = 1024;
constexpr int kMaxBig = kSegD / 32 + 2;
constexpr int kMaxPieces = kMaxBig + 2 * (kSegD / kPiece);   // lengths sum to at most 2 kSegD

template <typename T, bool NEG>
__device__ __forceinline__ void reduce_big_blocks(const uint32_t (*s_big)[4], int nbig,
                                                  int64_t lo, const T* __restrict__ V,
                                                  T* __restrict__ out, T* __restrict__ pF,
                                                  T* __restrict__ pC, uint16_t* s_piece,
                                                  T* s_pval, uint32_t* s4, int tid, int lane,
                                                  int wave) {
    static_assert(kSegD / 33 + 1 <= 256, "a thread per block");
    static_assert(kSegD / kPiece <= 8 && kMaxBig * 8 < 65536, "piece index in 16 bits");
    int64_t ps = 0, seg_s = 0, seg_e = 0;
    uint32_t b = 0, cnt = 0;
    T o = T(0);
    if (tid < nbig) {
        ps = lo + s_big[tid][0];
        b = s_big[tid][1];
        seg_s = s_big[tid][2];
        seg_e = s_big[tid][3];
        const int64_t len = (seg_e - ps) < kSegD ? (seg_e - ps) : kSegD;
        cnt = (uint32_t)cdiv(len, kPiece);
        if (seg_e - seg_s <= kSegD) o = out[b];   // the old value, read before the pieces
    }
    uint32_t total;
    const uint32_t first = block_excl_scan_u32(cnt, s4, &total);
    for (uint32_t k = 0; k < cnt; ++k) s_piece[first + k] = (uint16_t)((tid << 3) | k);
    __syncthreads();
    for (int u = wave; u < (int)total; u += 4) {
        const int h = s_piece[u] >> 3, k = s_piece[u] & 7;
        const int64_t hp = lo + s_big[h][0];
        const int64_t hlen = ((int64_t)s_big[h][3] - hp) < kSegD ? ((int64_t)s_big[h][3] - hp)
                                                                  : kSegD;
        const int64_t l = (hlen - (int64_t)k * kPiece) < kPiece ? (hlen - (int64_t)k * kPiece)
                                                                : kPiece;
        const T* v = V + hp + (int64_t)k * kPiece;
        const T S = l <= 512 ? wave_pw_range<T, 2, NEG>(v, l, lane, false, ident<T>())
                             : wave_pw_range<T, 4, NEG>(v, l, lane, false, ident<T>());
        if (lane == 0) s_pval[u] = S;
    }
    __syncthreads();
    if (tid < nbig) {
        T a[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) a[k] = k < (int)cnt ? s_pval[first + k] : ident<T>();
        const T S = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
        if (seg_e - seg_s <= kSegD) out[b] = o + S;
        else if (ps == seg_s) pF[ps / kSegD] = S;
        else pC[ps / kSegD] = S;
    }
}

// NEG: every value enters negated (scatter-subtract: the values are negated, then added in the
// same order).
template <typename T, typename KT, bool NEG>
__global__ __launch_bounds__(256) void k_segred_scalar(const KT* __restrict__ K,
                                                       const T* __restrict__ V,
                                                       const uint32_t* __restrict__ off,
                                                       const uint32_t* __restrict__ nvalid,
                                                       T* __restrict__ out, T* __restrict__ pF,
                                                       T* __restrict__ pC) {
    // blocks longer than 32 values, for the waves: position in the range, destination, and the
    // destination's first and end positions (read once, by the thread that found the block)
    __shared__ uint32_t s_big[kMaxBig][4];
    __shared__ uint32_t s_nbig;
    __shared__ uint16_t s_piece[kMaxPieces];
    __shared__ T s_pval[kMaxPieces];
    __shared__ uint32_t s4[4];
    __shared__ KT s_key[kSegD];
    __shared__ uint32_t s_prev;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t m = *nvalid;
    const int64_t lo = (int64_t)blockIdx.x * kSegD;
    if (lo >= m) return;
    const int64_t hi = (lo + kSegD < m) ? lo + kSegD : m;
    if (tid == 0) {
        s_nbig = 0u;
        s_prev = lo > 0 ? (uint32_t)K[lo - 1] : ~(uint32_t)K[lo];
    }
    // the range's keys into LDS in one round trip (16-byte loads when the range is whole; K is
    // 256-byte aligned and lo a multiple of kSegD)
    if (hi - lo == kSegD) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        constexpr int KPV = 16 / sizeof(KT);             // keys per 16-byte load
        u32x4 q[kSegD / KPV / 256];
#pragma unroll
        for (int i = 0; i < kSegD / KPV / 256; ++i)
            q[i] = reinterpret_cast<const u32x4*>(K + lo)[i * 256 + tid];
#pragma unroll
        for (int i = 0; i < kSegD / KPV / 256; ++i) {
            reinterpret_cast<u32x4*>(s_key)[i * 256 + tid] = q[i];
        }
    } else {
        for (int i = tid; i < (int)(hi - lo); i += 256) s_key[i] = K[lo + i];
    }
    __syncthreads();

    // a block starts at every segment start, and at most once more inside this range: the
    // next multiple of D (in local rank) of the destination running into the range
    auto item = [&](int64_t ps, uint32_t b, int64_t seg_s, int64_t seg_e) {
        const int64_t len = (seg_e - ps) < kSegD ? (seg_e - ps) : kSegD;
        if (len <= 32) {
            const T S = lane_pw_32<T, NEG>(V + ps, (int)len);
            emit_scalar<T>(S, ps, b, seg_s, seg_e, out, pF, pC);
        } else {
            uint32_t* e = s_big[atomicAdd(&s_nbig, 1u)];
            e[0] = (uint32_t)(ps - lo);
            e[1] = b;
            e[2] = (uint32_t)seg_s;
            e[3] = (uint32_t)seg_e;
        }
    };
    for (int i = 0; i < kSegD / 256; ++i) {
        const int e = i * 256 + tid;
        const int64_t p = lo + e;
        if (p < hi) {
            const uint32_t b = s_key[e];
            const bool head = (e == 0 ? s_prev : s_key[e - 1]) != b;
            if (head || p == lo) {
                const int64_t s0 = off[b], e0 = off[b + 1];
                if (head) item(p, b, s0, e0);
                if (p == lo && s0 < lo) {
                    const int64_t pc = s0 + cdiv(lo - s0, kSegD) * kSegD;
                    if (pc < hi && pc < e0) item(pc, b, s0, e0);
                }
            }
        }
    }
    __syncthreads();
    reduce_big_blocks<T, NEG>(s_big, (int)s_nbig, lo, V, out, pF, pC, s_piece, s_pval, s4, tid,
                              lane, wave);
}

// k_segred_scalar without keys (the byte path): the destinations meeting this range are
// rbin[range] (the one holding its first position) and those after it that start before the
// range's end, found from the offsets; every block and every value as in k_segred_scalar.
// Workgroup (range, y) of gridDim.y takes every gridDim.y-th group of 256 of them, so a range
// holding many short destinations is shared out (each destination to one workgroup).
template <typename T, bool NEG>
__global__ __launch_bounds__(256) void k_segred_off(const T* __restrict__ V,
                                                    const uint32_t* __restrict__ off, int64_t B,
                                                    const uint32_t* __restrict__ rbin,
                                                    const uint32_t* __restrict__ nvalid,
                                                    T* __restrict__ out, T* __restrict__ pF,
                                                    T* __restrict__ pC) {
    __shared__ uint32_t s_big[kMaxBig][4];
    __shared__ uint32_t s_nbig;
    __shared__ uint16_t s_piece[kMaxPieces];
    __shared__ T s_pval[kMaxPieces];
    __shared__ uint32_t s4[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t m = *nvalid;
    const int64_t lo = (int64_t)blockIdx.x * kSegD;
    if (lo >= m) return;
    const int64_t hi = (lo + kSegD < m) ? lo + kSegD : m;
    if (tid == 0) s_nbig = 0u;
    const int64_t b0 = rbin[blockIdx.x];
    __syncthreads();
    auto item = [&](int64_t ps, uint32_t b, int64_t seg_s, int64_t seg_e) {
        const int64_t len = (seg_e - ps) < kSegD ? (seg_e - ps) : kSegD;
        if (len <= 32) {
            const T S = lane_pw_32<T, NEG>(V + ps, (int)len);
            emit_scalar<T>(S, ps, b, seg_s, seg_e, out, pF, pC);
        } else {
            uint32_t* e = s_big[atomicAdd(&s_nbig, 1u)];
            e[0] = (uint32_t)(ps - lo);
            e[1] = b;
            e[2] = (uint32_t)seg_s;
            e[3] = (uint32_t)seg_e;
        }
    };
    // destinations b0, b0 + 1, ... while they start before hi (at most kSegD + 1 of them)
    for (int64_t bb = b0 + (int64_t)blockIdx.y * 256;; bb += 256 * (int64_t)gridDim.y) {
        const int64_t b = bb + tid;
        bool more = false;
        if (b < B) {
            const int64_t s0 = off[b], e0 = off[b + 1];
            more = s0 < hi;
            if (more && s0 < e0) {
                if (s0 >= lo) {
                    item(s0, (uint32_t)b, s0, e0);
                } else {
                    // the destination running into the range: its next multiple of D
                    const int64_t pc = s0 + cdiv(lo - s0, kSegD) * kSegD;
                    if (pc < hi && pc < e0) item(pc, (uint32_t)b, s0, e0);
                }
            }
        }
        if (!__syncthreads_or(more)) break;
    }
    __syncthreads();
    reduce_big_blocks<T, NEG>(s_big, (int)s_nbig, lo, V, out, pF, pC, s_piece, s_pval, s4, tid,
                              lane, wave);
}

// destinations with more than D members: PW over their block values, then apply
template <typename T>
__global__ __launch_bounds__(256) void k_segred_scalar_long(const uint32_t* __restrict__ off,
                                                            int64_t B, const T* __restrict__ pF,
                                                            const T* __restrict__ pC,
                                                            T* __restrict__ out) {
    __shared__ T s_stk[4][40];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
    const int64_t nw = (int64_t)gridDim.x * 4;
    // lane l of wave w checks destination w + l * nw (+ 64 nw per round), so neighbouring long
    // destinations (a skewed head) go to different waves; a wave then combines its long ones
    // one after another (64 neighbours per wave: f64 2^29 into 2^20 Zipf bins on MI355X, 0.24
    // ms for this kernel; one destination per wave and round: 26 us with no long destination
    // at 65,536 bins)
    for (int64_t g = gw; g < B; g += 64 * nw) {
        const int64_t b = g + (int64_t)lane * nw;
        const bool lng = b < B && (int64_t)off[b + 1] - (int64_t)off[b] > kSegD;
        uint64_t mask = __ballot(lng);
        while (mask) {
            const int l = __ffsll((long long)mask) - 1;
            mask &= mask - 1;
            const int64_t bb = g + (int64_t)l * nw;
            const int64_t seg_s = off[bb], seg_e = off[bb + 1];
            const int64_t nblk = cdiv(seg_e - seg_s, kSegD);
            const int64_t r0 = seg_s / kSegD;
            // block values: pF[r0] for the first block, pC[r0 + k] for block k >= 1
            const T S = wave_pw_long<T>(pC + r0, nblk, lane, true, pF[r0], s_stk[wave]);
            if (lane == 0) out[bb] = out[bb] + S;
        }
    }
}

// ---------------------------------------------------------------- row reduction

template <typename T, bool NEG>
__global__ __launch_bounds__(256) void k_segred_rows(const uint32_t* __restrict__ K,
                                                     const uint32_t* __restrict__ R,
                                                     const uint32_t* __restrict__ off,
                                                     const uint32_t* __restrict__ nvalid,
                                                     const T* __restrict__ src, int64_t d,
                                                     T* __restrict__ out, T* __restrict__ pF,
                                                     T* __restrict__ pC) {
    constexpr int CPL = 4;   // columns per lane per pass
    // the keys and source rows of positions [lo, lo + 2 kRowD) (a block starting in this range
    // reaches at most kRowD positions past it), and per block its first position and its
    // destination's bounds, all fetched up front so a block's only dependent loads are its rows
    __shared__ uint32_t s_K[2 * kRowD];
    __shared__ uint32_t s_R[2 * kRowD];
    __shared__ uint32_t s_item[kRowD + 2];
    __shared__ uint32_t s_seg[kRowD + 2][2];
    __shared__ uint32_t s_nitem;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t m = *nvalid;
    const int64_t lo = (int64_t)blockIdx.x * kRowD;
    if (lo >= m) return;
    const int64_t hi = (lo + kRowD < m) ? lo + kRowD : m;
    if (tid == 0) s_nitem = 0u;
    if (tid < 2 * kRowD && lo + tid < m) {
        s_K[tid] = K[lo + tid];
        s_R[tid] = R[lo + tid];
    }
    __syncthreads();
    if (tid < kRowD) {
        const int64_t p = lo + tid;
        if (p < hi) {
            const uint32_t b = s_K[tid];
            const bool head = p == 0 || (tid > 0 ? s_K[tid - 1] : K[p - 1]) != b;
            if (head || p == lo) {
                const uint32_t s0 = off[b], e0 = off[b + 1];
                if (head) {
                    const uint32_t k = atomicAdd(&s_nitem, 1u);
                    s_item[k] = (uint32_t)p;
                    s_seg[k][0] = s0;
                    s_seg[k][1] = e0;
                } else if ((int64_t)s0 < lo) {
                    // the destination running into the range: its block at the next multiple of
                    // kRowD of its ranks
                    const int64_t pc = s0 + cdiv(lo - s0, kRowD) * kRowD;
                    if (pc < hi && pc < (int64_t)e0) {
                        const uint32_t k = atomicAdd(&s_nitem, 1u);
                        s_item[k] = (uint32_t)pc;
                        s_seg[k][0] = s0;
                        s_seg[k][1] = e0;
                    }
                }
            }
        }
    }
    __syncthreads();
    const int nitem = (int)s_nitem;
    // block it: its first position, length, source rows, and where its value goes (added to
    // the destination row when the destination has at most kRowD members, else a partial)
    auto block = [&](int it, int& len, const uint32_t*& rows, T*& dst, bool& single) {
        const int64_t ps = s_item[it];
        const uint32_t b = s_K[ps - lo];
        const int64_t seg_s = s_seg[it][0], seg_e = s_seg[it][1];
        len = (int)((seg_e - ps) < kRowD ? (seg_e - ps) : kRowD);
        rows = s_R + (ps - lo);   // ps - lo + len <= 2 kRowD
        single = seg_e - seg_s <= kRowD;
        if (single) dst = out + (int64_t)b * d;
        else if (ps == seg_s) dst = pF + (ps / kRowD) * d;
        else dst = pC + (ps / kRowD) * d;
    };
    auto reduce_block = [&](int it) {
        int len;
        const uint32_t* rows;
        T* dst;
        bool single;
        block(it, len, rows, dst, single);
        for (int64_t c0 = 0; c0 < d; c0 += 64 * CPL) {
            // PW over the 64 rank positions of the block (identity past len): 8 groups of 8
            // rows, each a 3-level tree, then a 3-level tree over the group values
            T g8[8][CPL];
#pragma unroll
            for (int gi = 0; gi < 8; ++gi) {
                if (gi * 8 >= len) {
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc) g8[gi][cc] = ident<T>();
                    continue;
                }
                T v[8][CPL];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int q = gi * 8 + r;
                    if (q < len) {
                        const T* row = src + (int64_t)rows[q] * d;
#pragma unroll
                        for (int cc = 0; cc < CPL; ++cc) {
                            const int64_t col = c0 + cc * 64 + lane;
                            v[r][cc] = col < d ? (NEG ? -row[col] : row[col]) : ident<T>();
                        }
                    } else {
#pragma unroll
                        for (int cc = 0; cc < CPL; ++cc) v[r][cc] = ident<T>();
                    }
                }
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc)
                    g8[gi][cc] = ((v[0][cc] + v[1][cc]) + (v[2][cc] + v[3][cc])) +
                                 ((v[4][cc] + v[5][cc]) + (v[6][cc] + v[7][cc]));
            }
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const T r = ((g8[0][cc] + g8[1][cc]) + (g8[2][cc] + g8[3][cc])) +
                            ((g8[4][cc] + g8[5][cc]) + (g8[6][cc] + g8[7][cc]));
                const int64_t col = c0 + cc * 64 + lane;
                if (col < d) dst[col] = single ? dst[col] + r : r;
            }
        }
    };
    int it = wave;
    // two blocks of at most 8 rows each (a few members per destination, the usual case) with
    // the loads of both, and the destination rows they add to, in flight together; a block of
    // at most 8 rows has the value of its first group (the other groups are the identity)
    for (; it + 4 < nitem; it += 8) {
        int la, lb;
        const uint32_t *ra, *rb;
        T *da, *db;
        bool sa, sb;
        block(it, la, ra, da, sa);
        block(it + 4, lb, rb, db, sb);
        if (la > 8 || lb > 8 || d > 64 * CPL) {
            reduce_block(it);
            reduce_block(it + 4);
            continue;
        }
        T va[8][CPL], vb[8][CPL], oa[CPL], ob[CPL];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const T* rowa = src + (int64_t)ra[r < la ? r : 0] * d;
            const T* rowb = src + (int64_t)rb[r < lb ? r : 0] * d;
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const int col = cc * 64 + lane;
                va[r][cc] = (r < la && col < d) ? (NEG ? -rowa[col] : rowa[col]) : ident<T>();
                vb[r][cc] = (r < lb && col < d) ? (NEG ? -rowb[col] : rowb[col]) : ident<T>();
            }
        }
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const int col = cc * 64 + lane;
            oa[cc] = (sa && col < d) ? da[col] : T(0);
            ob[cc] = (sb && col < d) ? db[col] : T(0);
        }
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const int col = cc * 64 + lane;
            const T xa = ((va[0][cc] + va[1][cc]) + (va[2][cc] + va[3][cc])) +
                         ((va[4][cc] + va[5][cc]) + (va[6][cc] + va[7][cc]));
            const T xb = ((vb[0][cc] + vb[1][cc]) + (vb[2][cc] + vb[3][cc])) +
                         ((vb[4][cc] + vb[5][cc]) + (vb[6][cc] + vb[7][cc]));
            if (col < d) {
                da[col] = sa ? oa[cc] + xa : xa;
                db[col] = sb ? ob[cc] + xb : xb;
            }
        }
    }
    if (it < nitem) reduce_block(it);
}

// rows of destinations with more than 64 members: PW over their block rows per column.  A wave
// takes one long destination and 64 columns (one per lane); blockIdx.y walks the column chunks.
// Blocks are read 8 at a time: 8 consecutive blocks starting at a multiple of 8 are an aligned
// subtree, reduced in registers and pushed as one node of a binary counter (levels of 8 blocks
// and up, in LDS); a last, partial group is the same 8-leaf tree with the identity past the end,
// which equals the PW of its blocks, and stands for the counter's three lowest levels.
template <typename T>
__global__ __launch_bounds__(256) void k_segred_rows_long(const uint32_t* __restrict__ off,
                                                          int64_t B, int64_t d,
                                                          const T* __restrict__ pF,
                                                          const T* __restrict__ pC,
                                                          T* __restrict__ out) {
    constexpr int LV = 24;   // counter levels of 8 .. 2^26 blocks (2^32 members)
    __shared__ T s_stk[4][LV][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
    const int64_t nw = (int64_t)gridDim.x * 4;
    // lane l checks destination g + l nw, as in the scalar case
    for (int64_t g = gw; g < B; g += 64 * nw) {
        const int64_t b = g + (int64_t)lane * nw;
        const bool lng = b < B && (int64_t)off[b + 1] - (int64_t)off[b] > kRowD;
        uint64_t mask = __ballot(lng);
        while (mask) {
            const int l = __ffsll((long long)mask) - 1;
            mask &= mask - 1;
            const int64_t bb = g + (int64_t)l * nw;
            const int64_t seg_s = off[bb], seg_e = off[bb + 1];
            const int64_t nblk = cdiv(seg_e - seg_s, kRowD);
            const int64_t r0 = seg_s / kRowD;
            for (int64_t col = (int64_t)blockIdx.y * 64 + lane; col < d;
                 col += 64 * (int64_t)gridDim.y) {
                // block k of the destination: pF[r0] for k = 0, pC[r0 + k] after it
                int64_t s = 0;
                for (; s + 8 <= nblk; s += 8) {
                    T v[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        v[j] = (s + j == 0 ? pF : pC)[(r0 + s + j) * d + col];
                    T t = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
                    int64_t k = s >> 3;
                    int lvl = 0;
                    while (k & 1) {
                        t = s_stk[wave][lvl][lane] + t;
                        k >>= 1;
                        ++lvl;
                    }
                    s_stk[wave][lvl][lane] = t;
                }
                T acc = ident<T>();
                if (s < nblk) {
                    T v[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        v[j] = s + j < nblk ? (s + j == 0 ? pF : pC)[(r0 + s + j) * d + col]
                                            : ident<T>();
                    acc = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
                }
                const int64_t q = nblk >> 3;
                for (int lvl = 0; lvl < LV; ++lvl)
                    if ((q >> lvl) & 1) acc = s_stk[wave][lvl][lane] + acc;
                out[bb * d + col] = out[bb * d + col] + acc;
            }
        }
    }
}

// Launch shape of k_segred_rows_long: one chunk of 64 columns per blockIdx.y, and enough
// waves that a few long destinations each get their own.
inline dim3 rows_long_grid(int64_t B, int64_t d) {
    int64_t gy = cdiv(d, 64);
    if (gy > 64) gy = 64;
    int64_t gx = cdiv(B, 4);
    const int64_t cap = 2048 / gy;
    if (gx > cap) gx = cap;
    return dim3((unsigned)gx, (unsigned)gy);
}


// ---------------------------------------------------------------- running prev

// The destination-grouped members, one column after another: G[c * n + s] = values[src[s] *
// d + c] for sorted positions s < nvalid and +0.0 past them.  A tile of 64 positions x 32
// columns goes through LDS so that both the row reads and the column writes are contiguous.
template <typename T>
__global__ __launch_bounds__(256) void k_group_gather(const T* __restrict__ values,
                                                      const uint32_t* __restrict__ src,
                                                      const uint32_t* __restrict__ nvalid,
                                                      int64_t n, int64_t d, T* __restrict__ G) {
    __shared__ T t[64][33];
    const int tid = threadIdx.x;
    const int64_t s0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 32;
    const int64_t m = *nvalid;
    const int cl = tid & 31;
    for (int r = tid >> 5; r < 64; r += 8) {
        const int64_t sp = s0 + r, c = c0 + cl;
        T v = T(0.0);
        if (sp < m && c < d) v = values[(int64_t)src[sp] * d + c];
        t[r][cl] = v;
    }
    __syncthreads();
    const int sl = tid & 63;
    for (int cc = tid >> 6; cc < 32; cc += 4) {
        const int64_t sp = s0 + sl, c = c0 + cc;
        if (sp < n && c < d) G[c * n + sp] = t[sl][cc];
    }
}

// Scalar destinations (one column): G[s] = values[src[s]] for s < nvalid, +0.0 past them.
template <typename T>
__global__ __launch_bounds__(256) void k_group_gather1(const T* __restrict__ values,
                                                       const uint32_t* __restrict__ src,
                                                       const uint32_t* __restrict__ nvalid,
                                                       int64_t n, T* __restrict__ G) {
    const int64_t m = *nvalid;
    for (int64_t sp = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; sp < n;
         sp += (int64_t)gridDim.x * blockDim.x)
        G[sp] = sp < m ? values[src[sp]] : T(0.0);
}

// The scalar f32 running prev sorts 8-byte payloads, an f32 value's bits above its source
// index, so the grouped values come out of the sort in order instead of through a gather of
// random reads by the sorted indices.
__global__ __launch_bounds__(256) void k_pack_value_index(const uint32_t* __restrict__ vbits,
                                                          int64_t n, uint64_t* __restrict__ pk) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        pk[i] = ((uint64_t)vbits[i] << 32) | (uint64_t)i;
}

// G[s] = the value and src[s] = the source index of sorted position s < nvalid; G = +0.0 past
// them (as k_group_gather1).
__global__ __launch_bounds__(256) void k_unpack_value_index(const uint64_t* __restrict__ SP,
                                                            const uint32_t* __restrict__ nvalid,
                                                            int64_t n, float* __restrict__ G,
                                                            uint32_t* __restrict__ src) {
    const int64_t m = *nvalid;
    for (int64_t sp = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; sp < n;
         sp += (int64_t)gridDim.x * blockDim.x) {
        if (sp < m) {
            const uint64_t v = SP[sp];
            G[sp] = __uint_as_float((uint32_t)(v >> 32));
            src[sp] = (uint32_t)v;
        } else {
            G[sp] = 0.0f;
        }
    }
}

// Scalar destinations: prev[src[s]] = out[r] at r's first position, else out[r] + E[s].
template <typename T>
__global__ __launch_bounds__(256) void k_running_prev1(const uint32_t* __restrict__ K,
                                                       const uint32_t* __restrict__ src,
                                                       const uint32_t* __restrict__ off,
                                                       const uint32_t* __restrict__ nvalid,
                                                       const T* __restrict__ E,
                                                       const T* __restrict__ out,
                                                       T* __restrict__ prev) {
    const int64_t m = *nvalid;
    for (int64_t sp = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; sp < m;
         sp += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t r = K[sp];
        const T init = out[r];
        prev[src[sp]] = off[r] == (uint32_t)sp ? init : init + E[sp];
    }
}

// The packed path's prev values, in sorted order, as (value bits above the source index)
// pairs keyed by the source's window (index >> wbits), so that a radix pass on the key groups
// the writes by window; positions past nvalid get a key past every window.  Windows of 2^wbits
// sources, about 256 of them (one radix pass, and a workgroup per window), at most 2^16.
constexpr int kPrevPart = 32768;   // sources per LDS pass of the window write (128 KB of f32)
inline int prev_window_bits(int64_t n) {
    int bits = 0;
    while (bits < 32 && ((n - 1) >> bits)) ++bits;
    const int w = bits - 8;
    return w < 10 ? 10 : w > 16 ? 16 : w;
}
__global__ __launch_bounds__(256) void k_running_prev1_pairs(const uint32_t* __restrict__ K,
                                                             const uint32_t* __restrict__ src,
                                                             const uint32_t* __restrict__ off,
                                                             const uint32_t* __restrict__ nvalid,
                                                             const float* __restrict__ E,
                                                             const float* __restrict__ out,
                                                             int64_t n, int wbits,
                                                             uint32_t* __restrict__ key2,
                                                             uint64_t* __restrict__ pair2) {
    const int64_t m = *nvalid;
    for (int64_t sp = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; sp < n;
         sp += (int64_t)gridDim.x * blockDim.x) {
        if (sp < m) {
            const uint32_t r = K[sp];
            const float init = out[r];
            const float v = off[r] == (uint32_t)sp ? init : init + E[sp];
            const uint32_t i = src[sp];
            pair2[sp] = ((uint64_t)__float_as_uint(v) << 32) | (uint64_t)i;
            key2[sp] = i >> wbits;
        } else {
            key2[sp] = 0xffffffffu;
        }
    }
}

// prev[i] = v for the (v, i) pairs of window w = blockIdx.x (positions wstart[w] ..
// wstart[w + 1] of the pairs sorted by window), kPrevPart sources at a time: the part's values
// go to a copy in LDS, with a bit per source written, and the part goes out with contiguous
// stores of the written sources (a window of 2^16 sources takes two parts, the second reading
// the window's pairs again, from cache).  Each source has at most one pair, so the order of
// the writes does not matter.
__global__ __launch_bounds__(1024) void k_write_prev_window(const uint64_t* __restrict__ SP,
                                                            const uint32_t* __restrict__ wstart,
                                                            int64_t n, int wbits,
                                                            float* __restrict__ prev) {
    __shared__ float s_v[kPrevPart];
    __shared__ uint32_t s_bits[kPrevPart / 32];
    const int t = threadIdx.x;
    const int64_t w = blockIdx.x;
    const int64_t a = wstart[w], b = wstart[w + 1];
    const uint32_t wmask = (1u << wbits) - 1u;
    const int parts = wbits > 15 ? 1 << (wbits - 15) : 1;
    const int psize = wbits > 15 ? kPrevPart : 1 << wbits;
    for (int part = 0; part < parts; ++part) {
        for (int i = t; i < psize / 32; i += 1024) s_bits[i] = 0u;
        __syncthreads();
        for (int64_t sp = a + t; sp < b; sp += 1024) {
            const uint64_t v = SP[sp];
            const uint32_t i = (uint32_t)v & wmask;
            if ((int)(i / (uint32_t)psize) == part) {
                const uint32_t j = i % (uint32_t)psize;
                s_v[j] = __uint_as_float((uint32_t)(v >> 32));
                atomicOr(&s_bits[j >> 5], 1u << (j & 31u));
            }
        }
        __syncthreads();
        const int64_t base = (w << wbits) + (int64_t)part * psize;
        for (int i = t; i < psize; i += 1024) {
            if (base + i < n && ((s_bits[i >> 5] >> (i & 31)) & 1u)) prev[base + i] = s_v[i];
        }
        __syncthreads();   // the next part reuses the LDS copy
    }
}

// Offsets of the grouped array as the segmented scan takes them: o[b] = off[b] for b <= B
// (destination b's members start at off[b]; off[B] = nvalid) and o[B + 1] = n (the skipped
// sources, one more segment).
__global__ void k_offsets64(const uint32_t* __restrict__ off, int64_t B, int64_t n,
                            int64_t* __restrict__ o) {
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b <= B + 1;
         b += (int64_t)gridDim.x * blockDim.x)
        o[b] = b <= B ? (int64_t)off[b] : n;
}

// prev[src[s] * d + c] = out[r * d + c] at its destination r's first position s = off[r], else
// out[r * d + c] + E[c * n + s] (E: the exclusive segmented scan of the grouped column c).
// Runs before out is updated.  The same 64 x 32 tiling as k_group_gather, the other way round.
template <typename T>
__global__ __launch_bounds__(256) void k_running_prev(const uint32_t* __restrict__ K,
                                                      const uint32_t* __restrict__ src,
                                                      const uint32_t* __restrict__ off,
                                                      const uint32_t* __restrict__ nvalid,
                                                      int64_t n, int64_t d,
                                                      const T* __restrict__ E,
                                                      const T* __restrict__ out,
                                                      T* __restrict__ prev) {
    __shared__ T t[64][33];
    __shared__ uint32_t s_src[64], s_dst[64], s_head[64];
    const int tid = threadIdx.x;
    const int64_t s0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 32;
    const int64_t m = *nvalid;
    if (s0 >= m) return;   // the same for the whole workgroup
    if (tid < 64) {
        const int64_t sp = s0 + tid;
        if (sp < m) {
            const uint32_t r = K[sp];
            s_dst[tid] = r;
            s_src[tid] = src[sp];
            s_head[tid] = (uint32_t)(off[r] == (uint32_t)sp);
        }
    }
    const int sl = tid & 63;
    for (int cc = tid >> 6; cc < 32; cc += 4) {
        const int64_t sp = s0 + sl, c = c0 + cc;
        if (sp < m && c < d) t[sl][cc] = E[c * n + sp];
    }
    __syncthreads();
    const int cl = tid & 31;
    for (int r = tid >> 5; r < 64; r += 8) {
        const int64_t sp = s0 + r, c = c0 + cl;
        if (sp < m && c < d) {
            const T init = out[(int64_t)s_dst[r] * d + c];
            prev[(int64_t)s_src[r] * d + c] = s_head[r] ? init : init + t[r][cl];
        }
    }
}

// ---------------------------------------------------------------- host side

int key_passes(int64_t B) {
    int bits = 0;
    while (bits < 32 && (B - 1) >> bits) ++bits;   // bits of B - 1 (0 for B = 1)
    const int p = (bits + 7) / 8;
    return p < 1 ? 1 : p;
}

struct SLayout {
    int64_t H, nchunks, nhist, nsums, nrange;
    int bytes;    // byte paths for scalar destinations: 2 passes for (256, 65536], 3 passes
                  // for (65536, 2^24]; 0 otherwise
    bool wide;    // f64 into (65536, 2^20] destinations, more than kSmallN keys: two 10-bit passes
    size_t keysA, keysB, payA, payB, cnt, hist, hist2, hist3, off2, sums, ctrl, off, rbin, pF,
        pC, total;
};

// idx_payload: the sort carries source indices (4 bytes) even for scalar destinations
// idx_payload: the sort carries source indices (rows, the running prev); packed: 8-byte
// payloads of an f32 value and its source index (the scalar f32 running prev).
SLayout slayout(int64_t n, int64_t num_out, int64_t row_len, det_dtype dt,
                bool idx_payload = false, bool packed = false) {
    SLayout L;
    const bool rows = row_len > 1;
    const size_t pw = packed ? 8 : (rows || idx_payload) ? 4 : dtype_size(dt);   // payload bytes
    L.H = n <= kSmallN ? kChunkSmall : (pw == 4 ? kChunkBig<uint32_t> : kChunkBig<uint64_t>);
    L.nchunks = cdiv(n > 0 ? n : 1, L.H);
    L.wide = !rows && !idx_payload && dt == DET_F64 && num_out > 65536 &&
             num_out <= ((int64_t)1 << 20) && n > kSmallN;   // chunks of kWideCH = 4096
    const int64_t cols = L.wide ? kWideCols : kBuckets0;
    L.nhist = cols * L.nchunks;
    // column sums (row blocks of 16 up to 4096 rows, else 128) + totals
    L.nsums = cols * cdiv(L.nchunks, L.nchunks <= 4096 ? kRowBlkFew : kRowBlk) +
              (L.wide ? 2048 : 512);
    const int64_t D = rows ? kRowD : kSegD;
    L.nrange = cdiv(n > 0 ? n : 1, D);
    const size_t es = dtype_size(dt);
    const size_t pe = rows ? (size_t)row_len * es : es;   // bytes per partial
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += round_up(bytes > 0 ? bytes : 1, 256);
        return at;
    };
    L.ctrl = take(256);
    L.keysA = take((size_t)n * 4);
    L.keysB = take((size_t)n * 4);
    L.payA = take((size_t)n * pw);
    L.payB = take((size_t)n * pw);
    L.cnt = take((size_t)L.nhist * 2);    // a pass's per-chunk digit counts (16-bit)
    L.hist = take((size_t)L.nhist * 4);   // its bucket offsets
    L.sums = take((size_t)L.nsums * 4);
    L.off = take((size_t)(num_out + 1) * 4);
    const int kp = key_passes(num_out);
    L.bytes = (!rows && !idx_payload && (kp == 2 || kp == 3)) ? kp : 0;
    L.hist2 = take(L.wide ? (size_t)kWideB * L.nchunks * 4
                          : L.bytes ? (size_t)256 * L.nchunks * 4 : 4);
    L.hist3 = take(L.bytes == 3 && !L.wide ? (size_t)256 * L.nchunks * 4 : 4);
    L.off2 = take(L.bytes == 3 && !L.wide ? (size_t)(65536 + 1) * 4 : 4);
    L.rbin = take(L.bytes || L.wide ? (size_t)L.nrange * 4 : 4);
    L.pF = take((size_t)L.nrange * pe);
    L.pC = take((size_t)L.nrange * pe);
    L.total = o;
    return L;
}

// Stable LSD radix sort of (destination, payload) by destination: the first pass takes the
// keys from index and the payloads from pay_in (ROWS: the source index itself), and routes
// out-of-range keys past the valid ones, whose count it leaves in ctrl[0]; later passes sort
// only the valid prefix.  *K and *SP receive the sorted keys (16-bit when k16) and payloads.
template <typename P, bool ROWS>
det_status sort_by_dest(const int32_t* index, const P* pay_in0, int64_t n, int64_t num_out,
                        const SLayout& L, char* ws, bool k16, hipStream_t s, const uint32_t** K,
                        const P** SP) {
    uint32_t* ctrl = reinterpret_cast<uint32_t*>(ws + L.ctrl);
    uint32_t* keys[2] = {reinterpret_cast<uint32_t*>(ws + L.keysA),
                         reinterpret_cast<uint32_t*>(ws + L.keysB)};
    P* pay[2] = {reinterpret_cast<P*>(ws + L.payA), reinterpret_cast<P*>(ws + L.payB)};
    uint16_t* cnt = reinterpret_cast<uint16_t*>(ws + L.cnt);
    uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.hist);
    uint32_t* sums = reinterpret_cast<uint32_t*>(ws + L.sums);
    const uint32_t B = (uint32_t)num_out;
    const int passes = key_passes(num_out);
    const unsigned grid = (unsigned)L.nchunks;
    // test hook: extra dynamic LDS per workgroup lowers the radix kernels' occupancy
    const size_t lds = (size_t)launch_override().extra_lds;
    for (int p = 0; p < passes; ++p) {
        const int shift = 8 * p;
        const bool first = p == 0;
        // with k16 every pass writes 16-bit keys (valid keys fit; the out-of-range ones, placed
        // past the valid ones by the first pass, are never read again)
        const uint32_t* kin = first ? reinterpret_cast<const uint32_t*>(index) : keys[(p - 1) & 1];
        const uint16_t* kin16 = reinterpret_cast<const uint16_t*>(kin);
        const P* pin = first ? pay_in0 : pay[(p - 1) & 1];
        const int nb = first ? kBuckets0 : 256;
        if (first)
            radix_hist<true>(kin, n, ctrl, B, shift, nb, L.nchunks, (int)L.H, cnt, lds, s);
        else if (k16)
            radix_hist<false>(kin16, n, ctrl, B, shift, nb, L.nchunks, (int)L.H, cnt, lds, s);
        else
            radix_hist<false>(kin, n, ctrl, B, shift, nb, L.nchunks, (int)L.H, cnt, lds, s);
        // bucket offsets; the first pass also counts the keys in range into ctrl[0]
        uint32_t* ident = ctrl + 16 + p;   // one word per pass (at most 4 passes)
        det_status st = hist_offsets(cnt, hist, L.nchunks, nb, sums + 512, sums,
                                     first ? ctrl : nullptr, ident, s);
        if (st != DET_SUCCESS) return st;
        KernelTimer kt("k_radix_scatter", s);
        uint32_t* ko = keys[p & 1];
        uint16_t* ko16 = reinterpret_cast<uint16_t*>(ko);
        if (first && k16)
            radix_scatter<P, true, ROWS, uint16_t, uint32_t>(L.H, grid, lds, s,
                kin, pin, ko16, pay[p & 1], n, ctrl, B, shift, L.nchunks, hist, ident);
        else if (first)
            radix_scatter<P, true, ROWS, uint32_t, uint32_t>(L.H, grid, lds, s,
                kin, pin, ko, pay[p & 1], n, ctrl, B, shift, L.nchunks, hist, ident);
        else if (k16)
            radix_scatter<P, false, ROWS, uint16_t, uint16_t>(L.H, grid, lds, s,
                kin16, pin, ko16, pay[p & 1], n, ctrl, B, shift, L.nchunks, hist, ident);
        else
            radix_scatter<P, false, ROWS, uint32_t, uint32_t>(L.H, grid, lds, s,
                kin, pin, ko, pay[p & 1], n, ctrl, B, shift, L.nchunks, hist, ident);
        st = launch_status();
        if (st != DET_SUCCESS) return st;
    }
    *K = keys[(passes - 1) & 1];
    *SP = pay[(passes - 1) & 1];
    return DET_SUCCESS;
}

// The byte paths (scalar destinations): the keys shrink pass by pass.  Two passes for
// (256, 65536]: the first sorts by the low byte and writes only each key's second byte, the
// second sorts by that byte and writes no keys.  Three passes for (65536, 2^24]: the first
// writes bits 8..23 as 16 bits, the second sorts by their low byte and writes the third byte,
// the third sorts by it and writes no keys.  The destination offsets then follow from the
// passes' offsets (k_bin_offsets_bytes, k_bin_offsets_third).  *SP receives the sorted
// payloads.
template <typename P>
det_status sort_by_dest_bytes(const int32_t* index, const P* pay_in0, int64_t n,
                              int64_t num_out, const SLayout& L, char* ws, hipStream_t s,
                              const P** SP) {
    uint32_t* ctrl = reinterpret_cast<uint32_t*>(ws + L.ctrl);
    P* pay[2] = {reinterpret_cast<P*>(ws + L.payA), reinterpret_cast<P*>(ws + L.payB)};
    uint16_t* cnt = reinterpret_cast<uint16_t*>(ws + L.cnt);
    uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.hist);
    uint32_t* hist2 = reinterpret_cast<uint32_t*>(ws + L.hist2);
    uint32_t* hist3 = reinterpret_cast<uint32_t*>(ws + L.hist3);
    uint32_t* sums = reinterpret_cast<uint32_t*>(ws + L.sums);
    const uint32_t* kin = reinterpret_cast<const uint32_t*>(index);
    const uint32_t B = (uint32_t)num_out;
    const unsigned grid = (unsigned)L.nchunks;
    const size_t lds = (size_t)launch_override().extra_lds;
    const int nc = (int)L.H;
    // each pass counts into cnt, and its offsets go to h
    auto hist_of = [&](uint32_t* h, int nb, uint32_t* ident, bool first) {
        return hist_offsets(cnt, h, L.nchunks, nb, sums + 512, sums, first ? ctrl : nullptr, ident,
                            s);
    };
    // pass 1: the low byte (and the out-of-range bucket)
    radix_hist<true>(kin, n, ctrl, B, 0, kBuckets0, L.nchunks, nc, cnt, lds, s);
    det_status st = hist_of(hist, kBuckets0, ctrl + 16, true);
    if (st != DET_SUCCESS) return st;
    if (L.bytes == 2) {
        uint8_t* kb = reinterpret_cast<uint8_t*>(ws + L.keysA);
        {
            KernelTimer kt("k_radix_scatter", s);
            radix_scatter<P, true, false, KeyHi8, uint32_t>(L.H, grid, lds, s,
                kin, pay_in0, reinterpret_cast<KeyHi8*>(kb), pay[0], n, ctrl, B, 0, L.nchunks,
                hist, ctrl + 16);
        }
        if ((st = launch_status()) != DET_SUCCESS) return st;
        radix_hist<false>(kb, n, ctrl, B, 0, 256, L.nchunks, nc, cnt, lds, s);
        if ((st = hist_of(hist2, 256, ctrl + 17, false)) != DET_SUCCESS) return st;
        {
            KernelTimer kt("k_radix_scatter", s);
            radix_scatter<P, false, false, NoKey, uint8_t>(L.H, grid, lds, s,
                kb, pay[0], static_cast<NoKey*>(nullptr), pay[1], n, ctrl, B, 0, L.nchunks,
                hist2, ctrl + 17);
        }
        if ((st = launch_status()) != DET_SUCCESS) return st;
        *SP = pay[1];
        return DET_SUCCESS;
    }
    uint16_t* k16 = reinterpret_cast<uint16_t*>(ws + L.keysA);
    uint8_t* kb = reinterpret_cast<uint8_t*>(ws + L.keysB);
    {
        KernelTimer kt("k_radix_scatter", s);
        radix_scatter<P, true, false, KeyHi16, uint32_t>(L.H, grid, lds, s,
            kin, pay_in0, reinterpret_cast<KeyHi16*>(k16), pay[0], n, ctrl, B, 0, L.nchunks,
            hist, ctrl + 16);
    }
    if ((st = launch_status()) != DET_SUCCESS) return st;
    // pass 2: the second byte, the low byte of the 16-bit keys
    radix_hist<false>(k16, n, ctrl, B, 0, 256, L.nchunks, nc, cnt, lds, s);
    if ((st = hist_of(hist2, 256, ctrl + 17, false)) != DET_SUCCESS) return st;
    {
        KernelTimer kt("k_radix_scatter", s);
        radix_scatter<P, false, false, KeyHi8, uint16_t>(L.H, grid, lds, s,
            k16, pay[0], reinterpret_cast<KeyHi8*>(kb), pay[1], n, ctrl, B, 0, L.nchunks, hist2,
            ctrl + 17);
    }
    if ((st = launch_status()) != DET_SUCCESS) return st;
    // pass 3: the third byte
    radix_hist<false>(kb, n, ctrl, B, 0, 256, L.nchunks, nc, cnt, lds, s);
    if ((st = hist_of(hist3, 256, ctrl + 18, false)) != DET_SUCCESS) return st;
    {
        KernelTimer kt("k_radix_scatter", s);
        radix_scatter<P, false, false, NoKey, uint8_t>(L.H, grid, lds, s,
            kb, pay[1], static_cast<NoKey*>(nullptr), pay[0], n, ctrl, B, 0, L.nchunks, hist3,
            ctrl + 18);
    }
    if ((st = launch_status()) != DET_SUCCESS) return st;
    *SP = pay[0];
    return DET_SUCCESS;
}

// The 10-bit path (L.wide): two passes over chunks of 4096, the first on the low 10 bits
// writing the high 10 as 16-bit keys (keysA), the second on those writing no key.  *SP
// receives the sorted payloads.
static_assert(kChunkBig<uint64_t> == kWideCH, "the 10-bit passes take the f64 chunk size");
det_status sort_by_dest_w(const int32_t* index, const uint64_t* pay_in0, int64_t n,
                          int64_t num_out, const SLayout& L, char* ws, hipStream_t s,
                          const uint64_t** SP) {
    uint32_t* ctrl = reinterpret_cast<uint32_t*>(ws + L.ctrl);
    uint64_t* pay[2] = {reinterpret_cast<uint64_t*>(ws + L.payA),
                        reinterpret_cast<uint64_t*>(ws + L.payB)};
    uint16_t* cnt = reinterpret_cast<uint16_t*>(ws + L.cnt);
    uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.hist);
    uint32_t* hist2 = reinterpret_cast<uint32_t*>(ws + L.hist2);
    uint32_t* sums = reinterpret_cast<uint32_t*>(ws + L.sums);
    uint16_t* k16 = reinterpret_cast<uint16_t*>(ws + L.keysA);
    const uint32_t* kin = reinterpret_cast<const uint32_t*>(index);
    const uint32_t B = (uint32_t)num_out;
    const unsigned grid = (unsigned)L.nchunks;
    const unsigned hgrid = (unsigned)cdiv(L.nchunks, 4);
    const size_t lds = (size_t)launch_override().extra_lds;
    const int H = (int)L.H;
    det_status st;
    {
        KernelTimer kt("k_radix_hist", s);
        k_radix_hist_w<true, uint32_t><<<hgrid, 256, lds, s>>>(kin, n, ctrl, B, kWideCols,
                                                                L.nchunks, H, cnt);
    }
    if ((st = hist_offsets_w(cnt, hist, L.nchunks, kWideCols, sums + 2048, sums, ctrl, ctrl + 16,
                             s)) != DET_SUCCESS)
        return st;
    {
        KernelTimer kt("k_radix_scatter", s);
        k_radix_scatter_w<true, KeyW16, uint32_t><<<grid, 256, lds, s>>>(
            kin, pay_in0, reinterpret_cast<KeyW16*>(k16), pay[0], n, ctrl, B, L.nchunks, hist,
            ctrl + 16);
    }
    if ((st = launch_status()) != DET_SUCCESS) return st;
    {
        KernelTimer kt("k_radix_hist", s);
        k_radix_hist_w<false, uint16_t><<<hgrid, 256, lds, s>>>(k16, n, ctrl, B, kWideB,
                                                                 L.nchunks, H, cnt);
    }
    if ((st = hist_offsets_w(cnt, hist2, L.nchunks, kWideB, sums + 2048, sums, nullptr,
                             ctrl + 17, s)) != DET_SUCCESS)
        return st;
    {
        KernelTimer kt("k_radix_scatter", s);
        k_radix_scatter_w<false, NoKey, uint16_t><<<grid, 256, lds, s>>>(
            k16, pay[0], static_cast<NoKey*>(nullptr), pay[1], n, ctrl, B, L.nchunks, hist2,
            ctrl + 17);
    }
    if ((st = launch_status()) != DET_SUCCESS) return st;
    *SP = pay[1];
    return DET_SUCCESS;
}

template <typename T, typename P, bool ROWS>
det_status scatter_impl(const T* values, const int32_t* index, int64_t n, int64_t row_len, T* out,
                        int64_t num_out, T* prev, int64_t* n_skipped, char* ws, bool neg,
                        hipStream_t s) {
    const SLayout L = slayout(n, num_out, row_len, sizeof(T) == 8 ? DET_F64 : DET_F32);
    if (n == 0) {
        if (n_skipped) {
            k_write_skipped_all<T><<<1, 1, 0, s>>>(n_skipped, 0);
            return launch_status();
        }
        return DET_SUCCESS;
    }
    if (prev) {
        const int64_t total = n * row_len;
        int64_t g = cdiv(total, 256);
        if (g > 65536) g = 65536;
        k_prev_gather<T><<<dim3((unsigned)g), dim3(256), 0, s>>>(index, n, row_len, num_out, out, prev);
    }
    if (num_out == 0) {
        if (n_skipped) k_write_skipped_all<T><<<1, 1, 0, s>>>(n_skipped, n);
        return launch_status();
    }
    uint32_t* ctrl = reinterpret_cast<uint32_t*>(ws + L.ctrl);   // [0] = number of valid keys
    uint32_t* off = reinterpret_cast<uint32_t*>(ws + L.off);
    if constexpr (!ROWS) {
        if (L.bytes || L.wide) {
            // byte keys (or 10-bit digits), offsets from the histograms, no key reads after the
            // sort
            const P* SP = nullptr;
            det_status st;
            if constexpr (std::is_same_v<P, uint64_t>) {
                if (L.wide)
                    st = sort_by_dest_w(index, reinterpret_cast<const uint64_t*>(values), n,
                                        num_out, L, ws, s, &SP);
                else
                    st = sort_by_dest_bytes<P>(index, reinterpret_cast<const P*>(values), n,
                                               num_out, L, ws, s, &SP);
            } else {
                st = sort_by_dest_bytes<P>(index, reinterpret_cast<const P*>(values), n, num_out,
                                           L, ws, s, &SP);
            }
            if (st != DET_SUCCESS) return st;
            uint32_t* rbin = reinterpret_cast<uint32_t*>(ws + L.rbin);
            const uint32_t* h1 = reinterpret_cast<const uint32_t*>(ws + L.hist);
            const uint32_t* h2 = reinterpret_cast<const uint32_t*>(ws + L.hist2);
            {
                KernelTimer kt("k_bin_offsets", s);
                if (L.wide) {
                    k_bin_offsets_w<<<kWideB, 256, 0, s>>>(
                        h1, h2, reinterpret_cast<const uint16_t*>(ws + L.keysA), ctrl, num_out, n,
                        L.H, off, n_skipped);
                } else if (L.bytes == 2) {
                    k_bin_offsets_bytes<uint8_t><<<256, 256, 0, s>>>(
                        h1, h2, reinterpret_cast<const uint8_t*>(ws + L.keysA), ctrl, num_out, n,
                        L.H, off, n_skipped);
                } else {
                    uint32_t* off2 = reinterpret_cast<uint32_t*>(ws + L.off2);
                    k_bin_offsets_bytes<uint16_t><<<256, 256, 0, s>>>(
                        h1, h2, reinterpret_cast<const uint16_t*>(ws + L.keysA), ctrl, 65536, n,
                        L.H, off2, nullptr);
                    k_bin_offsets_third<<<65536 / 4, 256, 0, s>>>(
                        off2, reinterpret_cast<const uint32_t*>(ws + L.hist3),
                        reinterpret_cast<const uint8_t*>(ws + L.keysB), ctrl, num_out, n, L.H,
                        off, n_skipped);
                }
                k_range_bins<<<dim3((unsigned)cdiv(L.nrange, 4)), dim3(256), 0, s>>>(
                    off, num_out, L.nrange, rbin);
            }
            T* pF = reinterpret_cast<T*>(ws + L.pF);
            T* pC = reinterpret_cast<T*>(ws + L.pC);
            const T* SV = reinterpret_cast<const T*>(SP);
            {
                KernelTimer kt("k_segred_scalar", s);
                // destinations per range (on average) in groups of 256, one workgroup each, at
                // most 32 per range
                int64_t split = cdiv(cdiv(num_out * kSegD, n), 256);
                if (split > 32) split = 32;
                const dim3 g((unsigned)L.nrange, (unsigned)split), b(256);
                if (!neg)
                    k_segred_off<T, false><<<g, b, 0, s>>>(SV, off, num_out, rbin, ctrl, out, pF,
                                                           pC);
                else
                    k_segred_off<T, true><<<g, b, 0, s>>>(SV, off, num_out, rbin, ctrl, out, pF,
                                                          pC);
            }
            int64_t lg = cdiv(num_out, 64 * 4);
            if (lg > 4096) lg = 4096;
            k_segred_scalar_long<T><<<dim3((unsigned)lg), dim3(256), 0, s>>>(off, num_out, pF, pC,
                                                                              out);
            return launch_status();
        }
    }
    // scalar destinations that all fit 16 bits: every pass writes 16-bit keys, which the next
    // pass, the destination offsets and the reduction read (out-of-range keys land past the
    // valid ones and are never read)
    const bool k16 = !ROWS && num_out <= 65536;
    const uint32_t* K = nullptr;
    const P* SP = nullptr;
    det_status st = sort_by_dest<P, ROWS>(index, reinterpret_cast<const P*>(values), n, num_out,
                                          L, ws, k16, s, &K, &SP);
    if (st != DET_SUCCESS) return st;
    const uint16_t* K16 = reinterpret_cast<const uint16_t*>(K);
    {
        int64_t g = cdiv(num_out + 1, 256);
        if (g > 8192) g = 8192;
        KernelTimer kt("k_bin_offsets", s);
        // the last pass's bucket starts: row 0 of its offsets, still in the histogram buffer
        const uint32_t* row0 = reinterpret_cast<const uint32_t*>(ws + L.hist);
        const int passes = key_passes(num_out);
        if (k16)
            k_bin_offsets<uint16_t><<<dim3((unsigned)g), dim3(256), 0, s>>>(
                K16, ctrl, num_out, n, off, n_skipped, row0, passes);
        else
            k_bin_offsets<uint32_t><<<dim3((unsigned)g), dim3(256), 0, s>>>(
                K, ctrl, num_out, n, off, n_skipped, row0, passes);
    }
    T* pF = reinterpret_cast<T*>(ws + L.pF);
    T* pC = reinterpret_cast<T*>(ws + L.pC);
    int64_t lg = cdiv(num_out, 64 * 4);
    if (lg > 4096) lg = 4096;
    if constexpr (!ROWS) {
        {
            KernelTimer kt("k_segred_scalar", s);
            const dim3 g((unsigned)L.nrange), b(256);
            const T* SV = reinterpret_cast<const T*>(SP);
            if (k16 && !neg)
                k_segred_scalar<T, uint16_t, false><<<g, b, 0, s>>>(K16, SV, off, ctrl, out, pF, pC);
            else if (k16)
                k_segred_scalar<T, uint16_t, true><<<g, b, 0, s>>>(K16, SV, off, ctrl, out, pF, pC);
            else if (!neg)
                k_segred_scalar<T, uint32_t, false><<<g, b, 0, s>>>(K, SV, off, ctrl, out, pF, pC);
            else
                k_segred_scalar<T, uint32_t, true><<<g, b, 0, s>>>(K, SV, off, ctrl, out, pF, pC);
        }
        k_segred_scalar_long<T><<<dim3((unsigned)lg), dim3(256), 0, s>>>(off, num_out, pF, pC, out);
    } else {
        {
            KernelTimer kt("k_segred_rows", s);
            const uint32_t* SR = reinterpret_cast<const uint32_t*>(SP);
            if (!neg)
                k_segred_rows<T, false><<<dim3((unsigned)L.nrange), dim3(256), 0, s>>>(
                    K, SR, off, ctrl, values, row_len, out, pF, pC);
            else
                k_segred_rows<T, true><<<dim3((unsigned)L.nrange), dim3(256), 0, s>>>(
                    K, SR, off, ctrl, values, row_len, out, pF, pC);
        }
        KernelTimer kt("k_segred_rows_long", s);
        k_segred_rows_long<T><<<rows_long_grid(num_out, row_len), dim3(256), 0, s>>>(
            off, num_out, row_len, pF, pC, out);
    }
    return launch_status();
}


// Scatter-add with the running prev: the sort carries source indices; the grouped members are
// gathered column by column, each column scanned (exclusive, forward, one segment per
// destination and one for the skipped sources), prev written from the scan and the initial
// values, and then out reduced exactly as det_scatter_add reduces it.
struct RLayout {
    SLayout S;
    size_t o64, G, E, sws, cagg, key2, pair2, wstart, total;
};

// The scalar f32 running prev above 2^21 members sorts 8-byte payloads (value and source index)
// instead of gathering the values through the sorted indices (MI355X, f32 into 65,536 bins:
// 2^24 members 1.04 -> 0.90 ms; 2^22 into 2^20 bins 0.41 -> 0.38 ms; 2^20 members 111 ->
// 117 us, the packing launch not paid back).
inline bool running_packed(int64_t n, int64_t row_len, det_dtype dt) {
    return row_len == 1 && dt == DET_F32 && n > ((int64_t)1 << 21);
}

RLayout rlayout(int64_t n, int64_t num_out, int64_t row_len, det_dtype dt) {
    RLayout R;
    R.S = slayout(n, num_out, row_len, dt, true, running_packed(n, row_len, dt));
    size_t o = R.S.total;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += round_up(bytes > 0 ? bytes : 1, 256);
        return at;
    };
    const size_t cells = (size_t)n * (size_t)row_len * dtype_size(dt);
    R.o64 = take((size_t)(num_out + 2) * 8);
    R.G = take(cells);
    R.E = take(cells);
    R.sws = take(scan_workspace(n > 0 ? n : 1, dt, DET_SCAN_EXCLUSIVE, num_out + 1));
    R.cagg = take(scan_columns_agg_bytes(n > 0 ? n : 1, row_len));
    // the packed path's (value, source) pairs and their window keys, for the bucketed write
    const bool pk = running_packed(n, row_len, dt);
    R.key2 = take(pk ? (size_t)n * 4 : 4);
    R.pair2 = take(pk ? (size_t)n * 8 : 8);
    R.wstart = take(pk ? (size_t)(cdiv(n, (int64_t)1 << prev_window_bits(n)) + 1) * 4 : 4);
    R.total = o;
    return R;
}

template <typename T>
det_status scatter_running_impl(const T* values, const int32_t* index, int64_t n, int64_t row_len,
                                T* out, int64_t num_out, T* prev, int64_t* n_skipped, char* ws,
                                hipStream_t s) {
    const det_dtype dt = sizeof(T) == 8 ? DET_F64 : DET_F32;
    const RLayout R = rlayout(n, num_out, row_len, dt);
    const SLayout& L = R.S;
    if (n == 0 || num_out == 0) {
        if (n_skipped) k_write_skipped_all<T><<<1, 1, 0, s>>>(n_skipped, num_out == 0 ? n : 0);
        return launch_status();
    }
    uint32_t* ctrl = reinterpret_cast<uint32_t*>(ws + L.ctrl);
    uint32_t* off = reinterpret_cast<uint32_t*>(ws + L.off);
    const uint32_t* K = nullptr;
    const uint32_t* SRC = nullptr;
    T* G = reinterpret_cast<T*>(ws + R.G);
    T* E = reinterpret_cast<T*>(ws + R.E);
    int64_t g1 = cdiv(n, 256);
    if (g1 > 16384) g1 = 16384;
    // value and source index travel through the sort together (scalar f32, large n)
    const bool packed = running_packed(n, row_len, dt);
    det_status st;
    if (packed) {
        // the packed input lives in G's and E's space (8 bytes per member, free until the
        // sort's first pass has read it)
        uint64_t* pk = reinterpret_cast<uint64_t*>(ws + R.G);
        k_pack_value_index<<<dim3((unsigned)g1), dim3(256), 0, s>>>(
            reinterpret_cast<const uint32_t*>(values), n, pk);
        const uint64_t* SP = nullptr;
        st = sort_by_dest<uint64_t, false>(index, pk, n, num_out, L, ws, false, s, &K, &SP);
        if (st != DET_SUCCESS) return st;
        // the source indices into the payload buffer the sort did not end in
        uint32_t* src = reinterpret_cast<uint32_t*>(
            reinterpret_cast<const char*>(SP) == ws + L.payA ? ws + L.payB : ws + L.payA);
        KernelTimer kt("k_unpack_value_index", s);
        k_unpack_value_index<<<dim3((unsigned)g1), dim3(256), 0, s>>>(
            SP, ctrl, n, reinterpret_cast<float*>(G), src);
        SRC = src;
    } else {
        st = sort_by_dest<uint32_t, true>(index, nullptr, n, num_out, L, ws, false, s, &K, &SRC);
    }
    if (st != DET_SUCCESS) return st;
    {
        int64_t g = cdiv(num_out + 1, 256);
        if (g > 8192) g = 8192;
        KernelTimer kt("k_bin_offsets", s);
        // the last pass's bucket starts (row 0 of its offsets) narrow each search
        k_bin_offsets<uint32_t><<<dim3((unsigned)g), dim3(256), 0, s>>>(
            K, ctrl, num_out, n, off, n_skipped, reinterpret_cast<const uint32_t*>(ws + L.hist),
            key_passes(num_out));
    }
    int64_t* o64 = reinterpret_cast<int64_t*>(ws + R.o64);
    {
        int64_t g = cdiv(num_out + 2, 256);
        if (g > 4096) g = 4096;
        k_offsets64<<<dim3((unsigned)g), dim3(256), 0, s>>>(off, num_out, n, o64);
    }
    const dim3 tg((unsigned)cdiv(n, 64), (unsigned)cdiv(row_len, 32));
    if (!packed) {
        KernelTimer kt("k_group_gather", s);
        if (row_len == 1)
            k_group_gather1<T><<<dim3((unsigned)g1), dim3(256), 0, s>>>(values, SRC, ctrl, n, G);
        else
            k_group_gather<T><<<tg, dim3(256), 0, s>>>(values, SRC, ctrl, n, row_len, G);
    }
    st = launch_status();
    if (st != DET_SUCCESS) return st;
    const size_t sbytes = scan_workspace(n, dt, DET_SCAN_EXCLUSIVE, num_out + 1);
    (void)sbytes;
    st = scan_columns_launch(G, E, n, row_len, dt, DET_SCAN_EXCLUSIVE, o64, num_out + 1,
                             ws + R.sws, ws + R.cagg, s);
    if (st != DET_SUCCESS) return st;
    {
        KernelTimer kt("k_running_prev", s);
        if (packed)
            k_running_prev1_pairs<<<dim3((unsigned)g1), dim3(256), 0, s>>>(
                K, SRC, off, ctrl, reinterpret_cast<const float*>(E),
                reinterpret_cast<const float*>(out), n, prev_window_bits(n),
                reinterpret_cast<uint32_t*>(ws + R.key2), reinterpret_cast<uint64_t*>(ws + R.pair2));
        else if (row_len == 1)
            k_running_prev1<T><<<dim3((unsigned)g1), dim3(256), 0, s>>>(K, SRC, off, ctrl, E, out,
                                                                        prev);
        else
            k_running_prev<T><<<tg, dim3(256), 0, s>>>(K, SRC, off, ctrl, n, row_len, E, out,
                                                       prev);
    }
    st = launch_status();
    if (st != DET_SUCCESS) return st;
    T* pF = reinterpret_cast<T*>(ws + L.pF);
    T* pC = reinterpret_cast<T*>(ws + L.pC);
    if (row_len == 1) {
        {
            KernelTimer kt("k_segred_scalar", s);
            k_segred_scalar<T, uint32_t, false><<<dim3((unsigned)L.nrange), dim3(256), 0, s>>>(
                K, G, off, ctrl, out, pF, pC);
        }
        int64_t lg = cdiv(num_out, 64 * 4);
        if (lg > 4096) lg = 4096;
        k_segred_scalar_long<T><<<dim3((unsigned)lg), dim3(256), 0, s>>>(off, num_out, pF, pC, out);
        if (packed) {
            // the prev writes grouped by window: one radix pass on the window keys (the sort's
            // buffers are free once the reduction has read them), then the writes
            const uint32_t* K2 = nullptr;
            const uint64_t* SP2 = nullptr;
            const int wbits = prev_window_bits(n);
            const int64_t nwin = cdiv(n, (int64_t)1 << wbits);
            st = sort_by_dest<uint64_t, false>(
                reinterpret_cast<const int32_t*>(ws + R.key2),
                reinterpret_cast<const uint64_t*>(ws + R.pair2), n, nwin, L, ws, false, s, &K2,
                &SP2);
            if (st != DET_SUCCESS) return st;
            // each window's first position among the sorted pairs (the pass's bucket starts,
            // row 0 of its offsets, narrow the search), then a workgroup per window
            uint32_t* wstart = reinterpret_cast<uint32_t*>(ws + R.wstart);
            k_bin_offsets<uint32_t><<<dim3((unsigned)cdiv(nwin + 1, 256)), dim3(256), 0, s>>>(
                K2, ctrl, nwin, n, wstart, nullptr,
                reinterpret_cast<const uint32_t*>(ws + L.hist), key_passes(nwin));
            KernelTimer kt("k_write_prev_window", s);
            k_write_prev_window<<<dim3((unsigned)nwin), dim3(1024), 0, s>>>(
                SP2, wstart, n, wbits, reinterpret_cast<float*>(prev));
        }
    } else {
        {
            KernelTimer kt("k_segred_rows", s);
            k_segred_rows<T, false><<<dim3((unsigned)L.nrange), dim3(256), 0, s>>>(
                K, SRC, off, ctrl, values, row_len, out, pF, pC);
        }
        KernelTimer kt("k_segred_rows_long", s);
        k_segred_rows_long<T><<<rows_long_grid(num_out, row_len), dim3(256), 0, s>>>(
            off, num_out, row_len, pF, pC, out);
    }
    return launch_status();
}
}  // namespace

size_t scatter_workspace(int64_t n, int64_t num_out, int64_t row_len, det_dtype dt) {
    return slayout(n, num_out, row_len, dt).total;
}

det_status scatter_launch(const void* values, const int32_t* index, int64_t n, int64_t row_len,
                          det_dtype dt, void* out, int64_t num_out, void* prev, int64_t* n_skipped,
                          void* ws, size_t ws_bytes, bool negate, hipStream_t s) {
    (void)ws_bytes;
    char* w = static_cast<char*>(ws);
    if (dt == DET_F32) {
        const float* v = static_cast<const float*>(values);
        float* o = static_cast<float*>(out);
        float* pr = static_cast<float*>(prev);
        if (row_len == 1)
            return scatter_impl<float, uint32_t, false>(v, index, n, 1, o, num_out, pr, n_skipped, w, negate, s);
        return scatter_impl<float, uint32_t, true>(v, index, n, row_len, o, num_out, pr, n_skipped, w, negate, s);
    }
    const double* v = static_cast<const double*>(values);
    double* o = static_cast<double*>(out);
    double* pr = static_cast<double*>(prev);
    if (row_len == 1)
        return scatter_impl<double, uint64_t, false>(v, index, n, 1, o, num_out, pr, n_skipped, w, negate, s);
    return scatter_impl<double, uint32_t, true>(v, index, n, row_len, o, num_out, pr, n_skipped, w, negate, s);
}

}  // namespace det

namespace det {

size_t scatter_running_workspace(int64_t n, int64_t num_out, int64_t row_len, det_dtype dt) {
    return rlayout(n, num_out, row_len, dt).total;
}

det_status scatter_running_launch(const void* values, const int32_t* index, int64_t n,
                                  int64_t row_len, det_dtype dt, void* out, int64_t num_out,
                                  void* prev, int64_t* n_skipped, void* ws, hipStream_t s) {
    char* w = static_cast<char*>(ws);
    if (dt == DET_F32)
        return scatter_running_impl<float>(static_cast<const float*>(values), index, n, row_len,
                                           static_cast<float*>(out), num_out,
                                           static_cast<float*>(prev), n_skipped, w, s);
    return scatter_running_impl<double>(static_cast<const double*>(values), index, n, row_len,
                                        static_cast<double*>(out), num_out,
                                        static_cast<double*>(prev), n_skipped, w, s);
}

}  // namespace det
