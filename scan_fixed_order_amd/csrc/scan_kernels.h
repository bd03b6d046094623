// scan_kernels.h -- the device side of det_scan: status slots, tile loads, the local step,
// the look-back through fixed anchors, the readout, and the kernels built from them.  The host
// side (workspace layout, launches) is scan.hip.  See scan.hip for the order these compute.
#pragma once

#include <type_traits>

#include "det_device.h"
#include "det_internal.h"

namespace det {
namespace {

constexpr int kV = kScanV;
constexpr int kT = kScanT;

constexpr int kWaveElems = kScanV * kScanW;                 // 2048
constexpr int kHeadWords = kT / 32 + 1;                     // bits for positions [F0, F0 + T]

constexpr uint32_t kReady = 1u;
constexpr uint32_t kHeadTag = 2u;

__device__ __forceinline__ int pad(int e) { return e + (e >> 5); }

template <typename T>
struct Seg {
    T v;
    uint32_t f;
};

template <bool SEG, typename T>
__device__ __forceinline__ Seg<T> op(const Seg<T>& a, const Seg<T>& b) {
    if constexpr (SEG) {
        return Seg<T>{b.f ? b.v : a.v + b.v, a.f | b.f};
    } else {
        return Seg<T>{a.v + b.v, 0u};
    }
}

template <typename T>
__device__ __forceinline__ Seg<T> seg_ident() {
    return Seg<T>{ident<T>(), 0u};
}

// ---------------------------------------------------------------- status slots

template <typename T>
constexpr int slot_words() {
    return sizeof(T) == 4 ? 1 : 2;
}

// 32-bit payload bits of a 4-byte element (f32, or the int32 scan's uint32_t)
template <typename T>
__device__ __forceinline__ uint32_t to_bits32(T v) {
    if constexpr (__is_same(T, float)) return __float_as_uint(v);
    else return (uint32_t)v;
}
template <typename T>
__device__ __forceinline__ T from_bits32(uint32_t u) {
    if constexpr (__is_same(T, float)) return __uint_as_float(u);
    else return (T)u;
}

template <typename T>
__device__ __forceinline__ void publish(uint64_t* slot, const Seg<T>& s) {
    const uint64_t tag = (uint64_t)(kReady | (s.f ? kHeadTag : 0u)) << 32;
    if constexpr (sizeof(T) == 4) {
        __hip_atomic_store(slot, tag | to_bits32<T>(s.v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
        const uint64_t b = (uint64_t)__double_as_longlong(s.v);
        __hip_atomic_store(slot, tag | (b & 0xffffffffull), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(slot + 1, tag | (b >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Wait bound: a predecessor's slot is normally ready within microseconds.  A wait that has
// polled for more than kWaitTicks of the GPU's constant 100 MHz clock (2 seconds) gives up and
// raises the error word, so no wave can wait forever; the scan's result is then unspecified.
constexpr uint64_t kWaitTicks = 200000000ull;

// Called once per unsuccessful poll; true once the wait has lasted past the bound.  The clock
// is read on the first poll and then every 256th.
__device__ __forceinline__ bool wait_expired(uint32_t& polls, uint64_t& t0) {
    if ((polls++ & 255u) != 0u) return false;
    const uint64_t now = __builtin_amdgcn_s_memrealtime();
    if (polls == 1u) {
        t0 = now;
        return false;
    }
    return now - t0 > kWaitTicks;
}

__device__ __forceinline__ uint64_t wait_word(uint64_t* w, uint32_t* err) {
    uint64_t v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t polls = 0;
    uint64_t t0 = 0;
    while (!((v >> 32) & kReady)) {
        if (wait_expired(polls, t0)) {
            __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return v;
}

template <typename T>
__device__ __forceinline__ Seg<T> unpack(uint64_t w0, uint64_t w1) {
    if constexpr (sizeof(T) == 4) {
        return Seg<T>{from_bits32<T>((uint32_t)w0), (uint32_t)(w0 >> 33) & 1u};
    } else {
        const uint64_t b = (w1 << 32) | (w0 & 0xffffffffull);
        return Seg<T>{__longlong_as_double((long long)b), (uint32_t)(w0 >> 33) & 1u};
    }
}

template <typename T>
__device__ __forceinline__ Seg<T> wait_slot(uint64_t* slot, uint32_t* err) {
    if constexpr (sizeof(T) == 4) {
        const uint64_t w = wait_word(slot, err);
        return Seg<T>{from_bits32<T>((uint32_t)w), (uint32_t)(w >> 33) & 1u};
    } else {
        const uint64_t w0 = wait_word(slot, err);
        const uint64_t w1 = wait_word(slot + 1, err);
        const uint64_t b = (w1 << 32) | (w0 & 0xffffffffull);
        return Seg<T>{__longlong_as_double((long long)b), (uint32_t)(w0 >> 33) & 1u};
    }
}

// Status polls in two halves, so the first round trip can overlap other memory traffic:
// poll_issue loads up to two slots (unused ones read as ready), poll_finish_set re-polls the
// words of one slot that were not ready yet (bounded) and unpacks the value.
template <typename T>
struct Poll {
    uint64_t w[2 * slot_words<T>()];
};

template <typename T>
__device__ __forceinline__ void poll_issue(Poll<T>& pl, const uint64_t* s1, bool use1,
                                           const uint64_t* s2, bool use2) {
    constexpr int SW = slot_words<T>();
    constexpr uint64_t kDone = (uint64_t)kReady << 32;
#pragma unroll
    for (int i = 0; i < SW; ++i) {
        pl.w[i] = use1 ? __hip_atomic_load(s1 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : kDone;
        pl.w[SW + i] = use2 ? __hip_atomic_load(s2 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                            : kDone;
    }
}

__device__ __forceinline__ void repoll(uint64_t& w, const uint64_t* slot) {
    if (!((w >> 32) & kReady)) w = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until one slot set of a Poll (words w[0 .. SW)) is ready, re-polling only that set, and
// unpacks it (the identity when unused).  Lets a tile finish the waits it needs first.
template <typename T>
__device__ __forceinline__ Seg<T> poll_finish_set(uint64_t* w, const uint64_t* slot, bool use,
                                                  uint32_t* err) {
    constexpr int SW = slot_words<T>();
    uint32_t polls = 0;
    uint64_t t0 = 0;
    for (;;) {
        bool all = (w[0] >> 32) & kReady;
        if constexpr (SW == 2) all = all && ((w[1] >> 32) & kReady);
        if (all) break;
        if (wait_expired(polls, t0)) {
            __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        repoll(w[0], slot);
        if constexpr (SW == 2) repoll(w[1], slot + 1);
    }
    return use ? unpack<T>(w[0], SW == 2 ? w[1] : 0ull) : seg_ident<T>();
}

// ---------------------------------------------------------------- cross-lane pieces

template <int M, bool SEG, typename T>
__device__ __forceinline__ Seg<T> bfly(const Seg<T>& v, int lane) {
    Seg<T> o{xor_partner<M>(v.v), 0u};
    if constexpr (SEG) {
        o.f = xor_partner<M>(v.f);
        return (lane & M) ? op<SEG>(o, v) : op<SEG>(v, o);   // lower lane is the left operand
    } else {
        return Seg<T>{v.v + o.v, 0u};
    }
}

// PW over the 256 threads of the workgroup (leaf i = thread i); uniform result.
template <bool SEG, typename T>
__device__ __forceinline__ Seg<T> block_pw(Seg<T> v, int lane, int wave, Seg<T>* s_tmp) {
    v = bfly<1, SEG>(v, lane);
    v = bfly<2, SEG>(v, lane);
    v = bfly<4, SEG>(v, lane);
    v = bfly<8, SEG>(v, lane);
    v = bfly<16, SEG>(v, lane);
    Seg<T> lo{readlane(v.v, 0), SEG ? readlane(v.f, 0) : 0u};
    Seg<T> hi{readlane(v.v, 32), SEG ? readlane(v.f, 32) : 0u};
    v = op<SEG>(lo, hi);
    if (lane == 0) s_tmp[wave] = v;
    __syncthreads();
    const Seg<T> r = op<SEG>(op<SEG>(s_tmp[0], s_tmp[1]), op<SEG>(s_tmp[2], s_tmp[3]));
    __syncthreads();
    return r;
}

// Two block_pw at once (leaf i = thread i of each), sharing the exchange and its barriers;
// s_tmp holds 2 * 4 entries.
template <bool SEG, typename T>
__device__ __forceinline__ void block_pw2(Seg<T> v, Seg<T> w, int lane, int wave, Seg<T>* s_tmp,
                                          Seg<T>& rv, Seg<T>& rw) {
    v = bfly<1, SEG>(v, lane);
    w = bfly<1, SEG>(w, lane);
    v = bfly<2, SEG>(v, lane);
    w = bfly<2, SEG>(w, lane);
    v = bfly<4, SEG>(v, lane);
    w = bfly<4, SEG>(w, lane);
    v = bfly<8, SEG>(v, lane);
    w = bfly<8, SEG>(w, lane);
    v = bfly<16, SEG>(v, lane);
    w = bfly<16, SEG>(w, lane);
    const Seg<T> vlo{readlane(v.v, 0), SEG ? readlane(v.f, 0) : 0u};
    const Seg<T> vhi{readlane(v.v, 32), SEG ? readlane(v.f, 32) : 0u};
    const Seg<T> wlo{readlane(w.v, 0), SEG ? readlane(w.f, 0) : 0u};
    const Seg<T> whi{readlane(w.v, 32), SEG ? readlane(w.f, 32) : 0u};
    if (lane == 0) {
        s_tmp[wave] = op<SEG>(vlo, vhi);
        s_tmp[4 + wave] = op<SEG>(wlo, whi);
    }
    __syncthreads();
    rv = op<SEG>(op<SEG>(s_tmp[0], s_tmp[1]), op<SEG>(s_tmp[2], s_tmp[3]));
    rw = op<SEG>(op<SEG>(s_tmp[4], s_tmp[5]), op<SEG>(s_tmp[6], s_tmp[7]));
    __syncthreads();
}

// ---------------------------------------------------------------- segment heads

// First k in [0, cnt) with offs[k] >= target (cnt if none).  All threads take part.
__device__ int64_t wg_lower_bound(const int64_t* __restrict__ offs, int64_t cnt, int64_t target,
                                  int tid) {
    int64_t lo = 0, hi = cnt;
    while (hi - lo > 256) {
        const int64_t step = (hi - lo + 255) / 256;
        const int64_t k = lo + (int64_t)(tid + 1) * step - 1;
        const int pred = (k < hi) && (offs[k] < target);
        const int c = __syncthreads_count(pred);
        const int64_t nhi = lo + (int64_t)(c + 1) * step - 1;
        lo = lo + (int64_t)c * step;
        if (nhi < hi) hi = nhi;
    }
    const int64_t k = lo + tid;
    const int pred = (k < hi) && (offs[k] < target);
    return lo + __syncthreads_count(pred);
}

// The smallest offset value that can mark a head in the tile starting at flipped position F0
// (forward: F0; reverse: n - F0 - T, at least 1).  The tile's heads start at the first offset
// index k in [0, nseg] with offs[k] >= that value.
__device__ __forceinline__ int64_t heads_lo(int64_t n, bool rev, int64_t F0) {
    if (!rev) return F0;
    return (n - F0 - kT > 1) ? n - F0 - kT : 1;
}

// Bit b of s_heads marks flipped position F0 + b (b in [0, T]) as a segment head.
// Forward: heads are the offsets o < n.  Reverse: flipped position n - o for offsets o > 0
// (the last element of every non-empty segment).  Used by single-workgroup scans; the others
// take the same bits from a bitmap built before the scan (k_mark_heads).
__device__ void build_heads(const int64_t* __restrict__ offs, int64_t nseg, int64_t n, bool rev,
                            int64_t F0, uint32_t* s_heads, int tid) {
    for (int i = tid; i < kHeadWords; i += 256) s_heads[i] = 0u;
    const int64_t lo_v = heads_lo(n, rev, F0);
    const int64_t hi_v = !rev ? ((F0 + kT < n - 1) ? F0 + kT : n - 1) : n - F0;
    const int64_t k0 = wg_lower_bound(offs, nseg + 1, lo_v, tid);   // ends with a barrier
    for (int64_t base = k0;; base += 256) {
        const int64_t k = base + tid;
        bool in = false;
        if (k <= nseg) {
            const int64_t o = offs[k];
            if (o <= hi_v) {
                in = true;
                // the range check only matters for offsets that break the sorted precondition:
                // they give unspecified results, never an out-of-range LDS write
                if (o >= lo_v) {
                    const int bit = (int)((rev ? n - o : o) - F0);
                    atomicOr(&s_heads[bit >> 5], 1u << (bit & 31));
                }
            }
        }
        if (!__syncthreads_and(in)) break;   // offsets are sorted: stop at the first miss
    }
}

// ---------------------------------------------------------------- wave load / store

// Vector types for 16-byte accesses with non-temporal hints (streaming data is touched once).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// the 16-byte vector of a 4-byte element type
template <typename T>
using v4_t = typename std::conditional<__is_same(T, float), f32x4, u32x4>::type;

template <typename T>
__device__ __forceinline__ bool aligned16(const T* p) {
    return (reinterpret_cast<uintptr_t>(p) & 15) == 0;
}

// Lane t's run (flipped positions f0 .. f0 + 31, f0 = fw + 32 t) straight into registers: each
// lane reads its own 128 (f32) or 256 (f64) contiguous bytes.  Identity past n.  `vec` (uniform)
// says the whole wave is in range and its runs are 16-byte aligned.  The 16-byte loads are
// issued on every path (from a 256-byte dummy line when `vec` is false, the element loads then
// supplying the values), so the count of loads issued after any earlier load is the same on
// every path and the compiler can wait for that earlier load with a partial counter instead of
// draining the queue.  No streaming hint: consecutive loads of a lane share cache lines.
template <typename T, bool REV>
__device__ __forceinline__ void load_run(const T* __restrict__ x, int64_t n, int64_t fw, bool vec,
                                         const T* __restrict__ dummy, T (&r)[kV], int lane) {
    const int64_t f0 = fw + (int64_t)lane * kV;
    // forward: run = x[f0 .. f0 + 32); reverse: original x[n - f0 - 32 .. n - f0) backwards
    const T* p = vec ? (REV ? x + (n - f0 - kV) : x + f0) : dummy;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int i = 0; i < kV / 4; ++i) {
            const v4_t<T> q = reinterpret_cast<const v4_t<T>*>(p)[i];
            if (REV) {
                r[kV - 1 - 4 * i] = q.x; r[kV - 2 - 4 * i] = q.y;
                r[kV - 3 - 4 * i] = q.z; r[kV - 4 - 4 * i] = q.w;
            } else {
                r[4 * i] = q.x; r[4 * i + 1] = q.y; r[4 * i + 2] = q.z; r[4 * i + 3] = q.w;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kV / 2; ++i) {
            const f64x2 q = reinterpret_cast<const f64x2*>(p)[i];
            if (REV) {
                r[kV - 1 - 2 * i] = q.x; r[kV - 2 - 2 * i] = q.y;
            } else {
                r[2 * i] = q.x; r[2 * i + 1] = q.y;
            }
        }
    }
    if (!vec) {
        // element loads; positions past n read element n - 1 and take the identity (both
        // operands of the select are plain values, so no branch around the load is formed)
        const T id = ident<T>();
#pragma unroll
        for (int k = 0; k < kV; ++k) {
            const int64_t f = f0 + k;
            const int64_t fc = f < n ? f : n - 1;
            const T v = x[REV ? n - 1 - fc : fc];
            r[k] = (f < n) ? v : id;
        }
    }
}

// One 16-byte non-temporal store of kGW consecutive elements (4 f32 or 2 f64): a lane writes
// 16 contiguous bytes per store, so a wave's store covers 1 KiB without gaps.  (Two 16-byte
// stores per lane at a 32-byte stride, each leaving every other 16 bytes to the other, made
// the f64 readout of a 2^28 scan about 25% to 80% slower on MI355X.)
template <typename T>
constexpr int kGW = 16 / (int)sizeof(T);

template <typename T>
__device__ __forceinline__ void nt_store16(T* p, const T (&v)[kGW<T>]) {
    if constexpr (sizeof(T) == 4) {
        v4_t<T> q = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(q, reinterpret_cast<v4_t<T>*>(p));
    } else {
        f64x2 q = {v[0], v[1]};
        __builtin_nontemporal_store(q, reinterpret_cast<f64x2*>(p));
    }
}

// Parked tile: each wave keeps its 2048 lane-serial prefixes in LDS in run order, lane t's run
// at t * 33 (one spare slot per run keeps both the run-wise writes and the element-wise reads
// free of bank conflicts), together with each lane's combine value X and head bits.
constexpr int kPark = kWaveElems + kWaveElems / 32;

template <typename T>
__device__ __forceinline__ void park_runs(T* pk, const T (&r)[kV], int lane) {
    const int rb = lane * (kV + 1);
#pragma unroll
    for (int k = 0; k < kV; ++k) pk[rb + k] = r[k];
}

// Flipped element e of the wave (lane e / 32, position e % 32): y = X + s, except that a
// segment head at or before the position inside the lane's run keeps s.
template <typename T, bool SEG>
__device__ __forceinline__ T combine_at(const T* pk, const T* xs, const uint32_t* hbs, int e) {
    const T sv = pk[pad(e)];
    const int L = e >> 5;
    if constexpr (SEG) {
        if (hbs[L] << (31 - (e & 31))) return sv;
    }
    return xs[L] + sv;
}

template <typename T, bool SEG, bool REV, bool EXCL>
__device__ __forceinline__ void readout_range(T* __restrict__ y, int64_t n, int64_t F0, int64_t fw,
                                              const T* pk, const T* xs, const uint32_t* hbs,
                                              const uint32_t* s_heads, int lane);

// Whole-wave readout, inclusive: flipped positions fw .. fw + 2047 to y.  16-byte
// non-temporal stores where the wave is in range and aligned, else readout_range (its aligned
// interior by 16-byte stores, the ends by elements).
template <typename T, bool SEG, bool REV>
__device__ __forceinline__ void readout_incl(T* __restrict__ y, int64_t n, int64_t fw, const T* pk,
                                             const T* xs, const uint32_t* hbs, int lane) {
    const bool full = fw + kWaveElems <= n;
    T* base = REV ? y + (n - fw - kWaveElems) : y + fw;   // lowest original index of the wave
    constexpr int GW = kGW<T>;
    if (full && aligned16(base)) {
#pragma unroll
        for (int r = 0; r < kWaveElems / (64 * GW); ++r) {
            const int o = r * 64 * GW + GW * lane;            // original offset within the wave
            T v[GW];
#pragma unroll
            for (int k = 0; k < GW; ++k)   // flipped element of offset o + k
                v[k] = combine_at<T, SEG>(pk, xs, hbs, REV ? (kWaveElems - 1) - o - k : o + k);
            nt_store16<T>(base + o, v);
        }
    } else {
        // a partial or unaligned wave: aligned interior with 16-byte stores, ends by elements
        readout_range<T, SEG, REV, false>(y, n, fw, fw, pk, xs, hbs, nullptr, lane);
    }
}

// Readout of a wave's range at any alignment: the output value of flipped position f is the
// inclusive value of f - SH (SH = 1 exclusive, 0 inclusive), +0.0 where an exclusive scan's f
// is a segment head.  The flipped positions fw + SH .. fw + 2047 + SH, clipped to n - 1, are
// one contiguous range of original addresses; its 16-byte-aligned interior is written with
// 16-byte non-temporal stores, the at most 3 + 3 elements at its ends with element stores.
template <typename T, bool SEG, bool REV, bool EXCL>
__device__ __forceinline__ T range_value(int64_t n, int64_t F0, int64_t fw, int64_t addr,
                                        const T* pk, const T* xs, const uint32_t* hbs,
                                        const uint32_t* s_heads) {
    constexpr int SH = EXCL ? 1 : 0;
    const int64_t fp = REV ? n - 1 - addr : addr;   // flipped position written
    const int e = (int)(fp - SH - fw);              // wave element whose inclusive value it takes
    if constexpr (SEG && EXCL) {
        const int bit = (int)(fp - F0);
        if ((s_heads[bit >> 5] >> (bit & 31)) & 1u) return T(0.0);
    }
    return combine_at<T, SEG>(pk, xs, hbs, e);
}

template <typename T, bool SEG, bool REV, bool EXCL>
__device__ __forceinline__ void readout_range(T* __restrict__ y, int64_t n, int64_t F0, int64_t fw,
                                              const T* pk, const T* xs, const uint32_t* hbs,
                                              const uint32_t* s_heads, int lane) {
    constexpr int SH = EXCL ? 1 : 0;
    // flipped positions fw + SH .. fw + 2047 + SH, clipped to n - 1; as addresses [lo, hi)
    const int64_t flo = fw + SH;
    const int64_t last = (fw + kWaveElems - 1 + SH < n - 1) ? fw + kWaveElems - 1 + SH : n - 1;
    if (last < flo) return;
    const int64_t lo = REV ? n - 1 - last : flo;
    const int64_t hi = REV ? n - flo : last + 1;
    // interior [A, Z): starts at the first 16-byte-aligned element, whole 16-byte groups
    constexpr int64_t GW = kGW<T>;   // elements per 16 bytes
    const int64_t ye = (int64_t)(reinterpret_cast<uintptr_t>(y) / sizeof(T));
    int64_t A = lo + ((GW - ((ye + lo) % GW)) % GW);
    if (A > hi) A = hi;
    const int64_t Z = A + ((hi - A) / GW) * GW;
    for (int64_t k = lo + lane; k < A; k += 64)
        y[k] = range_value<T, SEG, REV, EXCL>(n, F0, fw, k, pk, xs, hbs, s_heads);
    for (int64_t k = Z + lane; k < hi; k += 64)
        y[k] = range_value<T, SEG, REV, EXCL>(n, F0, fw, k, pk, xs, hbs, s_heads);
    const int ngroups = (int)((Z - A) / GW);   // at most 2048 / GW
    // wave element read for address A + m: forward e = e0 + m, reverse e = e0 - m (e0 small);
    // its segment-head bit, when segmented: flipped position - F0 = hoff + e + SH
    const int e0 = REV ? (int)(n - 1 - SH - fw - A) : (int)(A - SH - fw);
    const int hoff = (int)(fw - F0);
    T* const yA = y + A;
#pragma unroll
    for (int r = 0; r < kWaveElems / (64 * (int)GW); ++r) {
        const int gi = r * 64 + lane;
        if (gi < ngroups) {
            T v[GW];
#pragma unroll
            for (int k = 0; k < (int)GW; ++k) {
                const int e = REV ? e0 - ((int)GW * gi + k) : e0 + ((int)GW * gi + k);
                T val = combine_at<T, SEG>(pk, xs, hbs, e);
                if constexpr (SEG && EXCL) {
                    const int bit = hoff + e + SH;
                    if ((s_heads[bit >> 5] >> (bit & 31)) & 1u) val = T(0.0);
                }
                v[k] = val;
            }
            nt_store16<T>(yA + (int64_t)GW * gi, v);
        }
    }
}

template <typename T, bool SEG, bool REV>
__device__ __forceinline__ void readout_excl(T* __restrict__ y, int64_t n, int64_t F0, int64_t fw,
                                             const T* pk, const T* xs, const uint32_t* hbs,
                                             const uint32_t* s_heads, int lane) {
    readout_range<T, SEG, REV, true>(y, n, F0, fw, pk, xs, hbs, s_heads, lane);
}

// ---------------------------------------------------------------- the kernel

template <typename T>
struct ScanArgs {
    const T* x;
    T* y;
    int64_t n;
    const int64_t* offs;
    int64_t nseg;
    uint64_t* agg;       // slot_words<T>() words per tile: tile totals
    uint64_t* gtot;      // slot_words<T>() words per anchor interval: interval totals
    uint64_t* carry;     // slot_words<T>() words per super-interval boundary: carries
    uint32_t* ticket;    // kCounters tile counters, kCounterStride words apart
    uint32_t* err;       // raised when a wait hit the spin bound
    const T* dummy;      // 256 bytes that the 16-byte loads of a non-vector run read instead
    const uint32_t* hbits;  // segmented: bit f marks flipped position f as a segment head
                            // (null: each tile searches the offsets itself)
    int64_t col_stride;  // k_scan_small: elements between the columns workgroups take in turn
    int ntiles;
    int nctr;            // tile counters in use: min(kCounters, grid)
    int rev;
    int excl;
    int A;               // tiles per anchor interval (the spec's 256; smaller only in tests)
    int A2;              // intervals per super-interval (likewise)
    uint32_t delay_seed; // test only: seeded pauses before status publications (delay_us > 0)
    uint32_t delay_us;
};

// Test only (delay_us > 0): a pause of up to delay_us microseconds, chosen by a hash of the
// seed, the tile and the kind of publication, taken by the publishing thread of one
// publication in four before it writes its status words.  Successors then find those words
// ready or not ready at different times from seed to seed, which must not change a bit.
template <typename T>
__device__ __forceinline__ void test_delay(const ScanArgs<T>& a, int j, uint32_t kind) {
    if (a.delay_us == 0u) return;
    uint32_t h = a.delay_seed ^ ((uint32_t)j * 0x9E3779B1u) ^ (kind * 0x85EBCA77u);
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    h *= 0x297A2D39u;
    h ^= h >> 15;
    if (h & 3u) return;
    const uint64_t ticks = (uint64_t)((h >> 2) % (a.delay_us + 1u)) * 100u;   // 100 MHz clock
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

// A tile's head words from the bitmap: word i of tile j is bitmap word 256 j + i, i in [0, 256]
// (word 256 is the next tile's first).  Every thread loads two words, the second the same for
// all, and a tile past the end reads tile 0's (never used), so every path issues the same loads.
struct HeadWords {
    uint32_t w, w256;
};

template <typename T, bool SEG>
__device__ __forceinline__ HeadWords load_head_words(const ScanArgs<T>& a, int j, int tid) {
    HeadWords h{0u, 0u};
    if constexpr (SEG) {
        if (a.hbits) {
            const size_t t = j < a.ntiles ? (size_t)j * (kHeadWords - 1) : 0;
            h.w = a.hbits[t + tid];
            h.w256 = a.hbits[t + (kHeadWords - 1)];
        }
    }
    return h;
}

// Local part of one tile once its runs are in registers: segment heads, lane-serial prefixes
// (left in r), in-wave and wave-level Kogge-Stone; returns the tile total.
template <typename T, bool SEG, bool REV>
__device__ __forceinline__ Seg<T> tile_local(const ScanArgs<T>& a, int j, T (&r)[kV], uint32_t& hb,
                                             Seg<T>& P, Seg<T>& p, uint32_t* s_heads,
                                             Seg<T>* s_wtot, int tid, int lane, int wave,
                                             HeadWords hw) {
    const int64_t F0 = (int64_t)j * kT;
    if constexpr (SEG) {
        if (a.hbits) {
            // the words were loaded with the tile; the barrier below publishes them before any
            // readout looks at another thread's word
            s_heads[tid] = hw.w;
            if (tid == 0) s_heads[kHeadWords - 1] = hw.w256;
            hb = hw.w;
        } else {
            build_heads(a.offs, a.nseg, a.n, REV, F0, s_heads, tid);
            hb = s_heads[wave * 64 + lane];
        }
    } else {
        hb = 0u;
    }

    // lane-serial prefix
#pragma unroll
    for (int k = 1; k < kV; ++k) {
        if (SEG && ((hb >> k) & 1u)) continue;
        r[k] = r[k - 1] + r[k];
    }
    Seg<T> u{r[kV - 1], hb != 0u ? 1u : 0u};

    // Kogge-Stone over the lane totals of the wave
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
        Seg<T> o{shfl_up(u.v, d, lane), SEG ? shfl_up(u.f, d, lane) : 0u};
        if (lane >= d) u = op<SEG>(o, u);
    }
    p = Seg<T>{shfl_up(u.v, 1, lane), SEG ? shfl_up(u.f, 1, lane) : 0u};
    if (lane == 0) p = seg_ident<T>();

    // Kogge-Stone over the 4 wave totals
    if (lane == 63) s_wtot[wave] = u;
    __syncthreads();
    const Seg<T> w0 = s_wtot[0], w1 = s_wtot[1], w2 = s_wtot[2], w3 = s_wtot[3];
    const Seg<T> o1 = op<SEG>(w0, w1), o2 = op<SEG>(w1, w2), o3 = op<SEG>(w2, w3);
    const Seg<T> om2 = op<SEG>(w0, o2), om3 = op<SEG>(o1, o3);
    P = wave == 0 ? seg_ident<T>() : wave == 1 ? w0 : wave == 2 ? o1 : om2;
    return om3;
}

// Where a whole wave's memory range [p0, p0 + 2048) meets 16-byte alignment: h elements before
// the first aligned one, then ng whole 16-byte groups, then 2048 - h - ng G trailing elements
// (h and the trailing count are below G).  The same for every lane.
template <typename T>
struct WaveSplit {
    int h, ng;
};

template <typename T>
__device__ __forceinline__ WaveSplit<T> wave_split(const T* p0) {
    constexpr int G = 16 / (int)sizeof(T);
    const int h = (int)(((uintptr_t)0 - reinterpret_cast<uintptr_t>(p0)) % 16 / sizeof(T));
    return WaveSplit<T>{h, (kWaveElems - h) / G};
}

// The edge element lane l loads for a split: index m in the wave's range, or -1.
template <typename T>
__device__ __forceinline__ int edge_index(WaveSplit<T> sp, int lane) {
    constexpr int G = 16 / (int)sizeof(T);
    const int tail0 = sp.h + sp.ng * G;
    if (lane < sp.h) return lane;
    if (lane - sp.h < kWaveElems - tail0) return tail0 + (lane - sp.h);
    return -1;
}

// The wave's 2048 elements in memory order, coalesced, for a whole wave: its ng whole 16-byte
// groups, r[g * G + i] = element h + (g * 64 + lane) * G + i of the wave's memory range (a lane
// past the last group loads that group again, unused), and the at most 2 (G - 1) elements
// before and after them, one per lane, into *edge; runs_from_lds turns them into runs.  Every
// address is the wave's base plus a lane offset.  (Each lane loading its own 128-byte run
// touches 64 lines per load instruction; coalesced, a load covers 1 KiB: on MI355X at 2^28 the
// exclusive f32 scan went 0.45 -> 0.42 ms, the segmented one 0.49 -> 0.46 ms, f64 0.39 -> 0.38
// ms, the inclusive f32 scan unchanged.)  A wave that is not whole loads the dummy line and
// then its run by elements, already in run order.  With ALN, a wave that starts 16-byte aligned
// skips the edge load (a wave-uniform branch); runs_from_lds takes the same flag.  On MI355X
// the branches paid in the segmented scan (f32 at 2^28: 448 -> 434 us) and cost in the others
// (inclusive 392 -> 398 us), so the segmented kernels take them.  NT marks the group loads
// non-temporal (taken for inputs of 512 MiB and more, twice the GPU's last-level cache).
template <typename T, bool REV, bool ALN, bool NT>
__device__ __forceinline__ void load_wave_coal(const T* __restrict__ x, int64_t n, int64_t fw,
                                               const T* __restrict__ dummy, T (&r)[kV], T& edge,
                                               int lane) {
    constexpr int G = 16 / (int)sizeof(T);
    const bool whole = fw + kWaveElems <= n;
    const T* p0 = whole ? x + (REV ? n - fw - kWaveElems : fw) : dummy;
    const WaveSplit<T> sp = whole ? wave_split<T>(p0) : WaveSplit<T>{0, 16};
    const v4_t<T>* base = reinterpret_cast<const v4_t<T>*>(p0 + sp.h);
#pragma unroll
    for (int g = 0; g < kV / G; ++g) {
        const int idx = g * 64 + lane;
        const int off = whole ? (idx < sp.ng ? idx : sp.ng - 1) : (g & 15);
        if constexpr (sizeof(T) == 4) {
            const v4_t<T> q = NT ? __builtin_nontemporal_load(base + off) : base[off];
            r[4 * g] = q.x; r[4 * g + 1] = q.y; r[4 * g + 2] = q.z; r[4 * g + 3] = q.w;
        } else {
            const f64x2* b2 = reinterpret_cast<const f64x2*>(base);
            const f64x2 q = NT ? __builtin_nontemporal_load(b2 + off) : b2[off];
            r[2 * g] = q.x; r[2 * g + 1] = q.y;
        }
    }
    edge = T(0);
    if (whole && (!ALN || sp.h != 0)) {
        const int m = edge_index<T>(sp, lane);
        edge = p0[m >= 0 ? m : 0];
    }
    if (!whole) {
        const int64_t f0 = fw + (int64_t)lane * kV;
        const T id = ident<T>();
#pragma unroll
        for (int k = 0; k < kV; ++k) {
            const int64_t f = f0 + k;
            const int64_t fc = f < n ? f : n - 1;
            const T v = x[REV ? n - 1 - fc : fc];
            r[k] = (f < n) ? v : id;
        }
    }
}

// Runs of the wave's part of tile j into registers (vector loads when the wave is whole and
// aligned, else element loads with identity past n).
template <typename T, bool REV>
__device__ __forceinline__ void load_tile(const ScanArgs<T>& a, int j, int wave, T (&r)[kV],
                                          int lane) {
    const int64_t fw = (int64_t)j * kT + (int64_t)wave * kWaveElems;
    const int64_t reg0 = REV ? a.n - fw - kWaveElems : fw;   // lowest original index
    const bool vec = (fw + kWaveElems <= a.n) && aligned16(a.x + reg0);
    load_run<T, REV>(a.x, a.n, fw, vec, a.dummy, r, lane);
}

// The same wave, coalesced (load_wave_coal); whole waves then go through runs_from_lds.
template <typename T, bool REV, bool ALN, bool NT>
__device__ __forceinline__ void load_tile_coal(const ScanArgs<T>& a, int j, int wave, T (&r)[kV],
                                               T& edge, int lane) {
    const int64_t fw = (int64_t)j * kT + (int64_t)wave * kWaveElems;
    load_wave_coal<T, REV, ALN, NT>(a.x, a.n, fw, a.dummy, r, edge, lane);
}

// Whether tile j's wave is whole (then load_tile_coal left it in memory order, for
// runs_from_lds).
template <typename T, bool REV>
__device__ __forceinline__ bool tile_vec(const ScanArgs<T>& a, int j, int wave) {
    const int64_t fw = (int64_t)j * kT + (int64_t)wave * kWaveElems;
    return fw + kWaveElems <= a.n;
}

// Coalesced wave data (memory order) to lane runs through the wave's park area: element m of
// the wave's memory range is flipped element e = m (forward) or 2047 - m (reverse), written at
// pad(e); lane t then reads its run at t * 33.  The park area must be free.
template <typename T, bool REV, bool ALN>
__device__ __forceinline__ void runs_from_lds(const ScanArgs<T>& a, int j, int wave, T* pk,
                                              T (&r)[kV], T edge, int lane) {
    constexpr int G = 16 / (int)sizeof(T);
    const int64_t fw = (int64_t)j * kT + (int64_t)wave * kWaveElems;
    const WaveSplit<T> sp = wave_split<T>(a.x + (REV ? a.n - fw - kWaveElems : fw));
    if (ALN && sp.h == 0) {
        // aligned: every lane holds whole groups, no edge
#pragma unroll
        for (int g = 0; g < kV / G; ++g) {
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const int m = (g * 64 + lane) * G + i;
                const int e = REV ? (kWaveElems - 1) - m : m;
                pk[pad(e)] = r[g * G + i];
            }
        }
    } else {
#pragma unroll
        for (int g = 0; g < kV / G; ++g) {
            if (g * 64 + lane < sp.ng) {
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    const int m = sp.h + (g * 64 + lane) * G + i;
                    const int e = REV ? (kWaveElems - 1) - m : m;
                    pk[pad(e)] = r[g * G + i];
                }
            }
        }
        const int me = edge_index<T>(sp, lane);
        if (me >= 0) {
            const int e = REV ? (kWaveElems - 1) - me : me;
            pk[pad(e)] = edge;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int rb = lane * (kV + 1);
#pragma unroll
    for (int k = 0; k < kV; ++k) r[k] = pk[rb + k];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Where tile j's look-back polls go: the earlier tile totals of its anchor interval and the
// earlier interval totals of its super-interval.
struct LookBack {
    int q, cnt, Q, qcnt;
};

__device__ __forceinline__ LookBack look_back_of(int j, int A, int A2) {
    LookBack lb;
    lb.q = j / A;
    lb.cnt = j - lb.q * A;
    lb.Q = lb.q / A2;
    lb.qcnt = lb.q - lb.Q * A2;
    return lb;
}

// Interval totals never change once published, so thread t keeps the total of interval
// Q * A2 + t once it has read it: gknown (uniform) counts the intervals of super-interval gQ
// held that way.  Only newer intervals are polled.
template <typename T>
struct GCache {
    Seg<T> g;
    int known;
    int Q;
};

template <typename T>
__device__ __forceinline__ bool g_cached(const GCache<T>& gc, const LookBack& lb, int tid) {
    return lb.Q == gc.Q && tid < gc.known;
}

template <typename T>
__device__ __forceinline__ void issue_look_back(const ScanArgs<T>& a, const LookBack& lb,
                                                const GCache<T>& gc, Poll<T>& pl, int tid) {
    constexpr int SW = slot_words<T>();
    poll_issue<T>(pl, a.agg + (size_t)(lb.q * a.A + tid) * SW, tid < lb.cnt,
                  a.gtot + (size_t)(lb.Q * a.A2 + tid) * SW,
                  tid < lb.qcnt && !g_cached(gc, lb, tid));
}

// ---- adaptive look-back: the NON-deterministic baseline the benchmark compares against.
// Only the benchmark's separate library instantiates it (libdet.so never does): the classic
// decoupled look-back, in which tile j uses the inclusive prefix of the nearest predecessor
// that has already published one and adds the totals of the tiles after it, so its bracketing
// follows which predecessors had finished (drjit-core pull request "Make CUDA floating-point
// prefix sums deterministic", section "Root cause").  Thread t of tile j polls tile
// base - 256 + t (base = j, then 256 further back per window): its total (published at its
// local step, a.agg) and its inclusive prefix (published when it finished, a.gtot).
template <typename T>
__device__ __forceinline__ void issue_adaptive(const ScanArgs<T>& a, int base, Poll<T>& pl,
                                               int tid) {
    constexpr int SW = slot_words<T>();
    const int t = base - 256 + tid;
    const size_t o = (size_t)(t >= 0 ? t : 0) * SW;
    poll_issue<T>(pl, a.agg + o, t >= 0, a.gtot + o, t >= 0);
}

// E_j of the adaptive look-back: waits for each polled tile's total (as the anchored kernel
// does, so forward progress is the same), takes the inclusive prefixes as observed, and forms
// E_j = incl(nearest finished tile) + (totals of the tiles after it, by PW over their window
// slots) + (the totals of nearer windows).  Uniform result.
template <bool SEG, typename T>
__device__ __forceinline__ Seg<T> adaptive_prefix(const ScanArgs<T>& a, int j, Poll<T>& pl,
                                                  Seg<T>* s_tmp, Seg<T>& s_carry, int* s_best,
                                                  int tid, int lane, int wave) {
    constexpr int SW = slot_words<T>();
    Seg<T> later = seg_ident<T>();
    for (int base = j;; base -= 256) {
        const int t = base - 256 + tid;
        const bool use = t >= 0;
        const size_t o = (size_t)(use ? t : 0) * SW;
        const Seg<T> ag = poll_finish_set<T>(pl.w, a.agg + o, use, a.err);
        repoll(pl.w[SW], a.gtot + o);
        if constexpr (SW == 2) repoll(pl.w[SW + 1], a.gtot + o + 1);
        bool inc = use && ((pl.w[SW] >> 32) & kReady);
        if constexpr (SW == 2) inc = inc && ((pl.w[SW + 1] >> 32) & kReady);
        const uint64_t m = __ballot(inc);
        if (lane == 0) s_best[wave] = m ? wave * 64 + 63 - (int)__builtin_clzll(m) : -1;
        __syncthreads();
        const int best = max(max(s_best[0], s_best[1]), max(s_best[2], s_best[3]));
        if (best == tid) s_carry = unpack<T>(pl.w[SW], SW == 2 ? pl.w[SW + 1] : 0ull);
        const bool done = best >= 0 || base <= 256;
        const Seg<T> S = block_pw<SEG, T>(use && tid > best ? ag : seg_ident<T>(), lane, wave,
                                          s_tmp);   // its barriers also publish s_carry
        if (done) {
            const Seg<T> prefix = best >= 0 ? s_carry : seg_ident<T>();
            __syncthreads();
            return op<SEG>(op<SEG>(prefix, S), later);
        }
        later = op<SEG>(S, later);
        issue_adaptive<T>(a, base - 256, pl, tid);
    }
}

// Everything after a parked tile's look-back polls were issued: finish the look-back, publish
// the interval total (the interval's last tile) and forward the super-interval carry (its last
// tile), then each lane's combine value X = ((((CC + WG) + W_j) + P) + p) goes to LDS and the
// wave reads its parked prefixes out, adds X and stores them.
template <typename T, bool SEG, bool REV, bool EXCL, bool ADAPTIVE>
__device__ __forceinline__ void finish_tile(const ScanArgs<T>& a, int j, const LookBack& lb,
                                            Poll<T>& pl, GCache<T>& gc, Seg<T> P, Seg<T> p,
                                            Seg<T> agg,
                                            Seg<T>* s_tmp, Seg<T>& s_carry, int* s_best,
                                            const T* pk, T* xs,
                                            const uint32_t* hbs, const uint32_t* s_heads, int tid,
                                            int lane, int wave) {
    constexpr int SW = slot_words<T>();
    uint32_t* err = a.err;
    Seg<T> E;
    if constexpr (ADAPTIVE) {
        E = adaptive_prefix<SEG, T>(a, j, pl, s_tmp, s_carry, s_best, tid, lane, wave);
        if (tid == 0) publish<T>(a.gtot + (size_t)j * SW, op<SEG>(E, agg));
    } else {
    (void)s_best;
    const Seg<T> mine =
        poll_finish_set<T>(pl.w, a.agg + (size_t)(lb.q * a.A + tid) * SW, tid < lb.cnt, err);
    const bool cached = g_cached(gc, lb, tid);
    Seg<T> gmine = poll_finish_set<T>(pl.w + SW, a.gtot + (size_t)(lb.Q * a.A2 + tid) * SW,
                                      tid < lb.qcnt && !cached, err);
    if (cached) gmine = gc.g;
    if (tid < lb.qcnt) gc.g = gmine;
    gc.known = lb.qcnt;
    gc.Q = lb.Q;
    Seg<T> Wj, WG;
    block_pw2<SEG, T>(mine, gmine, lane, wave, s_tmp, Wj, WG);
    (void)agg;

    // carry into the super-interval (the identity for the first), published by the previous
    // super-interval's last tile in its local step (publish_interval_total)
    Seg<T> CC = seg_ident<T>();
    if (lb.Q > 0) {
        if (tid == 0) s_carry = wait_slot<T>(a.carry + (size_t)lb.Q * SW, err);
        __syncthreads();
        CC = s_carry;
    }
    E = op<SEG>(op<SEG>(CC, WG), Wj);
    }
    xs[lane] = op<SEG>(op<SEG>(E, P), p).v;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t F0 = (int64_t)j * kT;
    const int64_t fw = F0 + (int64_t)wave * kWaveElems;
    if (!EXCL)
        readout_incl<T, SEG, REV>(a.y, a.n, fw, pk, xs, hbs, lane);
    else
        readout_excl<T, SEG, REV>(a.y, a.n, F0, fw, pk, xs, hbs, s_heads, lane);
    if (EXCL && j == 0 && tid == 0) a.y[REV ? a.n - 1 : 0] = T(0.0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Tiles are claimed from nc <= kCounters counters (nc <= the grid), one per 256-byte line, and
// counter c's k-th claim is tile k * nc + c.  One counter would serialise every claim on a
// single address (about 87 claims per microsecond on this chip, below the tile rate of an f32
// scan at full bandwidth: 2^28 elements 380 -> 440 us, 2^24 28 -> 50 us).  Workgroup b belongs
// to group g = b mod 8 (on MI355X the XCD it runs on) and takes a rank r in its group as it
// starts (one rank word per group); it draws from counter (g + r) mod nc while r < nc, else
// from counter g mod nc.  Each counter's tiles are claimed in order, and a workgroup claims
// until its counter's tiles run out, so once some group has started nc workgroups every counter
// has a running workgroup until its tiles are gone, and every tile a workgroup waits on is, or
// will be, claimed by a running one.  That holds whatever else shares the GPU: with the counter
// tied to the workgroup index alone (b mod nc) two f64 scans on two streams, each filling the
// chip, could each hold every slot of an XCD the other needed for the first workgroup of a
// counter, and both waited until the wait bound gave up.  By rank, while no group of a scan has
// started nc workgroups the scan holds fewer than nc slots per XCD, and an XCD has 64 or more
// per scan kernel, so more workgroups start.  (A CPU model of two full-chip scans checks both
// choices.)  Workgroups after the first nc of a group keep the counter of their XCD, whose
// claims then stay mostly on one XCD; one rank word for the whole grid cost 7 us at the start
// of every call (about 768 workgroups on one address).  A grid larger than the resident count
// (a test hook) changes nothing as long as there are no more counters than resident workgroups
// (the host sees to it).
constexpr int kCounters = 8;
constexpr int kCounterStride = 64;   // words between counters
constexpr int kRankWord = 32;        // group g's rank word: word 32 of counter g's line

// The last tile of an anchor interval publishes the interval total G_q = PW(all A tile totals)
// right after its own local step, while its later tiles are still loading: G_q needs nothing but
// those totals, and the first tiles of the next interval need G_q when they finish.  Every tile
// total awaited here belongs to a smaller tile, published at that tile's local step.
template <bool SEG, typename T>
__device__ __forceinline__ void publish_interval_total(const ScanArgs<T>& a, int u, Seg<T> aggu,
                                                       Seg<T>* s_tmp, int tid, int lane, int wave) {
    const LookBack lb = look_back_of(u, a.A, a.A2);
    if (!(lb.cnt == a.A - 1 && u + 1 < a.ntiles)) return;
    constexpr int SW = slot_words<T>();
    const uint64_t* slot = a.agg + (size_t)(lb.q * a.A + tid) * SW;
    Poll<T> pa;
    poll_issue<T>(pa, slot, tid < lb.cnt, slot, false);
    const Seg<T> m = poll_finish_set<T>(pa.w, slot, tid < lb.cnt, a.err);
    const Seg<T> G = block_pw<SEG, T>(tid == a.A - 1 ? aggu : m, lane, wave, s_tmp);
    if (tid == 0) {
        test_delay<T>(a, u, 1u);
        publish<T>(a.gtot + (size_t)lb.q * SW, G);
    }
    // The super-interval's last tile forwards the carry CC_{Q+1} = CC_Q + PW(all A2 interval
    // totals of Q) here, in its local step, where it waits only on smaller tiles and the
    // previous carry.  (Forwarded from the tile's finish instead, the carry waited behind the
    // workgroup's next tile: when that tile closed a later interval, its local step waited on
    // tiles whose workgroups were waiting for this carry.)
    if (lb.qcnt != a.A2 - 1) return;
    const uint64_t* gslot = a.gtot + (size_t)(lb.Q * a.A2 + tid) * SW;
    Poll<T> pg;
    poll_issue<T>(pg, gslot, tid < lb.qcnt, gslot, false);
    const Seg<T> gm = poll_finish_set<T>(pg.w, gslot, tid < lb.qcnt, a.err);
    const Seg<T> H = block_pw<SEG, T>(tid == a.A2 - 1 ? G : gm, lane, wave, s_tmp);
    if (tid == 0) {
        const Seg<T> CC = lb.Q > 0 ? wait_slot<T>(a.carry + (size_t)lb.Q * SW, a.err)
                                   : seg_ident<T>();
        test_delay<T>(a, u, 2u);
        publish<T>(a.carry + (size_t)(lb.Q + 1) * SW, op<SEG>(CC, H));
    }
}

// Issues the claim of counter c's next ticket k; the tile is k * nc + c.  The counter offset
// passes through a vector register, so the compiler treats the atomic as per-lane and does not
// combine it across the wave: that expansion reads the result back at once, which would wait
// for every load issued before it.  The caller reads the ticket an iteration later.
__device__ __forceinline__ uint32_t claim_issue(uint32_t* counters, int c) {
    int off = c * kCounterStride;
    asm volatile("" : "+v"(off));
    return __hip_atomic_fetch_add(counters + off, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int ticket_tile(uint32_t k, int c, int nc) { return (int)k * nc + c; }

// Persistent workgroups, three tiles in flight each: tile c parked in LDS (published, waiting
// for its look-back), tile u in registers (its loads were issued one iteration earlier) and
// tile v loading.  Per iteration: u's local part runs and u's total is published; c's
// look-back polls leave; v's loads are issued and the tile after v is claimed; c finishes and
// is stored from LDS while v's loads are in flight; u is parked in c's place.  A tile's total
// is thus published one iteration before its workgroup waits on anything.  Tile indices are
// kept wave-uniform (scalar) and every path issues the same loads, so the wait for c's polls
// counts only the loads issued after them.  Every value a tile waits for (tile totals,
// interval totals, super-interval carries) is published in the local step of a smaller tile,
// and a local step waits only on values published by smaller tiles' local steps (its
// workgroup's previous finish waits likewise).  Tiles are claimed in counter order by running
// workgroups, so the smallest tile whose local step has not run can always run it, and every
// wait ends.  (A value published in a finish instead would wait behind that workgroup's next
// local step, whose tile may be far later.)
template <typename T, bool SEG, bool REV, bool EXCL, bool NT, bool ADAPTIVE = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 4 ? 3 : 2)))
void k_scan(ScanArgs<T> a) {
    __shared__ T s_park[kScanWaves][kPark];
    __shared__ T s_x[kScanWaves][kScanW];
    __shared__ uint32_t s_hbits[SEG ? kScanWaves : 1][kScanW];
    __shared__ uint32_t s_heads[2][SEG ? kHeadWords : 1];
    __shared__ Seg<T> s_tmp[2 * kScanWaves];
    __shared__ Seg<T> s_wtot[kScanWaves];
    __shared__ Seg<T> s_carry;
    __shared__ int s_tick[2];
    __shared__ int s_ctr;
    __shared__ int s_best[ADAPTIVE ? 4 : 1];

    const int tid = threadIdx.x;
    const int lane0 = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int SW = slot_words<T>();
    T* pk = s_park[wave];
    T* xs = s_x[wave];
    const uint32_t* hbs = s_hbits[SEG ? wave : 0];
    const int nc = a.nctr;

    // ---- prologue: the counter from this workgroup's start rank, then c loaded, local,
    // published, parked; u's loads issued
    if (tid == 0) {
        const int g = (int)(blockIdx.x & 7u);
        const uint32_t rank = __hip_atomic_fetch_add(a.ticket + g * kCounterStride + kRankWord,
                                                     1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        const int cr = rank < (uint32_t)nc ? (int)((g + (int)rank) % nc) : g % nc;
        s_ctr = cr;
        s_tick[0] = ticket_tile(claim_issue(a.ticket, cr), cr, nc);
    }
    __syncthreads();
    const int ctr = __builtin_amdgcn_readfirstlane(s_ctr);
    int c = __builtin_amdgcn_readfirstlane(s_tick[0]);
    if (c >= a.ntiles) return;
    T r[kV];
    T edc;
    load_tile_coal<T, REV, SEG, NT>(a, c, wave, r, edc, lane0);
    HeadWords hwc = load_head_words<T, SEG>(a, c, tid);
    uint32_t claimed = 0u;
    if (tid == 0) claimed = claim_issue(a.ticket, ctr);
    if (tile_vec<T, REV>(a, c, wave)) runs_from_lds<T, REV, SEG>(a, c, wave, pk, r, edc, lane0);
    uint32_t hbc;
    Seg<T> Pc, pc;
    Seg<T> aggc = tile_local<T, SEG, REV>(a, c, r, hbc, Pc, pc, s_heads[0], s_wtot, tid, lane0,
                                          wave, hwc);
    if (tid == 0) {
        test_delay<T>(a, c, 0u);
        publish<T>(a.agg + (size_t)c * SW, aggc);
        s_tick[1] = ticket_tile(claimed, ctr, nc);
    }
    if constexpr (!ADAPTIVE) publish_interval_total<SEG, T>(a, c, aggc, s_tmp, tid, lane0, wave);
    if constexpr (SEG) s_hbits[wave][lane0] = hbc;
    __syncthreads();
    int u = __builtin_amdgcn_readfirstlane(s_tick[1]);
    // u's loads (a tile past the end reads element n - 1 and is never used), brought into
    // runs through the park area before c is parked there
    T ru[kV];
    T edu;
    load_tile_coal<T, REV, SEG, NT>(a, u, wave, ru, edu, lane0);
    HeadWords hwu = load_head_words<T, SEG>(a, u, tid);
    if (tile_vec<T, REV>(a, u, wave)) runs_from_lds<T, REV, SEG>(a, u, wave, pk, ru, edu, lane0);
    park_runs<T>(pk, r, lane0);
#pragma unroll
    for (int k = 0; k < kV; ++k) r[k] = ru[k];
    if (tid == 0 && u < a.ntiles) claimed = claim_issue(a.ticket, ctr);
    LookBack lbc = look_back_of(c, a.A, a.A2);
    GCache<T> gc{seg_ident<T>(), 0, -1};
    int par = 0;   // s_heads[par] holds c's heads, s_heads[par ^ 1] receives u's

    for (;;) {
        // Re-derive the lane index each iteration so per-lane addresses are recomputed instead
        // of being held live across the loop (register pressure decides occupancy).
        int lane = lane0;
        asm volatile("" : "+v"(lane));
        const bool have_u = u < a.ntiles;

        // ---- u: local part (its loads were issued an iteration ago), total published at once
        uint32_t hbu = 0u;
        Seg<T> Pu = seg_ident<T>(), pu = seg_ident<T>(), aggu = seg_ident<T>();
        if (have_u) {
            aggu = tile_local<T, SEG, REV>(a, u, r, hbu, Pu, pu, s_heads[par ^ 1], s_wtot, tid,
                                           lane, wave, hwu);
            if (tid == 0) {
                test_delay<T>(a, u, 0u);
                publish<T>(a.agg + (size_t)u * SW, aggu);
            }
            if constexpr (!ADAPTIVE)
                publish_interval_total<SEG, T>(a, u, aggu, s_tmp, tid, lane, wave);
        }
        // the ticket claimed last iteration (v, if u exists); then c's look-back polls go out
        // ahead of v's loads
        if (tid == 0) s_tick[par] = ticket_tile(claimed, ctr, nc);
        Poll<T> pl;
        if constexpr (ADAPTIVE)
            issue_adaptive<T>(a, c, pl, tid);
        else
            issue_look_back<T>(a, lbc, gc, pl, tid);
        __syncthreads();
        const int v = have_u ? __builtin_amdgcn_readfirstlane(s_tick[par]) : a.ntiles;
        const bool have_v = v < a.ntiles;

        // ---- v: loads issued now, consumed in the next iteration; the tile after v claimed
        T rv[kV];
        T edv;
        load_tile_coal<T, REV, SEG, NT>(a, v, wave, rv, edv, lane);
        const HeadWords hwv = load_head_words<T, SEG>(a, v, tid);
        if (tid == 0 && have_v) claimed = claim_issue(a.ticket, ctr);

        // ---- c: finish the look-back, store from LDS
        finish_tile<T, SEG, REV, EXCL, ADAPTIVE>(a, c, lbc, pl, gc, Pc, pc, aggc, s_tmp, s_carry,
                                                 s_best, pk, xs,
                                       hbs, s_heads[par], tid, lane, wave);
        if (!have_u) break;

        // ---- v's data into runs through the park area (this wave's readout of c is complete),
        // then u takes c's place there
        if (tile_vec<T, REV>(a, v, wave)) runs_from_lds<T, REV, SEG>(a, v, wave, pk, rv, edv, lane);
        park_runs<T>(pk, r, lane);
        if constexpr (SEG) s_hbits[wave][lane] = hbu;
#pragma unroll
        for (int k = 0; k < kV; ++k) r[k] = rv[k];
        hwu = hwv;
        Pc = Pu;
        pc = pu;
        aggc = aggu;
        lbc = look_back_of(u, a.A, a.A2);
        c = u;
        u = v;
        par ^= 1;
        // the next tile's heads go where c's were: every wave must be done reading them
        if constexpr (SEG) __syncthreads();
    }
}

// Scans that fit in the first anchor interval: one workgroup walks the tiles in order, keeping
// the tile totals in LDS, so there are no status words to clear, no counters and no polls (one
// launch).  Workgroup b scans column b: x and y start b * col_stride elements on, all columns
// share n and the segment offsets.  Tile j's trees are those of k_scan: W_j = PW(leaf t =
// Agg_t for t < j, else the identity) and WG = PW(identity leaves); the carry is the identity;
// E = (CC + WG) + W_j.  The next tile's loads are issued before the current tile's readout.
constexpr int kSmallTiles = 1;   // from 2 tiles on the two-launch kernel is faster on MI355X

template <typename T, bool SEG, bool REV, bool EXCL>
__global__ __launch_bounds__(256) void k_scan_small(ScanArgs<T> a0) {
    __shared__ T s_park[kScanWaves][kPark];
    __shared__ T s_x[kScanWaves][kScanW];
    __shared__ uint32_t s_hbits[SEG ? kScanWaves : 1][kScanW];
    __shared__ uint32_t s_heads[2][SEG ? kHeadWords : 1];
    __shared__ Seg<T> s_tmp[2 * kScanWaves];
    __shared__ Seg<T> s_wtot[kScanWaves];
    __shared__ Seg<T> s_agg[kScanA];

    ScanArgs<T> a = a0;
    a.x += (int64_t)blockIdx.x * a0.col_stride;
    a.y += (int64_t)blockIdx.x * a0.col_stride;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (blockIdx.x == 0 && tid == 0) *a0.err = 0u;   // nothing here waits: the health word is 0
    T* pk = s_park[wave];
    T* xs = s_x[wave];
    const uint32_t* hbs = s_hbits[SEG ? wave : 0];
    T r[kV], rn[kV];
    load_tile<T, REV>(a, 0, wave, r, lane);
    HeadWords hw = load_head_words<T, SEG>(a, 0, tid);
    for (int j = 0; j < a.ntiles; ++j) {
        uint32_t hb;
        Seg<T> P, p;
        const Seg<T> agg = tile_local<T, SEG, REV>(a, j, r, hb, P, p, s_heads[j & 1], s_wtot, tid,
                                                   lane, wave, hw);
        if (tid == 0) s_agg[j] = agg;
        park_runs<T>(pk, r, lane);
        if constexpr (SEG) s_hbits[wave][lane] = hb;
        __syncthreads();
        // the next tile's loads (past the end: element n - 1, never used)
        load_tile<T, REV>(a, j + 1, wave, rn, lane);
        const HeadWords hwn = load_head_words<T, SEG>(a, j + 1, tid);
        // W_j; for tile 0 every leaf is the identity, whose tree is the identity; WG is a tree
        // of identity leaves here, the identity
        Seg<T> Wj = seg_ident<T>();
        if (j > 0) Wj = block_pw<SEG, T>(tid < j ? s_agg[tid] : seg_ident<T>(), lane, wave, s_tmp);
        const Seg<T> E = op<SEG>(op<SEG>(seg_ident<T>(), seg_ident<T>()), Wj);
        xs[lane] = op<SEG>(op<SEG>(E, P), p).v;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int64_t F0 = (int64_t)j * kT;
        const int64_t fw = F0 + (int64_t)wave * kWaveElems;
        if (!EXCL)
            readout_incl<T, SEG, REV>(a.y, a.n, fw, pk, xs, hbs, lane);
        else
            readout_excl<T, SEG, REV>(a.y, a.n, F0, fw, pk, xs, hbs, s_heads[j & 1], lane);
        if (EXCL && j == 0 && tid == 0) a.y[REV ? a.n - 1 : 0] = T(0.0);
        // every wave is done with this tile's LDS before the next tile overwrites it
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kV; ++k) r[k] = rn[k];
        hw = hwn;
    }
}

// Scans that fit in the first anchor interval (at most A tiles), in two launches with no
// status words to clear and no waiting: the first (SECOND = false) computes every tile's total
// and stores it; the second, a workgroup per tile again, recomputes its tile's local part,
// reads the totals of the tiles before it (all stored by the first launch) for W_j, and stores
// its outputs.  The trees are k_scan_small's, so the bits are the same.  x is read twice, from
// the caches at these sizes.  Grid (tiles, columns): column c scans x + c * col_stride into
// y + c * col_stride, its tile totals at agg + c * ntiles slots.
template <typename T, bool SEG, bool REV, bool EXCL, bool SECOND>
__global__ __launch_bounds__(256) void k_scan_two(ScanArgs<T> a0) {
    __shared__ T s_park[kScanWaves][kPark];
    __shared__ T s_x[kScanWaves][kScanW];
    __shared__ uint32_t s_hbits[SEG ? kScanWaves : 1][kScanW];
    __shared__ uint32_t s_heads[SEG ? kHeadWords : 1];
    __shared__ Seg<T> s_tmp[2 * kScanWaves];
    __shared__ Seg<T> s_wtot[kScanWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = (int)blockIdx.x;
    // nothing here waits: the first launch leaves the health word at 0
    if (!SECOND && j == 0 && blockIdx.y == 0 && tid == 0) *a0.err = 0u;
    ScanArgs<T> a = a0;
    a.x += (int64_t)blockIdx.y * a0.col_stride;
    a.y += (int64_t)blockIdx.y * a0.col_stride;
    T* pk = s_park[wave];
    T* xs = s_x[wave];
    const uint32_t* hbs = s_hbits[SEG ? wave : 0];
    Seg<T>* agg_slots = reinterpret_cast<Seg<T>*>(a0.agg) + (int64_t)blockIdx.y * a0.ntiles;
    T r[kV];
    T ed;
    load_tile_coal<T, REV, SEG, false>(a, j, wave, r, ed, lane);
    const HeadWords hw = load_head_words<T, SEG>(a, j, tid);
    // the second launch's totals of the earlier tiles, loaded with the tile
    Seg<T> before = seg_ident<T>();
    if (SECOND && tid < j) before = agg_slots[tid];
    if (tile_vec<T, REV>(a, j, wave)) runs_from_lds<T, REV, SEG>(a, j, wave, pk, r, ed, lane);
    uint32_t hb;
    Seg<T> P, p;
    const Seg<T> agg = tile_local<T, SEG, REV>(a, j, r, hb, P, p, s_heads, s_wtot, tid, lane,
                                               wave, hw);
    if constexpr (!SECOND) {
        if (tid == 0) agg_slots[j] = agg;
        return;
    } else {
        park_runs<T>(pk, r, lane);
        if constexpr (SEG) s_hbits[wave][lane] = hb;
        __syncthreads();
        Seg<T> Wj = seg_ident<T>();
        if (j > 0) Wj = block_pw<SEG, T>(before, lane, wave, s_tmp);
        const Seg<T> E = op<SEG>(op<SEG>(seg_ident<T>(), seg_ident<T>()), Wj);
        xs[lane] = op<SEG>(op<SEG>(E, P), p).v;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int64_t F0 = (int64_t)j * kT;
        const int64_t fw = F0 + (int64_t)wave * kWaveElems;
        if (!EXCL)
            readout_incl<T, SEG, REV>(a.y, a.n, fw, pk, xs, hbs, lane);
        else
            readout_excl<T, SEG, REV>(a.y, a.n, F0, fw, pk, xs, hbs, s_heads, lane);
        if (EXCL && j == 0 && tid == 0) a.y[REV ? a.n - 1 : 0] = T(0.0);
    }
}

// Segment heads as a bitmap over flipped positions, built before a segmented scan on a
// cleared bitmap: forward, bit o for every offset o < n; reverse, bit n - o for every offset
// o > 0 (offsets outside [0, n] are ignored, so broken preconditions never write out of
// range).  A thread per offset; lanes on the same 32-bit word (neighbours, the offsets being
// sorted) OR their bits together and the first of them sets them with one atomic OR (order-
// free, so the bitmap does not depend on timing).
__global__ __launch_bounds__(256) void k_mark_heads(const int64_t* __restrict__ offs,
                                                    int64_t nseg, int64_t n, int rev,
                                                    uint32_t* __restrict__ bits) {
    const int lane = threadIdx.x & 63;
    for (int64_t k0 = (int64_t)blockIdx.x * blockDim.x; k0 <= nseg;
         k0 += (int64_t)gridDim.x * blockDim.x) {
        const int64_t k = k0 + threadIdx.x;
        int64_t f = -1;
        if (k <= nseg) {
            const int64_t o = offs[k];
            if (!rev) {
                if (o >= 0 && o < n) f = o;
            } else {
                if (o > 0 && o <= n) f = n - o;
            }
        }
        const int64_t w = f >= 0 ? (f >> 5) : -1;
        uint32_t m = f >= 0 ? (1u << (f & 31)) : 0u;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t mo = __shfl_down(m, d, 64);
            const int64_t wo = __shfl_down(w, d, 64);
            if (lane + d < 64 && wo == w) m |= mo;
        }
        const int64_t wp = __shfl_up(w, 1, 64);
        if (w >= 0 && (lane == 0 || wp != w)) atomicOr(&bits[w], m);
    }
}

__global__ void k_copy_error(const uint32_t* err, int32_t* out) {
    out[0] = (int32_t)(err[0] != 0u);
}

__global__ void k_zero_words(uint64_t* p, int64_t nwords) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0ull;
}

}  // namespace
}  // namespace det
