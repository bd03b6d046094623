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
//   C_q    carry into interval q: C_0 = -0.0, C_{q+1} = C_q + PW(all 256 Agg of interval q),
//          published only by the last tile of interval q (the anchor);
//   y      (((C_q + W_j) + P) + p) + s.
// A tile never reads an inclusive prefix of a non-anchor predecessor, so whether a
// predecessor was seen as finished or not cannot change the association order.
//
// Status slots are 64-bit words (tag << 32 | payload): tag bit 0 = ready, bit 1 = segment
// head seen; f64 payloads take two words, each carrying the tag.  Every word validates itself,
// so relaxed agent-scope atomics suffice and no fence is needed.  The slots and the tile
// ticket are cleared by a small kernel before each scan.
//
// Segmented scans run the pair operator (f1 | f2, f2 ? b : a + b) through the same dataflow;
// head flags of a tile come from a workgroup-parallel search of the offsets.  Reverse scans
// read and write through mirrored indices (n - 1 - f); exclusive scans store each inclusive
// value one position later (and +0.0 at position 0 and at segment heads).
#include "det_device.h"
#include "det_internal.h"

namespace det {
namespace {

constexpr int kV = kScanV;
constexpr int kT = kScanT;
constexpr int kA = kScanA;
constexpr int kWaveElems = kScanV * kScanW;                 // 2048
constexpr int kStage = kWaveElems + kWaveElems / 32;        // one spare LDS slot per 32
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

template <typename T>
__device__ __forceinline__ void publish(uint64_t* slot, const Seg<T>& s) {
    const uint64_t tag = (uint64_t)(kReady | (s.f ? kHeadTag : 0u)) << 32;
    if constexpr (sizeof(T) == 4) {
        __hip_atomic_store(slot, tag | __float_as_uint(s.v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
        const uint64_t b = (uint64_t)__double_as_longlong(s.v);
        __hip_atomic_store(slot, tag | (b & 0xffffffffull), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(slot + 1, tag | (b >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Spin bound: a predecessor's slot is normally ready within microseconds.  Past the bound the
// wait gives up and raises the error word, so no wave can wait forever.
constexpr uint32_t kSpinLimit = 1u << 24;

__device__ __forceinline__ uint64_t wait_word(uint64_t* w, uint32_t* err) {
    uint64_t v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t spins = 0;
    while (!((v >> 32) & kReady)) {
        if (++spins > kSpinLimit) {
            __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return v;
}

template <typename T>
__device__ __forceinline__ Seg<T> wait_slot(uint64_t* slot, uint32_t* err) {
    if constexpr (sizeof(T) == 4) {
        const uint64_t w = wait_word(slot, err);
        return Seg<T>{__uint_as_float((uint32_t)w), (uint32_t)(w >> 33) & 1u};
    } else {
        const uint64_t w0 = wait_word(slot, err);
        const uint64_t w1 = wait_word(slot + 1, err);
        const uint64_t b = (w1 << 32) | (w0 & 0xffffffffull);
        return Seg<T>{__longlong_as_double((long long)b), (uint32_t)(w0 >> 33) & 1u};
    }
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

// Bit b of s_heads marks flipped position F0 + b (b in [0, T]) as a segment head.
// Forward: heads are the offsets o < n.  Reverse: flipped position n - o for offsets o > 0
// (the last element of every non-empty segment).
__device__ void build_heads(const int64_t* __restrict__ offs, int64_t nseg, int64_t n, bool rev,
                            int64_t F0, uint32_t* s_heads, int tid) {
    for (int i = tid; i < kHeadWords; i += 256) s_heads[i] = 0u;
    int64_t lo_v, hi_v;
    if (!rev) {
        lo_v = F0;
        hi_v = (F0 + kT < n - 1) ? F0 + kT : n - 1;
    } else {
        lo_v = (n - F0 - kT > 1) ? n - F0 - kT : 1;
        hi_v = n - F0;
    }
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

template <typename T>
__device__ __forceinline__ void load_wave(const T* __restrict__ x, int64_t n, bool rev, int64_t fw,
                                          T* st, int lane) {
    const bool vec = !rev && (fw + kWaveElems <= n) &&
                     ((reinterpret_cast<uintptr_t>(x + fw) & 15) == 0);
    if (vec) {
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int r = 0; r < kWaveElems / 256; ++r) {
                const int e = r * 256 + 4 * lane;
                const float4 q = *reinterpret_cast<const float4*>(x + fw + e);
                const int a = pad(e);
                st[a] = q.x; st[a + 1] = q.y; st[a + 2] = q.z; st[a + 3] = q.w;
            }
        } else {
#pragma unroll
            for (int r = 0; r < kWaveElems / 128; ++r) {
                const int e = r * 128 + 2 * lane;
                const double2 q = *reinterpret_cast<const double2*>(x + fw + e);
                const int a = pad(e);
                st[a] = q.x; st[a + 1] = q.y;
            }
        }
    } else {
#pragma unroll 8
        for (int r = 0; r < kWaveElems / 64; ++r) {
            const int e = r * 64 + lane;
            const int64_t f = fw + e;
            st[pad(e)] = (f < n) ? x[rev ? n - 1 - f : f] : ident<T>();
        }
    }
}

template <typename T, bool SEG>
__device__ __forceinline__ void store_wave(T* __restrict__ y, int64_t n, bool rev, bool excl,
                                           int64_t F0, int64_t fw, const T* st,
                                           const uint32_t* s_heads, int lane) {
    if (!excl) {
        const bool vec = !rev && (fw + kWaveElems <= n) &&
                         ((reinterpret_cast<uintptr_t>(y + fw) & 15) == 0);
        if (vec) {
            if constexpr (sizeof(T) == 4) {
#pragma unroll
                for (int r = 0; r < kWaveElems / 256; ++r) {
                    const int e = r * 256 + 4 * lane;
                    const int a = pad(e);
                    *reinterpret_cast<float4*>(y + fw + e) =
                        make_float4(st[a], st[a + 1], st[a + 2], st[a + 3]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < kWaveElems / 128; ++r) {
                    const int e = r * 128 + 2 * lane;
                    const int a = pad(e);
                    *reinterpret_cast<double2*>(y + fw + e) = make_double2(st[a], st[a + 1]);
                }
            }
        } else {
#pragma unroll 8
            for (int r = 0; r < kWaveElems / 64; ++r) {
                const int e = r * 64 + lane;
                const int64_t f = fw + e;
                if (f < n) y[rev ? n - 1 - f : f] = st[pad(e)];
            }
        }
    } else {
        // inclusive value of position f goes to position f + 1; +0.0 at segment heads
#pragma unroll 8
        for (int r = 0; r < kWaveElems / 64; ++r) {
            const int e = r * 64 + lane;
            const int64_t f = fw + e + 1;
            if (f < n) {
                T v = st[pad(e)];
                if constexpr (SEG) {
                    const int bit = (int)(f - F0);
                    if ((s_heads[bit >> 5] >> (bit & 31)) & 1u) v = T(0.0);
                }
                y[rev ? n - 1 - f : f] = v;
            }
        }
    }
}

// ---------------------------------------------------------------- the kernel

template <typename T>
struct ScanArgs {
    const T* x;
    T* y;
    int64_t n;
    const int64_t* offs;
    int64_t nseg;
    uint64_t* agg;       // slot_words<T>() words per tile
    uint64_t* carry;     // slot_words<T>() words per interval boundary
    uint32_t* ticket;    // [0] tile ticket, [1] error word (a wait hit the spin bound)
    int ntiles;
    int rev;
    int excl;
};

template <typename T, bool SEG>
__global__ __launch_bounds__(256) void k_scan(ScanArgs<T> a) {
    __shared__ T s_stage[kScanWaves][kStage];
    __shared__ uint32_t s_heads[SEG ? kHeadWords : 1];
    __shared__ Seg<T> s_tmp[kScanWaves];
    __shared__ Seg<T> s_wtot[kScanWaves];
    __shared__ Seg<T> s_carry;
    __shared__ int s_tile;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    constexpr int SW = slot_words<T>();
    const bool rev = a.rev != 0;

    for (;;) {
        if (tid == 0)
            s_tile = (int)__hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int j = s_tile;
        if (j >= a.ntiles) break;
        const int64_t F0 = (int64_t)j * kT;
        const int64_t fw = F0 + (int64_t)wave * kWaveElems;
        T* st = s_stage[wave];

        if constexpr (SEG) build_heads(a.offs, a.nseg, a.n, rev, F0, s_heads, tid);

        // ---- load the wave's 2048 elements, then each lane takes its run of 32
        load_wave<T>(a.x, a.n, rev, fw, st, lane);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        T r[kV];
#pragma unroll
        for (int k = 0; k < kV; ++k) r[k] = st[lane * 33 + k];
        const uint32_t hb = SEG ? s_heads[wave * 64 + lane] : 0u;

        // ---- lane-serial prefix
#pragma unroll
        for (int k = 1; k < kV; ++k) {
            if (SEG && ((hb >> k) & 1u)) continue;
            r[k] = r[k - 1] + r[k];
        }
        Seg<T> u{r[kV - 1], hb != 0u ? 1u : 0u};

        // ---- Kogge-Stone over the lane totals of the wave
#pragma unroll
        for (int d = 1; d < 64; d *= 2) {
            Seg<T> o{shfl_up(u.v, d, lane), SEG ? shfl_up(u.f, d, lane) : 0u};
            if (lane >= d) u = op<SEG>(o, u);
        }
        Seg<T> p{shfl_up(u.v, 1, lane), SEG ? shfl_up(u.f, 1, lane) : 0u};
        if (lane == 0) p = seg_ident<T>();

        // ---- Kogge-Stone over the 4 wave totals
        if (lane == 63) s_wtot[wave] = u;
        __syncthreads();
        const Seg<T> w0 = s_wtot[0], w1 = s_wtot[1], w2 = s_wtot[2], w3 = s_wtot[3];
        const Seg<T> o1 = op<SEG>(w0, w1), o2 = op<SEG>(w1, w2), o3 = op<SEG>(w2, w3);
        const Seg<T> om1 = o1, om2 = op<SEG>(w0, o2), om3 = op<SEG>(o1, o3);
        const Seg<T> P = wave == 0 ? seg_ident<T>() : wave == 1 ? w0 : wave == 2 ? om1 : om2;
        const Seg<T> agg = om3;

        // ---- publish this tile's total
        if (tid == 0) publish<T>(a.agg + (size_t)j * SW, agg);

        // ---- look-back inside the anchor interval
        const int q = j / kA;
        const int cnt = j - q * kA;
        Seg<T> mine = seg_ident<T>();
        if (tid < cnt) mine = wait_slot<T>(a.agg + (size_t)(q * kA + tid) * SW, a.ticket + 1);
        const Seg<T> Wj = block_pw<SEG, T>(mine, lane, wave, s_tmp);
        const bool anchor = (cnt == kA - 1) && (j + 1 < a.ntiles);
        Seg<T> G = seg_ident<T>();
        if (anchor) G = block_pw<SEG, T>(tid == kA - 1 ? agg : mine, lane, wave, s_tmp);

        // ---- carry into the interval; the anchor forwards the next one
        if (tid == 0) {
            const Seg<T> C = (q == 0) ? seg_ident<T>() : wait_slot<T>(a.carry + (size_t)q * SW, a.ticket + 1);
            if (anchor) publish<T>(a.carry + (size_t)(q + 1) * SW, op<SEG>(C, G));
            s_carry = C;
        }
        __syncthreads();
        const Seg<T> E = op<SEG>(s_carry, Wj);
        const Seg<T> X = op<SEG>(op<SEG>(E, P), p);

        // ---- combine and stage the results
#pragma unroll
        for (int k = 0; k < kV; ++k) {
            if constexpr (SEG) {
                const uint32_t upto = (k == 31) ? hb : (hb & ((2u << k) - 1u));
                if (!upto) r[k] = X.v + r[k];
            } else {
                r[k] = X.v + r[k];
            }
            st[lane * 33 + k] = r[k];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        store_wave<T, SEG>(a.y, a.n, rev, a.excl != 0, F0, fw, st, s_heads, lane);
        if (a.excl && j == 0 && tid == 0) a.y[rev ? a.n - 1 : 0] = T(0.0);
        __syncthreads();
    }
}

__global__ void k_zero_words(uint64_t* p, int64_t nwords) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0ull;
}

struct Layout {
    int64_t ntiles, nq;
    size_t agg_off, carry_off, total;
};

Layout layout(int64_t n, det_dtype dt) {
    Layout L;
    const size_t sw = dt == DET_F64 ? 2 : 1;
    L.ntiles = (n + kT - 1) / kT;
    L.nq = (L.ntiles + kA - 1) / kA;
    L.agg_off = 256;
    L.carry_off = L.agg_off + round_up((size_t)L.ntiles * sw * 8, 256);
    L.total = L.carry_off + round_up((size_t)(L.nq + 1) * sw * 8, 256);
    return L;
}

template <typename T>
det_status scan_impl(const T* x, T* y, int64_t n, unsigned flags, const int64_t* offs,
                     int64_t nseg, char* ws, hipStream_t s) {
    if (n == 0) return DET_SUCCESS;
    const Layout L = layout(n, sizeof(T) == 8 ? DET_F64 : DET_F32);
    const int64_t words = (int64_t)(L.total / 8);
    int zg = (int)((words + 255) / 256);
    if (zg > 1024) zg = 1024;
    k_zero_words<<<zg, 256, 0, s>>>(reinterpret_cast<uint64_t*>(ws), words);
    det_status st = launch_status();
    if (st != DET_SUCCESS) return st;
    ScanArgs<T> a;
    a.x = x;
    a.y = y;
    a.n = n;
    a.offs = offs;
    a.nseg = nseg;
    a.agg = reinterpret_cast<uint64_t*>(ws + L.agg_off);
    a.carry = reinterpret_cast<uint64_t*>(ws + L.carry_off);
    a.ticket = reinterpret_cast<uint32_t*>(ws);
    a.ntiles = (int)L.ntiles;
    a.rev = (flags & DET_SCAN_REVERSE) ? 1 : 0;
    a.excl = (flags & DET_SCAN_EXCLUSIVE) ? 1 : 0;
    int64_t grid = L.ntiles;
    const LaunchOverride& ov = launch_override();
    if (ov.grid_wgs > 0 && grid > ov.grid_wgs) grid = ov.grid_wgs;
    if (offs)
        k_scan<T, true><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
    else
        k_scan<T, false><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
    return launch_status();
}

}  // namespace

size_t scan_workspace(int64_t n, det_dtype dt, unsigned flags, int64_t num_segments) {
    (void)flags;
    (void)num_segments;
    return layout(n, dt).total;
}

det_status scan_launch(const void* x, void* y, int64_t n, det_dtype dt, unsigned flags,
                       const int64_t* offs, int64_t nseg, void* ws, size_t ws_bytes,
                       hipStream_t s) {
    (void)ws_bytes;
    if (dt == DET_F32)
        return scan_impl<float>(static_cast<const float*>(x), static_cast<float*>(y), n, flags,
                                offs, nseg, static_cast<char*>(ws), s);
    return scan_impl<double>(static_cast<const double*>(x), static_cast<double*>(y), n, flags,
                             offs, nseg, static_cast<char*>(ws), s);
}

}  // namespace det
