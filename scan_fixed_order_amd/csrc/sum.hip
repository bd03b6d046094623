// sum.hip -- det_sum: the adjacent-pair tree PW over the whole array.
//
// Order (course page "Floating point and reproducibility", section "Fix the order of every
// addition": a fixed bracket over pairs replaces the atomic tail): pad x with -0.0 to a power
// of two and add adjacent pairs level by level.  Every aligned power-of-two block of x is a
// subtree of that tree, so the GPU may cut x into aligned blocks of any power-of-two size and
// combine the block values by the same rule; the block size and the grid never move a bit.
//
// Mapping on gfx950 (wave64):
//   block  = 256 consecutive elements; lane l holds x[4l .. 4l+4) (one 16-byte load for f32,
//            two for f64), adds them as (x0 + x1) + (x2 + x3), then a 6-level butterfly over
//            the 64 lanes (DPP / ds_swizzle / readlane) completes the block's subtree;
//   wave   = 16 blocks = 4096 elements, combined by a 4-level tree in registers;
//   unit   = 4 waves = 16384 elements, combined by 2 levels through LDS;
//   chunk  = 2^c units' worth of elements (c chosen by the host, default one unit), combined
//            by a binary counter (right-nested fold of the leftover dyadic blocks at the end);
//   levels = one launch writes one value per chunk; the next launch reduces those values the
//            same way until one value remains, written to *out.  When the chunk values fit
//            one chunk and number at most 1024, the launch that writes them also finishes: each
//            chunk value goes into a slot with a tag unique to the call, and the grid's last
//            workgroup, after its own chunks, waits until every slot carries the tag, reduces
//            the values (the same PW over them a next launch would take) and clears the tags.
//            Waiting picks who finishes, never the order; no workgroup waits on the waiter.
#include <atomic>
#include <chrono>
#include <mutex>
#include <random>

#include "det_device.h"
#include "det_internal.h"

namespace det {
namespace {

constexpr int kUnitLog2 = 14;               // elements per workgroup step
constexpr int kWaveUnit = 4096;             // elements per wave step (16 blocks of 256)
constexpr int kBlocksPerWave = 16;

// v[0..4) = x[i .. i+4); identity at or past n.  `full_vec`: all four in range and x
// 16-byte aligned, so one (f32) or two (f64) 16-byte loads are used, with the non-temporal
// hint (each line is read once: 2^28 f32 sums in 168 us with it on MI355X, 184 us without).
template <typename T>
__device__ __forceinline__ void load4(const T* __restrict__ x, int64_t i, int64_t n, bool full_vec,
                                      T (&v)[4]) {
    if (full_vec) {
        if constexpr (sizeof(T) == 4) {
            typedef float v4f __attribute__((ext_vector_type(4)));
            const v4f q = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(x + i));
            v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
        } else {
            typedef double v2d __attribute__((ext_vector_type(2)));
            const v2d a = __builtin_nontemporal_load(reinterpret_cast<const v2d*>(x + i));
            const v2d b = __builtin_nontemporal_load(reinterpret_cast<const v2d*>(x + i + 2));
            v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y;
        }
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (i + r < n) ? x[i + r] : ident<T>();
    }
}

// Chunk values of a finishing launch: slot c = two 64-bit words, each written by one atomic
// store and read by one atomic load at device scope, each carrying half of the call's 64-bit
// tag in its high half: word 0 = (tag >> 32) << 32 | low 32 bits of the value, word 1 =
// (tag & 0xffffffff) << 32 | high 32 bits (0 for f32).  A slot whose two halves show the tag
// holds this call's value, with no fence between writer and reader (a device-scope fence
// would write back a whole L2 per workgroup).
struct SumSlots {
    uint64_t* w;
};

// the high (tag) half of a slot word
__device__ __forceinline__ uint32_t slot_high(const uint64_t* w) {
    return __hip_atomic_load(reinterpret_cast<const uint32_t*>(w) + 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// The value of a slot already seen tagged: the low 32-bit halves of its words (the halves
// alone, so the reads take no more registers than the value)
__device__ __forceinline__ uint32_t slot_low(const uint64_t* w) {
    return __hip_atomic_load(reinterpret_cast<const uint32_t*>(w), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ T slot_value(const uint64_t* w, int64_t c) {
    if constexpr (sizeof(T) == 4) {
        return __uint_as_float(slot_low(w + 2 * c));
    } else {
        const uint64_t lo = slot_low(w + 2 * c), hi = slot_low(w + 2 * c + 1);
        return __longlong_as_double((long long)((hi << 32) | lo));
    }
}

// v[0..4) = slot values i .. i+4; identity at or past n
template <typename T>
__device__ __forceinline__ void load4(const SumSlots& x, int64_t i, int64_t n, bool, T (&v)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = (i + r < n) ? slot_value<T>(x.w, i + r) : ident<T>();
}

// PW over x[base .. base + 4096) (identity past n); uniform over the wave.  X: a T array or
// the slots of a finishing launch.
template <typename T, typename X>
__device__ __forceinline__ T wave_unit(const X& x, int64_t base, int64_t n, int lane, bool vec) {
    constexpr int G = sizeof(T) == 4 ? 16 : 8;   // blocks whose loads are in flight together
    const bool full = vec && (base + kWaveUnit <= n);
    T b[kBlocksPerWave];
#pragma unroll
    for (int g0 = 0; g0 < kBlocksPerWave; g0 += G) {
        T v[G][4];
#pragma unroll
        for (int g = 0; g < G; ++g)
            load4<T>(x, base + (int64_t)(g0 + g) * 256 + 4 * lane, n, full, v[g]);
#pragma unroll
        for (int g = 0; g < G; ++g) b[g0 + g] = wave_pw<T>((v[g][0] + v[g][1]) + (v[g][2] + v[g][3]));
    }
#pragma unroll
    for (int w = kBlocksPerWave; w > 1; w /= 2) {
#pragma unroll
        for (int i = 0; i < w / 2; ++i) b[i] = b[2 * i] + b[2 * i + 1];
    }
    return b[0];
}

// PW over x[cbase .. cbase + units * 2^14) (identity past n), in thread 0 of the workgroup:
// the units of 4 waves merged by a binary counter in LDS, then the right-nested fold of the
// leftover dyadic blocks, largest leftmost.  Every thread must call it (it holds barriers).
template <typename T, typename X>
__device__ __forceinline__ T chunk_pw(const X& x, int64_t n, int64_t cbase, int64_t units,
                                      bool vec, T* s_wave, T* s_stack) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    for (int64_t u = 0; u < units; ++u) {
        const int64_t base = cbase + (u << kUnitLog2) + (int64_t)wave * kWaveUnit;
        const T wv = (base < n) ? wave_unit<T>(x, base, n, lane, vec) : ident<T>();
        if (lane == 0) s_wave[wave] = wv;
        __syncthreads();
        if (threadIdx.x == 0) {
            // binary counter: merge with the older subtree of equal size on each carry
            T v = (s_wave[0] + s_wave[1]) + (s_wave[2] + s_wave[3]);
            int64_t k = u;
            int lvl = 0;
            while (k & 1) {
                v = s_stack[lvl] + v;
                k >>= 1;
                ++lvl;
            }
            s_stack[lvl] = v;
        }
        __syncthreads();
    }
    T acc = ident<T>();
    if (threadIdx.x == 0) {
        bool have = false;
        for (int lvl = 0; lvl < 48; ++lvl) {
            if ((units >> lvl) & 1) {
                acc = have ? s_stack[lvl] + acc : s_stack[lvl];
                have = true;
            }
        }
    }
    __syncthreads();
    return acc;
}

// Bound on the waiting workgroup's wait: the other workgroups never wait, so their slots
// are normally tagged within microseconds of their chunks; after 2 seconds of the GPU's
// constant 100 MHz clock it gives up and writes a NaN instead of the sum.
constexpr uint64_t kSumWaitTicks = 200000000ull;

// One value per chunk of 2^chunk_log2 elements: out[c] = PW(x[c*2^chunk_log2 ...]) with
// identity past n.  Workgroups stride over chunks, so any grid gives the same values.  With
// `slots` set (a finishing launch, nchunks <= kMaxFinish), the values go to the tagged slots
// and the grid's last workgroup writes *fin = PW(values[0 .. nchunks)).  At most 80 VGPRs, so
// 6 waves per SIMD stream the input (the waiting code alone would raise it to 82).
template <typename T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6))) void k_sum_chunks(const T* __restrict__ x, int64_t n,
                                                    int chunk_log2, int64_t nchunks,
                                                    T* __restrict__ out, uint64_t* slots,
                                                    uint64_t tag, T* __restrict__ fin) {
    __shared__ T s_wave[4];
    __shared__ T s_stack[48];
    const bool vec = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
    const int64_t units_max = int64_t(1) << (chunk_log2 - kUnitLog2);
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t cbase = c << chunk_log2;
        const int64_t left = (n - cbase + (int64_t(1) << kUnitLog2) - 1) >> kUnitLog2;
        const int64_t units = left < units_max ? left : units_max;
        const T v = chunk_pw<T>(x, n, cbase, units, vec, s_wave, s_stack);
        if (threadIdx.x == 0) {
            if (slots) {
                const uint64_t b = sizeof(T) == 4 ? (uint64_t)__float_as_uint((float)v)
                                                  : (uint64_t)__double_as_longlong((double)v);
                __hip_atomic_store(slots + 2 * c, (tag >> 32) << 32 | (b & 0xffffffffull),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(slots + 2 * c + 1, (tag << 32) | (b >> 32), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            } else {
                out[c] = v;
            }
        }
    }
    if (!slots || blockIdx.x != gridDim.x - 1) return;
    // the waiting workgroup: every slot tagged by this call (each thread polls 8 slots per
    // round trip), then the values' PW
    constexpr int kPoll = 8;
    bool late = false;
    for (int64_t c0 = threadIdx.x; c0 < nchunks && !late; c0 += 256 * kPoll) {
        uint64_t t0 = 0;
        uint32_t polls = 0;
        for (;;) {
            uint32_t h0[kPoll], h1[kPoll];
#pragma unroll
            for (int k = 0; k < kPoll; ++k) {
                const int64_t c = c0 + 256 * k;
                const bool in = c < nchunks;
                h0[k] = in ? slot_high(slots + 2 * c) : (uint32_t)(tag >> 32);
                h1[k] = in ? slot_high(slots + 2 * c + 1) : (uint32_t)tag;
            }
            bool ready = true;
#pragma unroll
            for (int k = 0; k < kPoll; ++k)
                ready = ready && h0[k] == (uint32_t)(tag >> 32) && h1[k] == (uint32_t)tag;
            if (ready) break;
            if ((polls++ & 255u) == 0u) {
                const uint64_t now = __builtin_amdgcn_s_memrealtime();
                if (polls == 1u) t0 = now;
                else if (now - t0 > kSumWaitTicks) { late = true; break; }
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    late = __syncthreads_or(late);
    const T v = chunk_pw<T>(SumSlots{slots}, nchunks, 0, 1, false, s_wave, s_stack);
    if (threadIdx.x == 0) *fin = late ? T(__builtin_nan("")) : v;
    // untag for the next call on this workspace (a captured graph replays the same tag): word
    // 0's tag half becomes 0, which no tag has; the barrier inside chunk_pw has ordered every
    // value load before these stores
    for (int64_t c = threadIdx.x; c < nchunks; c += 256)
        __hip_atomic_store(slots + 2 * c, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__global__ void k_write_pos_zero(T* out) {
    out[0] = T(0.0);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A different tag for every finishing launch the host enqueues (64 bits, both halves nonzero,
// so a cleared slot never matches), counting from a value drawn when the library loads, so
// that bytes a fresh workspace happens to hold match it with negligible probability.
uint64_t next_tag() {
    static std::atomic<uint64_t> t{((uint64_t)std::random_device{}() << 32) ^
                                   (uint64_t)std::random_device{}() ^
                                   (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count()};
    for (;;) {
        const uint64_t v = t.fetch_add(1, std::memory_order_relaxed);
        if ((v >> 32) != 0 && (v & 0xffffffffull) != 0) return v;
    }
}

// Workspace: the slots of a finishing launch (16 bytes per chunk value, at most kMaxFinish),
// then one array of chunk values per level before it.  Up to 1024 chunk values a launch
// finishes the sum itself: on MI355X (f32, median of isolated calls) 2^16 elements 17.0 ->
// 14.7 us, 2^20 17.5 -> 15.5 us, 2^22 21.0 -> 16.1 us, 2^24 26.3 -> 24.6 us.  With more, the
// waiting workgroup's polls take longer than a second launch (2^26 58.7 -> 60.8 us, 2^28
// 176 -> 200 us), so those sums keep two launches.
constexpr int64_t kMaxFinish = 1024;

size_t slots_bytes(int64_t n) {
    const int64_t c = ceil_div(n > 0 ? n : 1, int64_t(1) << kUnitLog2);
    return round_up((size_t)16 * (size_t)(c < kMaxFinish ? c : kMaxFinish), 256);
}

template <typename T>
det_status sum_impl(const T* x, int64_t n, T* out, char* ws, hipStream_t s) {
    if (n == 0) {
        k_write_pos_zero<T><<<1, 1, 0, s>>>(out);
        return launch_status();
    }
    const LaunchOverride& ov = launch_override();
    const int clog2 = ov.sum_chunk_log2 ? ov.sum_chunk_log2 : kUnitLog2;
    uint64_t* slots = reinterpret_cast<uint64_t*>(ws);
    ws += slots_bytes(n);
    const T* src = x;
    int64_t m = n;
    for (;;) {
        const int64_t nchunks = ceil_div(m, int64_t(1) << clog2);
        // one workgroup per chunk; the test hook sets any grid (workgroups stride over chunks)
        int64_t grid = nchunks;
        if (ov.grid_wgs > 0) grid = ov.grid_wgs;
        // the chunk values fit one chunk: this launch also finishes
        const bool finish = nchunks > 1 && nchunks <= kMaxFinish;
        T* dst = (nchunks == 1) ? out : reinterpret_cast<T*>(ws);
        if (src == x) note_sum_grid(grid);
        KernelTimer kt(sizeof(T) == 4 ? "k_sum_chunks<f32>" : "k_sum_chunks<f64>", s);
        k_sum_chunks<T><<<dim3((unsigned)grid), dim3(256), (size_t)ov.extra_lds, s>>>(
            src, m, clog2, nchunks, dst, finish ? slots : nullptr, finish ? next_tag() : 0,
            finish ? out : nullptr);
        det_status st = launch_status();
        if (st != DET_SUCCESS || nchunks == 1 || finish) return st;
        src = dst;
        ws += round_up((size_t)nchunks * sizeof(T), 256);
        m = nchunks;
    }
}

}  // namespace

size_t sum_workspace(int64_t n, det_dtype dt) {
    // the slots, then the chunk arrays of every level before the finishing one, at the
    // smallest chunk size
    size_t bytes = slots_bytes(n);
    int64_t m = n;
    while (m > (int64_t(1) << kUnitLog2)) {
        m = ceil_div(m, int64_t(1) << kUnitLog2);
        bytes += round_up((size_t)m * dtype_size(dt), 256);
    }
    return bytes;
}

det_status sum_launch(const void* x, int64_t n, det_dtype dt, void* out, void* ws, size_t ws_bytes,
                      hipStream_t s) {
    (void)ws_bytes;
    if (dt == DET_F32)
        return sum_impl<float>(static_cast<const float*>(x), n, static_cast<float*>(out),
                               static_cast<char*>(ws), s);
    return sum_impl<double>(static_cast<const double*>(x), n, static_cast<double*>(out),
                            static_cast<char*>(ws), s);
}

// ---------------------------------------------------------------- det_sum_noalloc

// The partials of det_sum_noalloc: one array per GPU, in the library's code object, so no
// call allocates.  Its size covers every n up to 2^31 - 1 in f64 (1024 slots of 16 bytes,
// 131072 first-level partials of 8 bytes, then 8 more).  Nothing in it needs to start at
// zero: each level writes every partial before the next level reads it, and a slot left by
// another call holds another tag (or none).  Host code never uses the array's name as an
// address: that is a host-side stand-in; the device address comes from hipGetSymbolAddress,
// once per device.
static __device__ __align__(256) unsigned char scratch[kSumNoAllocBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

det_status sum_noalloc_launch(const void* x, int64_t n, det_dtype dt, void* out, hipStream_t s) {
    if (sum_workspace(n, dt) > kSumNoAllocBytes) return DET_ERROR_TOO_LARGE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return DET_ERROR_LAUNCH;
    void* ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch_ptr[dev]) {
            void* p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return DET_ERROR_LAUNCH;
            g_scratch_ptr[dev] = p;
        }
        ptr = g_scratch_ptr[dev];
    }
    return sum_launch(x, n, dt, out, ptr, kSumNoAllocBytes, s);
}

}  // namespace det
