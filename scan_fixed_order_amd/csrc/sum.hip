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
//            same way until one value remains, written to *out.
#include <mutex>

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

// PW over x[base .. base + 4096) (identity past n); uniform over the wave.
template <typename T>
__device__ __forceinline__ T wave_unit(const T* __restrict__ x, int64_t base, int64_t n, int lane,
                                       bool vec) {
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

// One value per chunk of 2^chunk_log2 elements: out[c] = PW(x[c*2^chunk_log2 ...]) with
// identity past n.  Workgroups stride over chunks, so any grid gives the same values.
template <typename T>
__global__ __launch_bounds__(256) void k_sum_chunks(const T* __restrict__ x, int64_t n,
                                                    int chunk_log2, int64_t nchunks,
                                                    T* __restrict__ out) {
    __shared__ T s_wave[4];
    __shared__ T s_stack[48];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const bool vec = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
    const int64_t units_max = int64_t(1) << (chunk_log2 - kUnitLog2);
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t cbase = c << chunk_log2;
        const int64_t left = (n - cbase + (int64_t(1) << kUnitLog2) - 1) >> kUnitLog2;
        const int64_t units = left < units_max ? left : units_max;
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
        if (threadIdx.x == 0) {
            // right-nested fold of the remaining dyadic blocks, largest leftmost
            T acc = ident<T>();
            bool have = false;
            for (int lvl = 0; lvl < 48; ++lvl) {
                if ((units >> lvl) & 1) {
                    acc = have ? s_stack[lvl] + acc : s_stack[lvl];
                    have = true;
                }
            }
            out[c] = acc;
        }
        __syncthreads();
    }
}

template <typename T>
__global__ void k_write_pos_zero(T* out) {
    out[0] = T(0.0);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <typename T>
det_status sum_impl(const T* x, int64_t n, T* out, char* ws, hipStream_t s) {
    if (n == 0) {
        k_write_pos_zero<T><<<1, 1, 0, s>>>(out);
        return launch_status();
    }
    const LaunchOverride& ov = launch_override();
    const int clog2 = ov.sum_chunk_log2 ? ov.sum_chunk_log2 : kUnitLog2;
    const T* src = x;
    int64_t m = n;
    for (;;) {
        const int64_t nchunks = ceil_div(m, int64_t(1) << clog2);
        T* dst = (nchunks == 1) ? out : reinterpret_cast<T*>(ws);
        // one workgroup per chunk; the test hook sets any grid (workgroups stride over chunks)
        int64_t grid = nchunks;
        if (ov.grid_wgs > 0) grid = ov.grid_wgs;
        if (src == x) note_sum_grid(grid);
        KernelTimer kt(sizeof(T) == 4 ? "k_sum_chunks<f32>" : "k_sum_chunks<f64>", s);
        k_sum_chunks<T><<<dim3((unsigned)grid), dim3(256), (size_t)ov.extra_lds, s>>>(
            src, m, clog2, nchunks, dst);
        det_status st = launch_status();
        if (st != DET_SUCCESS || nchunks == 1) return st;
        src = dst;
        ws += round_up((size_t)nchunks * sizeof(T), 256);
        m = nchunks;
    }
}

}  // namespace

size_t sum_workspace(int64_t n, det_dtype dt) {
    // partial arrays of every level but the last, at the smallest chunk size
    size_t bytes = 0;
    int64_t m = n;
    while (m > (int64_t(1) << kUnitLog2)) {
        m = ceil_div(m, int64_t(1) << kUnitLog2);
        bytes += round_up((size_t)m * dtype_size(dt), 256);
    }
    return bytes < 256 ? 256 : bytes;
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
// call allocates.  Its size covers every n up to 2^31 - 1 in f64 (131072 first-level partials
// of 8 bytes, then 8 more).  Nothing in it needs to start at zero: each level writes every
// partial before the next level reads it.  Host code never uses the array's name as an
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
