// baselines.hip -- NON-deterministic reference kernels, built into libdet_baselines.so for the
// benchmark only (not part of det.h).  They show what the deterministic library replaces:
//
//  detbase_atomic_sum      grid-stride partial sums, a shared-memory tree per block, then one
//                          float atomicAdd per block into the total: the arrival order of the
//                          blocks picks the bracketing (course page "Floating point and
//                          reproducibility", the atomic-tail kernel).
//  detbase_atomic_scatter  one float atomicAdd per element into out[index[i]] (Warp
//                          "Deterministic Execution", "Performance", the accumulation kernel).
//  detbase_dlb_scan        single-pass decoupled look-back that folds predecessors until it
//                          meets one already marked inclusive, so the bracketing depends on
//                          which states it observed (drjit-core pull request "Make CUDA
//                          floating-point prefix sums deterministic", "Root cause").
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

template <typename T>
__global__ void k_zero1(T* p) {
    p[0] = T(0);
}

template <typename T>
__global__ __launch_bounds__(256) void k_atomic_sum(const T* __restrict__ x, int64_t n, T* out) {
    __shared__ T s[256];
    T acc = T(0);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        acc += x[i];
    s[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) s[threadIdx.x] += s[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) atomicAdd(out, s[0]);
}

template <typename T>
__global__ __launch_bounds__(256) void k_atomic_scatter(const T* __restrict__ v,
                                                        const int32_t* __restrict__ idx, int64_t n,
                                                        T* out, int64_t B) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int32_t b = idx[i];
        if (b >= 0 && b < B) atomicAdd(out + b, v[i]);
    }
}

// ---- adaptive decoupled look-back scan (tile = 256 threads x 16 elements)
constexpr int kIt = 16;
constexpr int kTile = 256 * kIt;

__global__ void k_zero_u64(uint64_t* p, int64_t nw) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nw;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// status word: bits 62..63 = state (0 none, 1 aggregate, 2 inclusive), low 32 = f32 bits
__global__ __launch_bounds__(256) void k_dlb_scan_f32(const float* __restrict__ x,
                                                      float* __restrict__ y, int64_t n,
                                                      uint64_t* status, uint32_t* ticket,
                                                      int ntiles) {
    __shared__ float s_w[4];
    __shared__ float s_excl;
    __shared__ int s_tile;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) s_tile = (int)atomicAdd(ticket, 1u);
    __syncthreads();
    const int j = s_tile;
    if (j >= ntiles) return;
    const int64_t base = (int64_t)j * kTile + (int64_t)tid * kIt;
    float v[kIt];
    float run = 0.f;
#pragma unroll
    for (int k = 0; k < kIt; ++k) {
        v[k] = (base + k < n) ? x[base + k] : 0.f;
        run += v[k];
        v[k] = run;
    }
    float inc = run;
    for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(inc, d, 64);
        if (lane >= d) inc += o;
    }
    if (lane == 63) s_w[wave] = inc;
    __syncthreads();
    float wpre = 0.f, agg = 0.f;
    for (int w = 0; w < 4; ++w) {
        if (w < wave) wpre += s_w[w];
        agg += s_w[w];
    }
    if (wave == 0) {
        if (lane == 0) {
            const uint64_t st = (j == 0 ? 2ull : 1ull) << 62;
            __hip_atomic_store(status + j, st | __float_as_uint(agg), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        float excl = 0.f;
        int64_t look = (int64_t)j - 1;
        while (look >= 0) {
            const int64_t k = look - lane;
            uint64_t w = 0;
            if (k >= 0) {
                uint32_t spins = 0;
                do {
                    w = __hip_atomic_load(status + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } while ((w >> 62) == 0 && ++spins < (1u << 26));
            } else {
                w = 2ull << 62;   // before the array: an inclusive zero
            }
            const bool incl = (w >> 62) == 2;
            const uint64_t im = __ballot(incl);
            const int stop = im ? __ffsll((long long)im) - 1 : 64;
            float val = (lane <= stop && lane < 64) ? __uint_as_float((uint32_t)w) : 0.f;
            if (k < 0) val = 0.f;
            for (int m = 32; m > 0; m >>= 1) val += __shfl_xor(val, m, 64);
            excl += val;
            if (im) break;
            look -= 64;
        }
        if (lane == 0) {
            __hip_atomic_store(status + j, (2ull << 62) | __float_as_uint(excl + agg), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            s_excl = excl;
        }
    }
    __syncthreads();
    float lex = __shfl_up(inc, 1, 64);
    if (lane == 0) lex = 0.f;
    const float pre = (s_excl + wpre) + lex;
#pragma unroll
    for (int k = 0; k < kIt; ++k)
        if (base + k < n) y[base + k] = pre + v[k];
}

}  // namespace

extern "C" {

int detbase_atomic_sum(const void* x, int64_t n, int dtype, void* out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    int64_t g = (n + 255) / 256;
    if (g > 1024) g = 1024;
    if (g < 1) g = 1;
    if (dtype == 0) {
        k_zero1<float><<<1, 1, 0, s>>>(static_cast<float*>(out));
        k_atomic_sum<float><<<(unsigned)g, 256, 0, s>>>(static_cast<const float*>(x), n,
                                                        static_cast<float*>(out));
    } else {
        k_zero1<double><<<1, 1, 0, s>>>(static_cast<double*>(out));
        k_atomic_sum<double><<<(unsigned)g, 256, 0, s>>>(static_cast<const double*>(x), n,
                                                         static_cast<double*>(out));
    }
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

int detbase_atomic_scatter(const void* v, const int32_t* idx, int64_t n, int dtype, void* out,
                           int64_t num_out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    int64_t g = (n + 255) / 256;
    if (g > 65536) g = 65536;
    if (g < 1) g = 1;
    if (dtype == 0)
        k_atomic_scatter<float><<<(unsigned)g, 256, 0, s>>>(static_cast<const float*>(v), idx, n,
                                                            static_cast<float*>(out), num_out);
    else
        k_atomic_scatter<double><<<(unsigned)g, 256, 0, s>>>(static_cast<const double*>(v), idx, n,
                                                             static_cast<double*>(out), num_out);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

size_t detbase_dlb_scan_workspace_size(int64_t n) {
    const int64_t nt = (n + kTile - 1) / kTile;
    return 256 + (size_t)nt * 8;
}

// f32 inclusive forward scan only
int detbase_dlb_scan(const float* x, float* y, int64_t n, void* ws, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n <= 0) return 0;
    const int64_t nt = (n + kTile - 1) / kTile;
    const int64_t words = (int64_t)(detbase_dlb_scan_workspace_size(n) / 8);
    int zg = (int)((words + 255) / 256);
    if (zg > 1024) zg = 1024;
    k_zero_u64<<<zg, 256, 0, s>>>(static_cast<uint64_t*>(ws), words);
    uint32_t* ticket = static_cast<uint32_t*>(ws);
    uint64_t* status = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + 256);
    k_dlb_scan_f32<<<(unsigned)nt, 256, 0, s>>>(x, y, n, status, ticket, (int)nt);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
