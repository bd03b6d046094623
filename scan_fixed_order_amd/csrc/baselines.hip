// baselines.hip -- NON-deterministic reference kernels, built into libdet_baselines.so for the
// benchmark only (not part of det.h).  They show what the deterministic library replaces, each
// written to run near this GPU's bandwidth so the overhead figures are fair:
//
//  detbase_atomic_sum      16-byte grid-stride loads, a butterfly per wave and an LDS step per
//                          workgroup, then one hardware float atomic add per workgroup into the
//                          total: the arrival order of the workgroups picks the bracketing
//                          (course page "Floating point and reproducibility", the atomic-tail
//                          kernel).
//  detbase_atomic_scatter  one hardware float atomic add per element into out[index[i]]
//                          (Warp "Deterministic Execution", "Performance", the accumulation
//                          kernel with ordinary atomics).
//  detbase_lib_scan        the ROCm library scan (hipCUB DeviceScan::InclusiveSum over rocPRIM's
//                          single-pass look-back), the call a user makes without this library;
//                          its float bracketing follows which predecessor states a block saw
//                          (drjit-core pull request "Make CUDA floating-point prefix sums
//                          deterministic", "Root cause").
#include <hip/hip_runtime.h>
#include <hipcub/hipcub.hpp>
#include <stdint.h>

namespace {

template <typename T>
__global__ void k_zero1(T* p) {
    p[0] = T(0);
}

template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
    typedef float4 type;
    static constexpr int n = 4;
    static __device__ __forceinline__ float sum(const float4& v) { return (v.x + v.y) + (v.z + v.w); }
};
template <>
struct Vec16<double> {
    typedef double2 type;
    static constexpr int n = 2;
    static __device__ __forceinline__ double sum(const double2& v) { return v.x + v.y; }
};

template <typename T>
__global__ __launch_bounds__(256) void k_atomic_sum(const T* __restrict__ x, int64_t n, T* out) {
    typedef typename Vec16<T>::type V;
    constexpr int E = Vec16<T>::n;
    constexpr int U = 8;   // 16-byte loads per thread in flight
    __shared__ T s[4];
    T acc = T(0);
    const int64_t nv = n / E;
    const V* xv = reinterpret_cast<const V*>(x);
    const int64_t stride = (int64_t)gridDim.x * 256 * U;
    for (int64_t i0 = (int64_t)blockIdx.x * 256 * U + threadIdx.x; i0 < nv; i0 += stride) {
        V v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + (int64_t)u * 256;
            if (i < nv) v[u] = xv[i];
            else v[u] = V{};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc += Vec16<T>::sum(v[u]);
    }
    if (blockIdx.x == 0)   // the tail that is not a whole vector
        for (int64_t i = nv * E + threadIdx.x; i < n; i += 256) acc += x[i];
    for (int m = 32; m > 0; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) unsafeAtomicAdd(out, (s[0] + s[1]) + (s[2] + s[3]));
}

template <typename T>
__global__ __launch_bounds__(256) void k_atomic_scatter(const T* __restrict__ v,
                                                        const int32_t* __restrict__ idx, int64_t n,
                                                        T* out, int64_t B) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int32_t b = idx[i];
        if (b >= 0 && b < B) unsafeAtomicAdd(out + b, v[i]);
    }
}

}  // namespace

extern "C" {

// x must be 16-byte aligned (returns 1 otherwise)
int detbase_atomic_sum(const void* x, int64_t n, int dtype, void* out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((reinterpret_cast<uintptr_t>(x) & 15) != 0) return 1;
    const int64_t g = 2048;   // 8 workgroups per CU
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

// Workspace the library scan needs for n f32 elements (0 on error).
size_t detbase_lib_scan_workspace_size(int64_t n) {
    size_t bytes = 0;
    if (hipcub::DeviceScan::InclusiveSum(nullptr, bytes, static_cast<const float*>(nullptr),
                                         static_cast<float*>(nullptr), (int)n) != hipSuccess)
        return 0;
    return bytes;
}

// f32 inclusive forward scan by the library (n < 2^31)
int detbase_lib_scan(const float* x, float* y, int64_t n, void* ws, size_t ws_bytes, void* stream) {
    if (n <= 0) return 0;
    size_t bytes = ws_bytes;
    return hipcub::DeviceScan::InclusiveSum(ws, bytes, x, y, (int)n,
                                            static_cast<hipStream_t>(stream)) == hipSuccess
               ? 0
               : 5;
}

// Workspace and f64 inclusive forward scan by the library (n < 2^31)
size_t detbase_lib_scan64_workspace_size(int64_t n) {
    size_t bytes = 0;
    if (hipcub::DeviceScan::InclusiveSum(nullptr, bytes, static_cast<const double*>(nullptr),
                                         static_cast<double*>(nullptr), (int)n) != hipSuccess)
        return 0;
    return bytes;
}

int detbase_lib_scan64(const double* x, double* y, int64_t n, void* ws, size_t ws_bytes,
                       void* stream) {
    if (n <= 0) return 0;
    size_t bytes = ws_bytes;
    return hipcub::DeviceScan::InclusiveSum(ws, bytes, x, y, (int)n,
                                            static_cast<hipStream_t>(stream)) == hipSuccess
               ? 0
               : 5;
}

}  // extern "C"
