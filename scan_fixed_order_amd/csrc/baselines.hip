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
//  detbase_adaptive_scan   det_scan's own look-back kernel with the anchors replaced by the
//                          classic adaptive look-back (the nearest predecessor's inclusive
//                          prefix when it is ready): the same tiles, loads, local step,
//                          pipeline and readout, so t_det / t_adaptive - 1 is what the fixed
//                          anchors cost (that pull request's "Microbenchmark" compares the
//                          same two kernels).  Every mode, segmented too.
//  detbase_stream_read, detbase_copy
//                          a plain streaming read and a plain copy with 16-byte non-temporal
//                          accesses: what this GPU's HBM delivers to a simple kernel.
#include <hip/hip_runtime.h>
#include <hipcub/hipcub.hpp>
#include <stdint.h>

#include <mutex>

#include "scan_kernels.h"

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

// ---------------------------------------------------------------- bandwidth probes

typedef float f32x4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_stream_read(const f32x4v* __restrict__ x, int64_t nv,
                                                     float* __restrict__ sink) {
    float acc = 0.f;
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < nv; i += 4 * stride) {
        const f32x4v a = __builtin_nontemporal_load(x + i);
        const f32x4v b = __builtin_nontemporal_load(x + i + stride);
        const f32x4v c = __builtin_nontemporal_load(x + i + 2 * stride);
        const f32x4v d = __builtin_nontemporal_load(x + i + 3 * stride);
        acc += (a.x + b.y) + (c.z + d.w);
    }
    for (; i < nv; i += stride) acc += __builtin_nontemporal_load(x + i).x;
    if (acc == 1234.5f) sink[blockIdx.x] = acc;   // keeps the loads; never true for the probe's data
}

__global__ __launch_bounds__(256) void k_copy16(const f32x4v* __restrict__ x,
                                                f32x4v* __restrict__ y, int64_t nv) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nv; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(x + i), y + i);
}

// ---------------------------------------------------------------- adaptive look-back scan

constexpr size_t kBErr = (size_t)(det::kCounters * det::kCounterStride * 4);
constexpr size_t kBDummy = kBErr + 256;
constexpr size_t kBHeader = kBDummy + 256;

size_t rup(size_t v) { return (v + 255) / 256 * 256; }

struct BLayout {
    int64_t ntiles;
    size_t agg, incl, hb, total;
};

BLayout blayout(int64_t n, int dtype, bool seg) {
    BLayout L;
    const size_t sw = dtype == 1 ? 2 : 1;
    L.ntiles = (n + det::kScanT - 1) / det::kScanT;
    L.agg = kBHeader;
    L.incl = L.agg + rup((size_t)L.ntiles * sw * 8);
    L.hb = L.incl + rup((size_t)L.ntiles * sw * 8);
    L.total = L.hb + (seg ? rup(((size_t)L.ntiles * (det::kScanT / 32) + 1) * 4) : 0);
    return L;
}

int64_t resident(const void* fn, int* cus_out) {
    static std::mutex mu;
    static const void* fns[64];
    static int64_t vals[64];
    static int used = 0, cus = 0;
    std::lock_guard<std::mutex> lock(mu);
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
    }
    *cus_out = cus;
    for (int i = 0; i < used; ++i)
        if (fns[i] == fn) return vals[i];
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess) return 0;
    const int64_t r = (int64_t)(per_cu < 1 ? 1 : per_cu) * cus;
    if (used < 64) {
        fns[used] = fn;
        vals[used++] = r;
    }
    return r;
}

template <typename T, bool NT>
const void* adaptive_fn(int mode) {
    using det::k_scan;
    switch (mode) {
        case 0: return (const void*)k_scan<T, false, false, false, NT, true>;
        case 1: return (const void*)k_scan<T, false, false, true, NT, true>;
        case 2: return (const void*)k_scan<T, false, true, false, NT, true>;
        case 3: return (const void*)k_scan<T, false, true, true, NT, true>;
        case 4: return (const void*)k_scan<T, true, false, false, NT, true>;
        case 5: return (const void*)k_scan<T, true, false, true, NT, true>;
        case 6: return (const void*)k_scan<T, true, true, false, NT, true>;
        default: return (const void*)k_scan<T, true, true, true, NT, true>;
    }
}

template <typename T>
int adaptive_scan(const T* x, T* y, int64_t n, unsigned flags, const int64_t* offs, int64_t nseg,
                  char* ws, hipStream_t s) {
    if (n <= 0) return 0;
    const bool seg = offs != nullptr;
    const BLayout L = blayout(n, sizeof(T) == 8 ? 1 : 0, seg);
    const int64_t words = (int64_t)(L.total / 8);
    int zg = (int)((words + 255) / 256);
    if (zg > 1024) zg = 1024;
    det::k_zero_words<<<zg, 256, 0, s>>>(reinterpret_cast<uint64_t*>(ws), words);
    const bool rev = (flags & 2u) != 0, excl = (flags & 1u) != 0;
    if (seg) {
        int64_t g = (nseg + 1 + 255) / 256;
        if (g > 16384) g = 16384;
        det::k_mark_heads<<<(unsigned)g, 256, 0, s>>>(offs, nseg, n, rev ? 1 : 0,
                                                      reinterpret_cast<uint32_t*>(ws + L.hb));
    }
    det::ScanArgs<T> a{};
    a.x = x;
    a.y = y;
    a.n = n;
    a.offs = offs;
    a.nseg = nseg;
    a.agg = reinterpret_cast<uint64_t*>(ws + L.agg);
    a.gtot = reinterpret_cast<uint64_t*>(ws + L.incl);
    a.carry = a.agg;   // unused by the adaptive look-back
    a.ticket = reinterpret_cast<uint32_t*>(ws);
    a.err = reinterpret_cast<uint32_t*>(ws + kBErr);
    a.dummy = reinterpret_cast<const T*>(ws + kBDummy);
    a.hbits = seg ? reinterpret_cast<const uint32_t*>(ws + L.hb) : nullptr;
    a.ntiles = (int)L.ntiles;
    a.rev = rev ? 1 : 0;
    a.excl = excl ? 1 : 0;
    a.A = det::kScanA;
    a.A2 = det::kScanA2;
    const int mode = (seg ? 4 : 0) | (rev ? 2 : 0) | (excl ? 1 : 0);
    const bool nt = (uint64_t)n * sizeof(T) >= (512ull << 20);
    const void* fn = nt ? adaptive_fn<T, true>(mode) : adaptive_fn<T, false>(mode);
    int cus = 0;
    const int64_t res = resident(fn, &cus);
    if (res <= 0) return 5;
    int64_t grid = res;
    if (grid > 3 * (int64_t)cus) grid = 3 * (int64_t)cus;   // as det_scan
    if (grid > L.ntiles) grid = L.ntiles;
    int64_t nc = grid < det::kCounters ? grid : det::kCounters;
    if (nc > res) nc = res;
    a.nctr = (int)nc;
    void* args[] = {&a};
    if (hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, s) != hipSuccess) return 5;
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // namespace

extern "C" {

// Bytes of workspace detbase_adaptive_scan needs (dtype 0 = f32, 1 = f64).
size_t detbase_adaptive_scan_workspace_size(int64_t n, int dtype, int64_t num_segments) {
    return blayout(n > 0 ? n : 1, dtype, num_segments > 0).total;
}

// Prefix sum through det_scan's kernel with the adaptive look-back (flags: 1 exclusive,
// 2 reverse; offs: NULL or int64 [num_segments + 1] on the device).  Not reproducible.
int detbase_adaptive_scan(const void* x, void* y, int64_t n, int dtype, unsigned flags,
                          const int64_t* offs, int64_t num_segments, void* ws, size_t ws_bytes,
                          void* stream) {
    if (ws_bytes < detbase_adaptive_scan_workspace_size(n, dtype, offs ? num_segments : 0))
        return 4;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == 0)
        return adaptive_scan<float>(static_cast<const float*>(x), static_cast<float*>(y), n,
                                    flags, offs, num_segments, static_cast<char*>(ws), s);
    return adaptive_scan<double>(static_cast<const double*>(x), static_cast<double*>(y), n,
                                 flags, offs, num_segments, static_cast<char*>(ws), s);
}

// Streaming read of nbytes (a multiple of 16, 16-byte aligned x) by 4096 workgroups.
int detbase_stream_read(const void* x, int64_t nbytes, void* sink, void* stream) {
    k_stream_read<<<4096, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const f32x4v*>(x), nbytes / 16, static_cast<float*>(sink));
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

// Copy of nbytes (a multiple of 16, both 16-byte aligned) by 4096 workgroups.
int detbase_copy(const void* x, void* y, int64_t nbytes, void* stream) {
    k_copy16<<<4096, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const f32x4v*>(x), static_cast<f32x4v*>(y), nbytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

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
