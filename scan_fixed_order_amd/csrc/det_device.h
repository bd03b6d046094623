// det_device.h -- device helpers shared by the gfx950 kernels of the library.
//
// Cross-lane moves are plain permutations (DPP, ds_swizzle, ds_bpermute, readlane): they
// copy bits and never add, so the only arithmetic is the explicit IEEE additions written in
// the kernels, in the order those kernels state.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace det {

constexpr int kWave = 64;

// Identity of the association order: -0.0 + a == a for every a (including +0.0).
template <typename T>
__device__ __forceinline__ T ident() {
    return T(-0.0);
}

// ---------------------------------------------------------------- lane permutations

// DPP controls (gfx9 encoding)
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppQuadRev = 0x1B;    // quad_perm [3,2,1,0]
constexpr int kDppRowMirror = 0x140; // lane i of a row of 16 reads lane 15 - i
constexpr int kDppHalfMirror = 0x141;// lane i of a half row of 8 reads lane 7 - i

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}

template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
    int lo = dpp_i<CTRL>(__double2loint(v));
    int hi = dpp_i<CTRL>(__double2hiint(v));
    return __hiloint2double(hi, lo);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)dpp_i<CTRL>((int)v);
}

// ds_swizzle in bit mode: lane i reads lane ((i & and) | or) ^ xor within 32 lanes
template <int PATTERN>
__device__ __forceinline__ int swz_i(int v) {
    return __builtin_amdgcn_ds_swizzle(v, PATTERN);
}
constexpr int kSwzXor16 = (0x10 << 10) | 0x1F;

__device__ __forceinline__ float swz_xor16(float v) {
    return __int_as_float(swz_i<kSwzXor16>(__float_as_int(v)));
}
__device__ __forceinline__ double swz_xor16(double v) {
    int lo = swz_i<kSwzXor16>(__double2loint(v));
    int hi = swz_i<kSwzXor16>(__double2hiint(v));
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ uint32_t swz_xor16(uint32_t v) {
    return (uint32_t)swz_i<kSwzXor16>((int)v);
}

// value of lane `src` (uniform result)
__device__ __forceinline__ float readlane(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}
__device__ __forceinline__ double readlane(double v, int src) {
    int lo = __builtin_amdgcn_readlane(__double2loint(v), src);
    int hi = __builtin_amdgcn_readlane(__double2hiint(v), src);
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ uint32_t readlane(uint32_t v, int src) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, src);
}

// lane l reads lane (l - d) (lanes below d read an unspecified lane; callers mask them)
__device__ __forceinline__ float shfl_up(float v, int d, int lane) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane - d) << 2, __float_as_int(v)));
}
__device__ __forceinline__ double shfl_up(double v, int d, int lane) {
    int a = (lane - d) << 2;
    int lo = __builtin_amdgcn_ds_bpermute(a, __double2loint(v));
    int hi = __builtin_amdgcn_ds_bpermute(a, __double2hiint(v));
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ uint32_t shfl_up(uint32_t v, int d, int lane) {
    return (uint32_t)__builtin_amdgcn_ds_bpermute((lane - d) << 2, (int)v);
}

// partner value for the butterfly level with lane mask m (lane l reads lane l ^ m)
template <int M, typename V>
__device__ __forceinline__ V xor_partner(V v) {
    if constexpr (M == 1) {
        return dpp<kDppQuadXor1>(v);
    } else if constexpr (M == 2) {
        return dpp<kDppQuadXor2>(v);
    } else if constexpr (M == 4) {
        return dpp<kDppQuadRev>(dpp<kDppHalfMirror>(v));   // (l ^ 7) ^ 3 = l ^ 4
    } else if constexpr (M == 8) {
        return dpp<kDppHalfMirror>(dpp<kDppRowMirror>(v)); // (l ^ 7) ^ 15 = l ^ 8
    } else {
        static_assert(M == 16, "xor partner mask");
        return swz_xor16(v);
    }
}

// ---------------------------------------------------------------- pairwise trees

// PW over the 64 lanes of the wave (leaf l = lane l): adjacent lanes pair first, then
// aligned pairs of pairs, ... (xor butterfly); returns the root, uniform over the wave.
template <typename T>
__device__ __forceinline__ T wave_pw(T v) {
    v = v + xor_partner<1>(v);
    v = v + xor_partner<2>(v);
    v = v + xor_partner<4>(v);
    v = v + xor_partner<8>(v);
    v = v + xor_partner<16>(v);
    return readlane(v, 0) + readlane(v, 32);
}

}  // namespace det
