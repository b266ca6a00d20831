// Device-side helpers shared by the gfx950 kernels: element types, 16-byte
// vector conversions and wave64 cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float u32_as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t f32_as_u32(float x) { return __builtin_bit_cast(uint32_t, x); }

// Storage element traits. `E` is the element size in bytes; `to_float`
// widens the elements of one 16-byte vector to float (exact for every type);
// `store` rounds a float to the storage type.
template <int DT> struct Elem;

template <> struct Elem<PA_F32> {
    static constexpr int E = 4;
    __device__ __forceinline__ static void to_float(const u32x4& w, float* f) {
        f[0] = u32_as_f32(w.x); f[1] = u32_as_f32(w.y);
        f[2] = u32_as_f32(w.z); f[3] = u32_as_f32(w.w);
    }
    __device__ __forceinline__ static void store(void* base, size_t i, float x) {
        static_cast<float*>(base)[i] = x;
    }
};

// bfloat16 is the upper half of a binary32: widening is a 16-bit shift.
template <> struct Elem<PA_BF16> {
    static constexpr int E = 2;
    __device__ __forceinline__ static void to_float(const u32x4& w, float* f) {
        const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = u32_as_f32(v[i] << 16);
            f[2 * i + 1] = u32_as_f32(v[i] & 0xffff0000u);
        }
    }
    // Round to nearest, ties to even; NaN stays a quiet NaN of the same sign.
    __device__ __forceinline__ static uint16_t round(float x) {
        uint32_t u = f32_as_u32(x);
        if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
        u += 0x7fffu + ((u >> 16) & 1u);
        return static_cast<uint16_t>(u >> 16);
    }
    __device__ __forceinline__ static void store(void* base, size_t i, float x) {
        static_cast<uint16_t*>(base)[i] = round(x);
    }
};

template <> struct Elem<PA_F16> {
    static constexpr int E = 2;
    __device__ __forceinline__ static void to_float(const u32x4& w, float* f) {
        const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v[i] & 0xffffu)));
            f[2 * i + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v[i] >> 16)));
        }
    }
    // Round to nearest, ties to even (the conversion's own rounding).
    __device__ __forceinline__ static uint16_t round(float x) {
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
    }
    __device__ __forceinline__ static void store(void* base, size_t i, float x) {
        static_cast<_Float16*>(base)[i] = static_cast<_Float16>(x);
    }
};

// DPP lane permutations inside a row of 16 lanes.
enum : int {
    DPP_QUAD_XOR1 = 0xB1,      // quad_perm [1,0,3,2]
    DPP_QUAD_XOR2 = 0x4E,      // quad_perm [2,3,0,1]
    DPP_ROW_HALF_MIRROR = 0x141,  // lane i <- 7 - i within each 8
    DPP_ROW_MIRROR = 0x140,       // lane i <- 15 - i within each 16
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return u32_as_f32(static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(f32_as_u32(v)), CTRL, 0xf, 0xf, false)));
}

// Sum over aligned groups of W lanes (W = 8, 16, 32 or 64); every lane of the
// group receives the group sum. The first four steps stay inside a 16-lane
// DPP row; wider groups use cross-row shuffles.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(W == 8 || W == 16 || W == 32 || W == 64, "group width");
    v += dpp<DPP_QUAD_XOR1>(v);
    v += dpp<DPP_QUAD_XOR2>(v);
    v += dpp<DPP_ROW_HALF_MIRROR>(v);
    if constexpr (W >= 16) v += dpp<DPP_ROW_MIRROR>(v);
    if constexpr (W >= 32) v += __shfl_xor(v, 16);
    if constexpr (W >= 64) v += __shfl_xor(v, 32);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Which of a grid's W = gridDim.x * WPG contiguous runs of a stream wave
// `wave` of this workgroup takes, when only the first `active` runs hold
// work. Workgroup ids go to MI355X's eight XCDs in turn; each XCD takes one
// contiguous stretch of the active runs (its eighth), so that neighbouring
// work -- the KV heads of one sequence, sequences that share blocks -- is
// read through that XCD's L2. The waves an XCD has beyond its stretch take
// the ids from `active` on, so the grid's ids are still 0 .. W - 1, each
// once. A grid that is not a multiple of eight keeps the plain order.
template <int WPG>
__device__ __forceinline__ int xcd_run_id(int active, int wave) {
    constexpr int kXcds = 8;
    const int b = static_cast<int>(blockIdx.x);
    if (gridDim.x % kXcds != 0) return b * WPG + wave;
    const int per = static_cast<int>(gridDim.x) / kXcds * WPG;  // waves per XCD
    const int x = b % kXcds;                                     // this XCD
    const int l = b / kXcds * WPG + wave;                        // wave index on it
    const int r0 = x * active / kXcds, r1 = (x + 1) * active / kXcds;
    return l < r1 - r0 ? r0 + l : active + x * per - r0 + (l - (r1 - r0));
}

}  // namespace pa
