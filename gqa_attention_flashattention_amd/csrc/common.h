// common.h -- device helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Two fp32 values -> packed bf16 pair (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of x held by lane l ^ 32 (v_permlane32_swap: lanes 0-31 <-> 32-63).
__device__ __forceinline__ float xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((__lane_id() & 32) ? r[0] : r[1]);
}

// Value of x held by lane l ^ 16 (v_permlane16_swap: 16-lane rows 0 <-> 1, 2 <-> 3).
__device__ __forceinline__ float xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((__lane_id() & 16) ? r[0] : r[1]);
}

// Value of x held by lane l ^ 8 (DPP row_ror:8 rotates each 16-lane row by 8).
__device__ __forceinline__ float xor8(float x) {
    return __uint_as_float(
        __builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0x128, 0xf, 0xf, false));
}

// Work-groups are dispatched to the 8 XCDs round-robin (block b runs on XCD
// b % 8).  This remaps block ids so that each XCD receives one contiguous
// range of logical ids: XCD x gets logical ids [x*q + min(x, r), ...) where
// q = n / 8, r = n % 8.  A bijection on [0, n).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_contiguous(int bid, int n) {
    const int xcd = bid % kXcds, i = bid / kXcds;
    const int q = n / kXcds, r = n % kXcds;
    return xcd * q + min(xcd, r) + i;
}

}  // namespace gqa
