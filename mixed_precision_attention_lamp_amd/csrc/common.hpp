// Device helpers shared by the gfx950 kernels of the LampAttention forward pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lamp {

// Tile geometry ("16-bit sub-blocks per tile", tables 1-6): 64 query rows by
// 64 keys, split into four sub-blocks of 16 keys.
constexpr int kTileRows = 64;
constexpr int kTileKeys = 64;
constexpr int kSubKeys = 16;
constexpr int kSubBlocks = kTileKeys / kSubKeys;
constexpr float kE4M3Max = 448.0f;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
    return __uint_as_float(h << 16);
}

// Two fp32 values -> two e4m3fn codes in the low (hi = false) or high half of
// `old`.  Magnitudes are clamped to 448 first: any value in (448, 464) rounds
// to 448 under round-to-nearest-even, and nothing here is larger.
template <bool Hi>
__device__ __forceinline__ uint32_t cvt_pk_e4m3(float a, float b, uint32_t old) {
    a = __builtin_fminf(__builtin_fmaxf(a, -kE4M3Max), kE4M3Max);
    b = __builtin_fminf(__builtin_fmaxf(b, -kE4M3Max), kE4M3Max);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, Hi);
}

// Same without the clamp, for values known to lie in [0, 1 + 2^-20].
template <bool Hi>
__device__ __forceinline__ uint32_t cvt_pk_e4m3_unit(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, Hi);
}

// Two e4m3 codes (low or high 16 bits of w) -> two bf16 values, exact.
template <bool Hi>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    v2bf r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, Hi);
    return __builtin_bit_cast(uint32_t, r);
}

// Two e4m3 codes (low or high 16 bits of w) -> two fp32 values, exact.
template <bool Hi>
__device__ __forceinline__ v2f e4m3x2_to_f32x2(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, Hi);
}

// fp32 -> bf16, round to nearest even (hardware conversion).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    v2bf r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2 by a polynomial whose steps are each one correctly rounded fp32
// operation in a fixed order, so that any evaluation of the same steps (on a
// CPU too) gives the same bits: x is clamped at -30 (2^-30 and all below it
// round to 0 in e4m3), split as n + f with n = rint(x) (ties to even) and
// |f| <= 1/2 (exact), 2^f ~ 1 + f (c1 + f (c2 + f (c3 + f (c4 + f c5)))) by
// Horner's rule with fused multiply-adds, and the exponent n added exactly
// (the result stays normal).  c1..c5: a minimax fit of the relative error on
// [-1/2, 1/2] with the constant term 1, rounded to fp32 (within 2^-22 of 2^x).
__device__ __forceinline__ float poly_exp2(float x) {
    x = __builtin_fmaxf(x, -30.0f);
    const float n = __builtin_rintf(x);
    const float f = x - n;
    float p = __builtin_fmaf(0x1.5c10d4p-10f, f, 0x1.3cee66p-7f);
    p = __builtin_fmaf(p, f, 0x1.c6b64ep-5f);
    p = __builtin_fmaf(p, f, 0x1.ebf9aep-3f);
    p = __builtin_fmaf(p, f, 0x1.62e42ap-1f);
    p = __builtin_fmaf(p, f, 1.0f);
    return __builtin_ldexpf(p, (int)n);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations
// (lgkmcnt = 0) but not for its outstanding global loads, then s_barrier.
// (__syncthreads() also drains vmcnt, which would stall on prefetches.)
__device__ __forceinline__ void lds_barrier() {
    __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Lane mask of a predicate, kept in scalar registers.
__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Cross-lane max over the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48).  A permlane swap of a value with itself leaves each lane holding its
// own value in one result and its partner's (l^32, resp. l^16) in the other,
// in registers and without LDS.
__device__ __forceinline__ float max_over_lane_groups(float x) {
    const uint32_t b = __float_as_uint(x);
    const auto s32 = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    x = __builtin_fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    const uint32_t c = __float_as_uint(x);
    const auto s16 = __builtin_amdgcn_permlane16_swap(c, c, false, false);
    return __builtin_fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
}

}  // namespace lamp
