// Tile geometry, masks and LDS operand helpers shared by the gfx950
// attention kernels of the LampAttention forward pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace lamp {

// XOR swizzle of the 16-byte chunks of a staged row (NC chunks per row): the
// lanes of a lane group read consecutive rows at one logical chunk, and every
// 8 (NC = 8, 16) or 4 (NC = 4) consecutive rows of that read hit distinct LDS
// banks.  The swizzle depends on the row modulo 16 only, so operand rows
// 16 apart share one address register plus an immediate offset.
template <int NC>
__device__ __forceinline__ int swz(int row) {
    if constexpr (NC >= 16) return row & 15;
    else if constexpr (NC == 8) return row & 7;
    else return ((row >> 1) ^ (row >> 2)) & 3;
}

// Byte offset of logical chunk `chunk` of row `row` in a staged tile.
template <int RowBytes>
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * RowBytes + ((chunk ^ swz<RowBytes / 16>(row)) << 4);
}

__device__ __forceinline__ int tile_lo(int r, int window) {
    if (window <= 0) return 0;
    const int j = r * kTileRows - window + 1;
    return j <= 0 ? 0 : j / kTileKeys;
}

__device__ __forceinline__ int tile_hi(int r, int nT, int causal) {
    return causal ? min(r, nT - 1) : nT - 1;
}

__device__ __forceinline__ bool tile_visited(int r, int t, int S, int causal, int window) {
    const int i0 = r * kTileRows, i1 = min(i0 + kTileRows - 1, S - 1);
    const int j0 = t * kTileKeys, j1 = min(j0 + kTileKeys - 1, S - 1);
    if (causal && i1 < j0) return false;
    if (window > 0 && i0 - j1 > window - 1) return false;
    return true;
}

// Every (query, key) pair of the tile exists and is visible.
__device__ __forceinline__ bool tile_full(int r, int t, int S, int causal, int window) {
    const int i0 = r * kTileRows, i1 = i0 + kTileRows - 1;
    const int j0 = t * kTileKeys, j1 = j0 + kTileKeys - 1;
    if (i1 >= S || j1 >= S) return false;
    if (causal && j1 > i0) return false;
    if (window > 0 && i1 - j0 > window - 1) return false;
    return true;
}

__device__ __forceinline__ bool pair_visible(int i, int j, int S, int causal, int window) {
    return i < S && j < S && (!causal || j <= i) && (window <= 0 || i - j < window);
}

// pair_visible(i, j0 + e, ...) for e = 0..3 as bits 0..3: the visible keys of
// a run of four are one contiguous range [lo, hi) of e (clamped counts from
// the end of the sequence, the causal bound and the window), so the mask is
// a difference of two low-bit masks.
__device__ __forceinline__ uint32_t visible4(int i, int j0, int S, int causal, int window) {
    int hi = min(max(S - j0, 0), 4);
    if (causal) hi = min(hi, max(i - j0 + 1, 0));
    const int lo = window > 0 ? min(max(i - window - j0 + 1, 0), 4) : 0;
    const uint32_t m = ((1u << hi) - 1u) & ~((1u << lo) - 1u);
    return i < S ? m : 0u;
}

// Smallest fp32 a >= 0 with fl32(a * c8) >= t2: then |s| >= t2 for the
// log2-domain logit s = fl32(acc * c8) exactly when |acc| >= a (rounding is
// monotone).  0 when every logit passes, +inf when none can.
__device__ inline float acc_threshold(float t2, float c8) {
    if (!(t2 > 0.0f)) return 0.0f;
    if (t2 == __builtin_inff()) return __builtin_inff();
    float a = t2 / c8;
    if (!(a < __builtin_inff())) return __builtin_inff();
    // positive finite floats step by one ulp with their bit pattern
    for (int it = 0; it < 8 && a > 0.0f; ++it) {
        const float p = __uint_as_float(__float_as_uint(a) - 1u);
        if (p * c8 >= t2) a = p; else break;
    }
    for (int it = 0; it < 8 && !(a * c8 >= t2); ++it) a = __uint_as_float(__float_as_uint(a) + 1u);
    return a;
}

// 32 bytes of the e4m3 operand of one 128-deep FP8 step from a staged
// (swizzled) LDS tile: lane group g holds depth 32g .. 32g+31 of step s; for
// D = 64 groups 2, 3 hold zeros.
template <int D>
__device__ __forceinline__ v8i fp8_operand(const uint8_t* tile, int row, int s, int g) {
    v8i x = {0, 0, 0, 0, 0, 0, 0, 0};
    if (D >= 128 || g * 32 < D) {
        const int gg = D >= 128 ? s * 4 + g : (g & 1);
        const u32x4 lo = *reinterpret_cast<const u32x4*>(tile + lds_off<D>(row, 2 * gg));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(tile + lds_off<D>(row, 2 * gg + 1));
        x = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    return x;
}

// The same operand read from a row of a row-major global e4m3 array.
template <int D>
__device__ __forceinline__ v8i fp8_operand_global(const uint8_t* row_ptr, int s, int g) {
    v8i x = {0, 0, 0, 0, 0, 0, 0, 0};
    if (D >= 128 || g * 32 < D) {
        const int gg = D >= 128 ? s * 4 + g : (g & 1);
        const u32x4 lo = *reinterpret_cast<const u32x4*>(row_ptr + 32 * gg);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(row_ptr + 32 * gg + 16);
        x = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    return x;
}

}  // namespace lamp
