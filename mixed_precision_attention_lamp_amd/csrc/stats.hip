// Device readback of the per-tile count of 16-bit sub-blocks.
//
// Tables 1-6 of "LampAttention: Look-Ahead Mixed-Precision FlashAttention for
// Dedicated Accelerators" report, for every run, the share of tiles with 0, 1
// and 2+ sub-blocks recomputed in 16-bit.  This kernel reduces the mask bytes
// written by the attention kernel to that histogram (0..4 per tile) plus the
// sub-block and entry counts behind the recompute fractions, so only ten
// integers cross PCIe.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"
#include "lamp.h"

namespace lamp {

namespace {

constexpr int kThreads = 256;

// Visible (query, key) pairs with queries [i0, i0 + 64) and keys [j0, j0 + w).
__device__ int64_t visible_pairs(int i0, int j0, int w, int S, int causal, int window) {
    const int i1 = min(i0 + kTileRows, S) - 1;
    const int j1 = min(j0 + w, S) - 1;
    if (i1 < i0 || j1 < j0) return 0;
    // fully visible block: no per-row walk needed
    const bool all = (!causal || j1 <= i0) && (window <= 0 || i1 - j0 < window);
    if (all) return (int64_t)(i1 - i0 + 1) * (j1 - j0 + 1);
    int64_t n = 0;
    for (int i = i0; i <= i1; ++i) {
        int hi = causal ? min(j1, i) : j1;
        int lo = window > 0 ? max(j0, i - window + 1) : j0;
        if (hi >= lo) n += hi - lo + 1;
    }
    return n;
}

__global__ void zero_stats_kernel(int64_t* stats) {
    if (threadIdx.x < LAMP_STATS_LEN) stats[threadIdx.x] = 0;
}

__device__ __forceinline__ int64_t wave_sum(int64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// One thread per (batch * head, r, t) tile.
__global__ __launch_bounds__(kThreads) void stats_kernel(const uint8_t* __restrict__ mask,
                                                         int64_t n_tiles, int nT, int S,
                                                         int causal, int window,
                                                         int64_t* __restrict__ stats) {
    int64_t local[LAMP_STATS_LEN];
#pragma unroll
    for (int k = 0; k < LAMP_STATS_LEN; ++k) local[k] = 0;
    for (int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x; idx < n_tiles;
         idx += (int64_t)gridDim.x * kThreads) {
        const uint8_t byte = mask[idx];
        if (!(byte & 0x80)) continue;
        const int t = (int)(idx % nT);
        const int r = (int)((idx / nT) % nT);
        const int nflag = __builtin_popcount(byte & 0x0F);
#pragma unroll
        for (int k = 0; k <= 4; ++k) local[k] += (nflag == k);
        local[5] += 1;
#pragma unroll
        for (int c = 0; c < kSubBlocks; ++c) {
            const int64_t n = visible_pairs(r * kTileRows, t * kTileKeys + c * kSubKeys, kSubKeys, S,
                                            causal, window);
            if (n == 0) continue;
            const bool f = (byte >> c) & 1;
            local[6] += 1;
            local[7] += f;
            local[8] += n;
            local[9] += f ? n : 0;
        }
    }
#pragma unroll
    for (int k = 0; k < LAMP_STATS_LEN; ++k) {
        const int64_t v = wave_sum(local[k]);
        if ((threadIdx.x & 63) == 0 && v != 0)
            atomicAdd(reinterpret_cast<unsigned long long*>(stats + k), (unsigned long long)v);
    }
}

}  // namespace

hipError_t launch_subblock_stats(const uint8_t* mask, int B, int Hq, int S, int causal,
                                 int window, int64_t* stats, hipStream_t st) {
    const int nT = (S + kTileKeys - 1) / kTileKeys;
    const int64_t n_tiles = (int64_t)B * Hq * nT * nT;
    hipLaunchKernelGGL(zero_stats_kernel, dim3(1), dim3(64), 0, st, stats);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int64_t blocks = (n_tiles + kThreads - 1) / kThreads;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(stats_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, mask, n_tiles,
                       nT, S, causal, window, stats);
    return hipGetLastError();
}

}  // namespace lamp
