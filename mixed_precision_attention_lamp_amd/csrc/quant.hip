// Quantisation pass of the LampAttention forward pass on gfx950.
//
// "LampAttention: Look-Ahead Mixed-Precision FlashAttention for Dedicated
// Accelerators" (abstract) accumulates key-query products in an 8-bit format.
// Here Q and K are quantised to e4m3fn with one scale per (batch, head):
// scale = fl32(amax / 448), codes = E4M3(fl32(x * fl32(448 / amax))).  The pass
// is bound by HBM bandwidth: each bf16 value is read twice (amax, then
// quantise; the second read is served mostly from the last-level cache) and
// one byte is written.  V is transposed per 64-key tile here as well, so that
// the attention kernel can stage it straight into the layout of the P.V
// matrix-core operand; that transpose runs in the same launch as the amax
// reduction (both only read the inputs).
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace lamp {

namespace {

constexpr int kChunk = 16384;      // bf16 values per amax / quantise block (8 loads per thread)
// the decode step's pass over K (a few large slabs) streams faster in half the chunk
constexpr int kDecodeChunk = 8192;
constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t max_bf16_mag(u32x4 w) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m = max(m, w[i] & 0x7FFFu);
        m = max(m, (w[i] >> 16) & 0x7FFFu);
    }
    return m;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) v = max(v, red[w]);
    return v;
}

// Partial max |x| of chunk `chunk` of slab `slab` (Q heads first, then K
// heads) into partial[slab * nch + chunk].
template <int kCh>
__device__ __forceinline__ void amax_block(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                           uint32_t* __restrict__ partial, int n_q_slabs, int slab_len,
                                           int nch, int slab, int chunk, uint32_t* red) {
    const uint16_t* src = slab < n_q_slabs ? q + (size_t)slab * slab_len
                                           : k + (size_t)(slab - n_q_slabs) * slab_len;
    const int begin = chunk * kCh;
    const int end = min(begin + kCh, slab_len);
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < kCh / (kThreads * 8); ++j) {
        const int i = begin + (j * kThreads + (int)threadIdx.x) * 8;
        if (i < end) m = max(m, max_bf16_mag(*reinterpret_cast<const u32x4*>(src + i)));
    }
    m = block_max_u32(m, red);
    if (threadIdx.x == 0) partial[(size_t)slab * nch + chunk] = m;
}

// blockIdx.y = slab (Q heads first, then K heads); blockIdx.x = chunk of kCh values.
template <int kCh>
__global__ __launch_bounds__(kThreads) void amax_kernel(const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ k,
                                                        uint32_t* __restrict__ partial,
                                                        int n_q_slabs, int slab_len, int nch) {
    __shared__ uint32_t red[kThreads / 64];
    amax_block<kCh>(q, k, partial, n_q_slabs, slab_len, nch, blockIdx.y, blockIdx.x, red);
}

// Kept K magnitudes of a KV cache: state[slab] becomes the larger of itself
// and the largest bf16 magnitude (bits & 0x7FFF, the integer the amax pass
// reduces) of the slab's new keys.  blockIdx.y = slab, blockIdx.x = chunk;
// one atomic max per block.  Integer maxima do not depend on their order, so
// the state equals the amax of every key passed so far, exactly.
__global__ __launch_bounds__(kThreads) void amax_update_kernel(const uint16_t* __restrict__ k,
                                                               uint32_t* __restrict__ state, int slab_len) {
    __shared__ uint32_t red[kThreads / 64];
    const uint16_t* src = k + (size_t)blockIdx.y * slab_len;
    const int begin = blockIdx.x * kChunk;
    const int end = min(begin + kChunk, slab_len);
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < kChunk / (kThreads * 8); ++j) {
        const int i = begin + (j * kThreads + (int)threadIdx.x) * 8;
        if (i < end) m = max(m, max_bf16_mag(*reinterpret_cast<const u32x4*>(src + i)));
    }
    m = block_max_u32(m, red);
    if (threadIdx.x == 0) atomicMax(state + blockIdx.y, m);
}

// One block per (slab, output chunk), slab-major: Q slabs first with
// q_chunks blocks each, then K slabs with k_chunks each.  Output slabs have
// rows_out rows of D codes; rows >= S are written as zero.  With q8 null
// (q_chunks = 1) the Q slabs only get their scale and inverse scale (the
// attention kernel quantises Q rows itself, with the same arithmetic).
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint32_t* __restrict__ partial, float* __restrict__ q_scale, float* __restrict__ k_scale,
    float* __restrict__ q_inv, uint8_t* __restrict__ q8, uint8_t* __restrict__ k8, int n_q_slabs,
    int S, int D, int nch, int rows_out, int q_chunks, int k_chunks) {
    __shared__ uint32_t red[kThreads / 64];
    const int n_qb = n_q_slabs * q_chunks;
    const int bid = blockIdx.x;
    const bool is_q = bid < n_qb;
    const int slab = is_q ? bid / q_chunks : n_q_slabs + (bid - n_qb) / k_chunks;
    const int chunk = is_q ? bid % q_chunks : (bid - n_qb) % k_chunks;
    const int hs = is_q ? slab : slab - n_q_slabs;
    const uint16_t* src = (is_q ? q : k) + (size_t)hs * S * D;
    uint8_t* dst = (is_q ? q8 : k8) + (size_t)hs * rows_out * D;

    const bool codes = !(is_q && q8 == nullptr);
    const int in_len = S * D;
    const int out_len = rows_out * D;
    const int begin = chunk * kChunk;
    const int end = min(begin + kChunk, out_len);
    // every load of the block's chunk is issued first: they do not depend on
    // the scale, and their latency runs under the reduction of the maxima
    constexpr int kPer = kChunk / (kThreads * 8);
    u32x4 w[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = begin + (j * kThreads + (int)threadIdx.x) * 8;
        w[j] = codes && i < in_len && i < end ? *reinterpret_cast<const u32x4*>(src + i) : u32x4{0u, 0u, 0u, 0u};
    }

    uint32_t m = 0;
    for (int i = threadIdx.x; i < nch; i += kThreads) m = max(m, partial[(size_t)slab * nch + i]);
    m = block_max_u32(m, red);
    const float amax = bf16_bits_to_float(m);
    float scale = 1.0f, inv = 1.0f;
    if (amax > 0.0f) {
        // fp64 quotients rounded once to fp32 are the correctly rounded fp32 quotients
        scale = (float)((double)amax / 448.0);
        inv = (float)(448.0 / (double)amax);
    }
    if (chunk == 0 && threadIdx.x == 0) {
        (is_q ? q_scale : k_scale)[hs] = scale;
        if (is_q && q_inv) q_inv[hs] = inv;
    }
    if (!codes) return;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = begin + (j * kThreads + (int)threadIdx.x) * 8;
        if (i >= end) break;
        float x[8];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            x[2 * h] = bf16_bits_to_float(w[j][h] & 0xFFFFu) * inv;
            x[2 * h + 1] = bf16_bits_to_float(w[j][h] >> 16) * inv;
        }
        u32x2 o;
        o[0] = cvt_pk_e4m3<true>(x[2], x[3], cvt_pk_e4m3<false>(x[0], x[1], 0u));
        o[1] = cvt_pk_e4m3<true>(x[6], x[7], cvt_pk_e4m3<false>(x[4], x[5], 0u));
        *reinterpret_cast<u32x2*>(dst + i) = o;
    }
}

template <int D>
constexpr int kTrStride = D + 8;   // bf16 per LDS row of the transpose tile

// One block per (tile t, batch*kv head bh): V[64 keys][D] -> vt[D][64 positions].
// Within each 32-key half, key 16*hi + 4*g + i goes to position 8*g + 4*hi + i:
// lane group g of the P.V operand then reads 8 consecutive positions.
template <int D>
__device__ __forceinline__ void transpose_v_block(const uint16_t* __restrict__ v, uint16_t* __restrict__ vt,
                                                  int S, int nT, int t, int bh, uint16_t* tile) {
    constexpr int kStride = kTrStride<D>;
    constexpr int kChunksPerRow = D / 8;
#pragma unroll
    for (int it = 0; it < kTileKeys * kChunksPerRow / kThreads; ++it) {
        const int c = threadIdx.x + it * kThreads;
        const int key = c / kChunksPerRow, col = c % kChunksPerRow;
        const int gk = t * kTileKeys + key;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (gk < S) w = *reinterpret_cast<const u32x4*>(v + ((size_t)bh * S + gk) * D + col * 8);
        uint32_t* dst = reinterpret_cast<uint32_t*>(tile + key * kStride + col * 8);
        dst[0] = w[0]; dst[1] = w[1]; dst[2] = w[2]; dst[3] = w[3];
    }
    __syncthreads();
    uint16_t* out = vt + ((size_t)bh * nT + t) * D * kTileKeys;
#pragma unroll
    for (int it = 0; it < D * 8 / kThreads; ++it) {
        const int w = threadIdx.x + it * kThreads;
        const int d = w / 8, pb = w % 8;          // 8 positions 8*pb .. 8*pb+7
        const int h = pb / 4, g = pb % 4;
        uint32_t packed[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p0 = 2 * j, p1 = 2 * j + 1;   // positions within the 8
            const int k0 = 32 * h + 16 * (p0 / 4) + 4 * g + (p0 % 4);
            const int k1 = 32 * h + 16 * (p1 / 4) + 4 * g + (p1 % 4);
            packed[j] = (uint32_t)tile[k0 * kStride + d] | ((uint32_t)tile[k1 * kStride + d] << 16);
        }
        *reinterpret_cast<u32x4*>(out + d * kTileKeys + pb * 8) =
            u32x4{packed[0], packed[1], packed[2], packed[3]};
    }
}

// The amax partial maxima of Q and K and the V transpose in one launch: blocks
// [0, n_amax) reduce chunk b % nch of slab b / nch, the rest transpose tile
// (b - n_amax) % nT of head (b - n_amax) / nT.  The two roles share nothing.
template <int D>
__global__ __launch_bounds__(kThreads) void amax_transpose_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, uint32_t* __restrict__ partial,
    int n_q_slabs, int slab_len, int nch, int n_amax, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ vt, int S, int nT) {
    __shared__ uint32_t red[kThreads / 64];
    __shared__ uint16_t tile[kTileKeys * kTrStride<D>];
    const int bid = blockIdx.x;
    if (bid < n_amax) {
        amax_block<kChunk>(q, k, partial, n_q_slabs, slab_len, nch, bid / nch, bid % nch, red);
        return;
    }
    const int tb = bid - n_amax;
    transpose_v_block<D>(v, vt, S, nT, tb % nT, tb / nT, tile);
}

// Decode scales: blocks [0, nq) are query heads (amax over their q_len
// values, read directly), the rest kv heads (max of their nch partial maxima).
// scale = fl32(amax / 448), inv = fl32(448 / amax); 1 and 1 for amax = 0.
__global__ __launch_bounds__(kThreads) void decode_scales_kernel(
    const uint16_t* __restrict__ q, const uint32_t* __restrict__ partial, float* __restrict__ q_scale,
    float* __restrict__ q_inv, float* __restrict__ k_scale, float* __restrict__ k_inv, int nq, int q_len,
    int nch) {
    __shared__ uint32_t red[kThreads / 64];
    const int h = blockIdx.x;
    uint32_t m = 0;
    if (h < nq) {
        const uint16_t* src = q + (size_t)h * q_len;
        for (int i = threadIdx.x * 8; i < q_len; i += kThreads * 8)
            m = max(m, max_bf16_mag(*reinterpret_cast<const u32x4*>(src + i)));
    } else {
        for (int i = threadIdx.x; i < nch; i += kThreads) m = max(m, partial[(size_t)(h - nq) * nch + i]);
    }
    m = block_max_u32(m, red);
    if (threadIdx.x != 0) return;
    const float amax = bf16_bits_to_float(m);
    float scale = 1.0f, inv = 1.0f;
    if (amax > 0.0f) {
        scale = (float)((double)amax / 448.0);
        inv = (float)(448.0 / (double)amax);
    }
    if (h < nq) {
        q_scale[h] = scale;
        q_inv[h] = inv;
    } else {
        k_scale[h - nq] = scale;
        k_inv[h - nq] = inv;
    }
}

__global__ void debug_convert_kernel(const float* __restrict__ x, int64_t n, uint8_t* e4m3,
                                     uint16_t* e4m3_bf16, uint16_t* bf16, float* exp2) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const float v = x[i];
        const uint32_t code = cvt_pk_e4m3<false>(v, 0.0f, 0u) & 0xFFu;
        if (e4m3) e4m3[i] = (uint8_t)code;
        if (e4m3_bf16) e4m3_bf16[i] = (uint16_t)(e4m3x2_to_bf16x2<false>(code) & 0xFFFFu);
        if (bf16) bf16[i] = (uint16_t)(f32x2_to_bf16x2(v, 0.0f) & 0xFFFFu);
        if (exp2) exp2[i] = fast_exp2(v);
    }
}

// Test hook: the polynomial exp2 of the bit-reproducible variant, elementwise.
__global__ void debug_poly_exp2_kernel(const float* __restrict__ x, int64_t n, float* y) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        y[i] = poly_exp2(x[i]);
}

}  // namespace

int amax_chunks(int S, int D) { return (S * D + kChunk - 1) / kChunk; }
int decode_amax_chunks(int Skv, int D) { return (Skv * D + kDecodeChunk - 1) / kDecodeChunk; }

hipError_t launch_quantize_codes(const Shape& sh, const uint16_t* q, const uint16_t* k,
                                 const uint32_t* partial, float* q_scale, float* k_scale, float* q_inv,
                                 uint8_t* q8, uint8_t* k8, int rows_out, hipStream_t st) {
    const int nq = sh.B * sh.Hq, nk = sh.B * sh.Hkv;
    const int nch = amax_chunks(sh.S, sh.D);
    const int nch_out = (rows_out * sh.D + kChunk - 1) / kChunk;
    const int q_chunks = q8 ? nch_out : 1;
    hipLaunchKernelGGL(quantize_kernel, dim3(nq * q_chunks + nk * nch_out), dim3(kThreads), 0, st, q, k,
                       partial, q_scale, k_scale, q_inv, q8, k8, nq, sh.S, sh.D, nch, rows_out, q_chunks,
                       nch_out);
    return hipGetLastError();
}

hipError_t launch_quantize(const Shape& sh, const uint16_t* q, const uint16_t* k,
                           uint32_t* partial, float* q_scale, float* k_scale, float* q_inv,
                           uint8_t* q8, uint8_t* k8, int rows_out, hipStream_t st) {
    const int nq = sh.B * sh.Hq, nk = sh.B * sh.Hkv;
    const int nch = amax_chunks(sh.S, sh.D);
    hipLaunchKernelGGL(amax_kernel<kChunk>, dim3(nch, nq + nk), dim3(kThreads), 0, st, q, k, partial, nq,
                       sh.S * sh.D, nch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_quantize_codes(sh, q, k, partial, q_scale, k_scale, q_inv, q8, k8, rows_out, st);
}

hipError_t launch_amax_transpose(const Shape& sh, const uint16_t* q, const uint16_t* k,
                                 uint32_t* partial, const uint16_t* v, uint16_t* vt, bool with_amax,
                                 hipStream_t st) {
    const int nq = sh.B * sh.Hq, nk = sh.B * sh.Hkv;
    const int nch = amax_chunks(sh.S, sh.D);
    const int n_amax = with_amax ? nch * (nq + nk) : 0;
    const int n_blocks = n_amax + sh.nT * sh.B * sh.Hkv;
    const int slab_len = sh.S * sh.D;
    if (sh.D == 64)
        hipLaunchKernelGGL(amax_transpose_kernel<64>, dim3(n_blocks), dim3(kThreads), 0, st, q, k, partial,
                           nq, slab_len, nch, n_amax, v, vt, sh.S, sh.nT);
    else if (sh.D == 128)
        hipLaunchKernelGGL(amax_transpose_kernel<128>, dim3(n_blocks), dim3(kThreads), 0, st, q, k, partial,
                           nq, slab_len, nch, n_amax, v, vt, sh.S, sh.nT);
    else
        hipLaunchKernelGGL(amax_transpose_kernel<256>, dim3(n_blocks), dim3(kThreads), 0, st, q, k, partial,
                           nq, slab_len, nch, n_amax, v, vt, sh.S, sh.nT);
    return hipGetLastError();
}

hipError_t launch_decode_scales(const DecodeShape& sh, const uint16_t* q, const uint16_t* k,
                                uint32_t* partial, float* q_scale, float* q_inv, float* k_scale,
                                float* k_inv, hipStream_t st) {
    const int nq = sh.B * sh.Hq, nk = sh.B * sh.Hkv;
    const int nch = decode_amax_chunks(sh.Skv, sh.D);
    // K partial maxima (every slab is a K slab)
    hipLaunchKernelGGL(amax_kernel<kDecodeChunk>, dim3(nch, nk), dim3(kThreads), 0, st, q, k, partial, 0,
                       sh.Skv * sh.D, nch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_scales_kernel, dim3(nq + nk), dim3(kThreads), 0, st, q, partial, q_scale, q_inv,
                       k_scale, k_inv, nq, sh.Sq * sh.D, nch);
    return hipGetLastError();
}

hipError_t launch_kv_amax_update(const uint16_t* k, int n_slabs, int slab_len, uint32_t* state,
                                 hipStream_t st) {
    const int nch = (slab_len + kChunk - 1) / kChunk;
    hipLaunchKernelGGL(amax_update_kernel, dim3(nch, n_slabs), dim3(kThreads), 0, st, k, state, slab_len);
    return hipGetLastError();
}

hipError_t launch_decode_scales_kept(const DecodeShape& sh, const uint16_t* q, const uint32_t* k_amax,
                                     float* q_scale, float* q_inv, float* k_scale, float* k_inv,
                                     hipStream_t st) {
    const int nq = sh.B * sh.Hq, nk = sh.B * sh.Hkv;
    // the kept maxima stand in for the partial maxima, one per K slab
    hipLaunchKernelGGL(decode_scales_kernel, dim3(nq + nk), dim3(kThreads), 0, st, q, k_amax, q_scale, q_inv,
                       k_scale, k_inv, nq, sh.Sq * sh.D, 1);
    return hipGetLastError();
}

hipError_t launch_debug_convert(const float* x, int64_t n, uint8_t* e4m3, uint16_t* e4m3_bf16,
                                uint16_t* bf16, float* exp2, hipStream_t st) {
    int64_t blocks = (n + kThreads - 1) / kThreads;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(debug_convert_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, x, n,
                       e4m3, e4m3_bf16, bf16, exp2);
    return hipGetLastError();
}

hipError_t launch_debug_poly_exp2(const float* x, int64_t n, float* y, hipStream_t st) {
    int64_t blocks = (n + kThreads - 1) / kThreads;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(debug_poly_exp2_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, x, n, y);
    return hipGetLastError();
}

}  // namespace lamp
