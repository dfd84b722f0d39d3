// Host-side launchers of the gfx950 kernels (defined in the .hip files).
// All return a hipError_t from the launch; none allocates memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lamp {

// Geometry of one forward call, shared by the launchers.
struct Shape {
    int B, Hq, Hkv, S, D;
    int nT;      // ceil(S / 64)
    int S_pad;   // nT * 64
};

// Number of amax partial maxima (chunks) for a slab of S*D bf16 values.
int amax_chunks(int S, int D);
// The same for the K pass of a decode step (launch_decode_scales).
int decode_amax_chunks(int Skv, int D);

// Quantisation pass (Q and K): per-(batch, head) amax partial maxima, then
// scales and e4m3 codes.  q8 / k8 are written with `rows_out` rows per head
// (rows >= S are zero).  With q8 null, Q gets only its scales and inverse
// scales (q_inv, nullable otherwise).  partial must hold
// (B*Hq + B*Hkv) * amax_chunks(S, D) uint32 values.
hipError_t launch_quantize(const Shape& sh, const uint16_t* q, const uint16_t* k,
                           uint32_t* partial, float* q_scale, float* k_scale, float* q_inv,
                           uint8_t* q8, uint8_t* k8, int rows_out, hipStream_t st);

// The amax partial maxima of launch_quantize (when with_amax), and in the same
// launch V [B, Hkv, S, D] -> vt [B, Hkv, nT, D, 64] (keys of each tile
// transposed and permuted into the order the P.V matrix-core operand reads;
// padding keys 0).
hipError_t launch_amax_transpose(const Shape& sh, const uint16_t* q, const uint16_t* k,
                                 uint32_t* partial, const uint16_t* v, uint16_t* vt, bool with_amax,
                                 hipStream_t st);

// The second half of launch_quantize: scales and codes from the partial maxima.
hipError_t launch_quantize_codes(const Shape& sh, const uint16_t* q, const uint16_t* k,
                                 const uint32_t* partial, float* q_scale, float* k_scale, float* q_inv,
                                 uint8_t* q8, uint8_t* k8, int rows_out, hipStream_t st);

struct AttnParams {
    const uint8_t* k8;      // [B, Hkv, S_pad, D]
    const uint16_t* q16;    // [B, Hq, S, D] bf16 (caller's Q)
    const uint16_t* k16;    // [B, Hkv, S, D] bf16 (caller's K)
    const uint16_t* vt;     // [B, Hkv, nT, D, 64] bf16
    const float* q_scale;   // [B * Hq]
    const float* q_inv;     // [B * Hq] inverse scales, as the quantisation pass uses them
    const float* k_scale;   // [B * Hkv]
    float* out;             // [B, Hq, S, D]
    uint8_t* mask;          // [B, Hq, nT, nT] or null
    float* dump_s = nullptr;     // debug dump of 8-bit accumulators [B, Hq, S, S]
    uint16_t* dump_p = nullptr;  // debug dump of final bf16 weights [B, Hq, S, S]
    double log2e_over_sqrt_d;
    float e_delta;          // smallest fp32 exponential that rounds to an e4m3 value >= delta
    float t2;               // second-stage threshold on |log2-domain logit|
    int causal, window;
    int plain = 0;          // 1: plain bf16 FlashAttention (no 8-bit pass; D <= 128)
    int logit8 = 0;         // 1: log2-domain logits rounded to e4m3 before use
    int exp_poly = 0;       // 1: 8-bit exponentials by the polynomial exp2 (not with logit8 or plain)
};

// The forward attention kernel (16-bit recompute inside the tile loop).
hipError_t launch_attention(const Shape& sh, const AttnParams& p, hipStream_t st);

// Split-KV decode: Sq <= 16 query rows (the last positions) against Skv keys.
struct DecodeShape {
    int B, Hq, Hkv, Sq, Skv, D;
    int nT;        // ceil(Skv / 64) KV tiles
    int tps;       // KV tiles per split
    int n_split;   // ceil(nT / tps)
};

struct DecodeParams {
    const uint16_t* q16;    // [B, Hq, Sq, D] bf16
    const uint16_t* k16;    // [B, Hkv, Skv, D] bf16
    const uint16_t* v16;    // [B, Hkv, Skv, D] bf16
    const float* q_scale;   // [B * Hq]
    const float* q_inv;
    const float* k_scale;   // [B * Hkv]
    const float* k_inv;
    float* part_o;          // [B, Hq, n_split, Sq, D] workspace
    float* part_ml;         // [B, Hq, n_split, Sq, 2] workspace
    float* out;             // [B, Hq, Sq, D]
    uint8_t* mask;          // [B, Hq, nT] or null
    double log2e_over_sqrt_d;
    float e_delta, t2;
    int causal, window;
};

// Per-head scales and inverse scales of the decode inputs: Q heads over
// their Sq rows, K heads over all Skv rows (partial must hold
// B * Hkv * decode_amax_chunks(Skv, D) uint32 values).
hipError_t launch_decode_scales(const DecodeShape& sh, const uint16_t* q, const uint16_t* k,
                                uint32_t* partial, float* q_scale, float* q_inv, float* k_scale,
                                float* k_inv, hipStream_t st);

// Kept K magnitudes: state[s] = max(state[s], max over slab s of k of the bf16
// magnitude bits), for n_slabs slabs of slab_len values (one atomic max per
// 16384-value chunk).
hipError_t launch_kv_amax_update(const uint16_t* k, int n_slabs, int slab_len, uint32_t* state,
                                 hipStream_t st);

// The decode scales with the K maxima taken from kept state (B * Hkv values)
// instead of a pass over K.
hipError_t launch_decode_scales_kept(const DecodeShape& sh, const uint16_t* q, const uint32_t* k_amax,
                                     float* q_scale, float* q_inv, float* k_scale, float* k_inv,
                                     hipStream_t st);

// The decode kernel (one workgroup per batch, kv head and split) and the merge
// of the splits into out.
// The decode kernel (split results into the workspace), then the merge of
// the splits into out.
hipError_t launch_decode(const DecodeShape& sh, const DecodeParams& p, hipStream_t st);
hipError_t launch_decode_merge(const DecodeShape& sh, const DecodeParams& p, hipStream_t st);

// Compute units of the current device (256 when it cannot be queried).
int cu_count();

// Sub-block statistics of a mask (see lamp_subblock_stats).
hipError_t launch_subblock_stats(const uint8_t* mask, int B, int Hq, int S, int causal,
                                 int window, int64_t* stats, hipStream_t st);

// n blocks of a [16][128] . b [16][128]^T (e4m3 codes) -> out [16][16] fp32 on
// the attention kernel's 8-bit Q.K^T instruction.
hipError_t launch_debug_fp8_dot(const uint8_t* a, const uint8_t* b, float* out, int n, hipStream_t st);

hipError_t launch_debug_convert(const float* x, int64_t n, uint8_t* e4m3, uint16_t* e4m3_bf16,
                                uint16_t* bf16, float* exp2, hipStream_t st);
// Test hook: the attention kernel's polynomial exp2 on n values.
hipError_t launch_debug_poly_exp2(const float* x, int64_t n, float* y, hipStream_t st);

}  // namespace lamp
