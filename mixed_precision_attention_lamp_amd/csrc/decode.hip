// Split-KV decode kernels of the LampAttention forward pass for gfx950.
//
// Decode: Sq <= 16 query rows, the last positions of a sequence, against all
// Skv cached keys.  The method per tile is that of the prefill kernel
// ("LampAttention: Look-Ahead Mixed-Precision FlashAttention for Dedicated
// Accelerators", abstract: 8-bit logits and exponentials, the two-stage
// look-ahead test, 16-bit recompute of the flagged sub-blocks, online
// softmax, P.V).  The Sq rows of one query head form the row block the test
// runs on.  The KV tiles are cut into contiguous splits; every split runs
// the tile loop from an empty state and leaves its running max, row sum and
// unnormalised output; a merge kernel combines the splits.
//
// The decode kernel is bound by HBM bandwidth, so it reads each bf16 K and V
// value once: a K tile is staged into LDS as bf16 (the recompute's operand)
// and quantised to e4m3 into a second LDS tile on the way (the arithmetic of
// the quantisation pass, with the per-head scale from the scale pass); a V
// tile is transposed on the way into the layout of the P.V operand.  No K8
// or V^T copy is written to HBM.
//
// Work decomposition: one workgroup per (batch, kv head, split), of four
// waves, or eight when the GQA group has more than four heads or D = 256
// (more threads to stage the larger tiles).  Wave w owns query head w of the
// group (if there is one), as one 16-row group (rows past Sq are masked
// out), so all heads of a group share each staged tile.
#include <hip/hip_runtime.h>

#include <cmath>

#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace lamp {

namespace {


struct DecodeArgs {
    const uint16_t* q16;   // [B, Hq, Sq, D]
    const uint16_t* k16;   // [B, Hkv, Skv, D]
    const uint16_t* v16;   // [B, Hkv, Skv, D]
    const float* q_scale;  // [B * Hq]
    const float* q_inv;
    const float* k_scale;  // [B * Hkv]
    const float* k_inv;
    float* part_o;         // [B, Hq, n_split, Sq, D]  unnormalised outputs of the splits
    float* part_ml;        // [B, Hq, n_split, Sq, 2]  (running max, row sum)
    uint8_t* mask;         // [B, Hq, nT] or null
    double l_d;
    float x_delta;
    float t2;
    int B, Hq, Hkv, Sq, Skv, nT, G;
    int causal, window;
    int tps, n_split;
    int tps_pad;           // tps rounded up to 16 (LDS bytes per wave for mask bytes)
};

template <int D, int kThreads>
struct DCfg {
    static constexpr int kKS = D >= 128 ? D / 128 : 1;   // 128-deep FP8 steps
    static constexpr int kK8Row = D;
    static constexpr int kK16Row = 2 * D;
    static constexpr int kVRow = 2 * D;
    static constexpr int kK8Bytes = kTileKeys * kK8Row;
    static constexpr int kK16Bytes = kTileKeys * kK16Row;
    static constexpr int kVBytes = kTileKeys * kVRow;
    static constexpr int kK8Off = 0;
    static constexpr int kK16Off = kK8Bytes;
    static constexpr int kVOff = kK16Off + kK16Bytes;
    static constexpr int kLdsBytes = kVOff + kVBytes;
    static constexpr int kDB = D / 16;
    static constexpr int kDC = D / 32;
    static constexpr int kRowChunks = D / 8;                     // 16-byte chunks per K/V row
    static constexpr int kCh = kTileKeys * kRowChunks / kThreads;   // chunks per thread and tile
    static_assert(kCh * kThreads == kTileKeys * kRowChunks, "tile chunks must split evenly");
    // A thread stages runs of kRun consecutive keys at one 16-byte column.
    static constexpr int kRun = kCh < 4 ? kCh : 4;
    static constexpr int kRuns = kCh / kRun;                     // runs per thread and tile
};

// Two fp32 values -> two e4m3fn codes, without the clamp of cvt_pk_e4m3: for
// values below 464 in magnitude, which round to at most 448.
template <bool Hi>
__device__ __forceinline__ uint32_t cvt_pk_e4m3_in_range(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, Hi);
}

// The P.V operand of d-block db and key half h, read from the staged V tile
// (row-major, one row per key, 16-byte chunks swizzled like the K16 tile) by
// two transposing LDS reads.  ds_read_b64_tr_b16 treats each 16-lane group as
// a 16 x 4 matrix of 16-bit values (lane l' supplies the 4 values at its
// address) and hands lane m element k of row 4k + m/4, column m % 4 (checked
// on the device).  So lane 4k + jj of group g reads 4 consecutive depths
// 16db + 4jj .. of key K(g, k), and lane n16 of group g receives depth
// 16db + n16 of keys K(g, 0..3).  K(g, k) = 32h + 4g + k (first read) and
// that + 16 (second): the order in which the exponentials of the Q.K^T
// output layout sit in the P operand of lane group g.
template <int D>
__device__ __forceinline__ v8bf v_operand_tr(const uint8_t* vl, int h, int db, int n16, int g) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef short v8s __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const int key = 32 * h + 4 * g + (n16 >> 2);
    const int dd = 16 * db + 4 * (n16 & 3);   // first depth of this lane's read
    const int in_chunk = (dd & 7) * 2;
    const uint8_t* p0 = vl + lds_off<2 * D>(key, dd >> 3) + in_chunk;
    const uint8_t* p1 = vl + lds_off<2 * D>(key + 16, dd >> 3) + in_chunk;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(__attribute__((address_space(3))) const void*)p0);
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(__attribute__((address_space(3))) const void*)p1);
    const v8s x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(v8bf, x);
}

// Query row i (sequence position Skv - Sq + i) sees key j.
__device__ __forceinline__ bool dec_visible(int i, int j, int Sq, int Skv, int causal, int window) {
    const int p = Skv - Sq + i;
    // bitwise, not short-circuit: selects rather than branches
    return (i < Sq) & (j < Skv) & ((causal == 0) | (j <= p)) & ((window <= 0) | (p - j < window));
}

// kW waves; kMode: 0 = no test (second stage off), 1 = both stages, 2 =
// second stage only.
template <int D, int kW, int kMode>
__global__ __launch_bounds__(kW * 64, 2) void lamp_decode_kernel(DecodeArgs a) {
    constexpr int kDThreads = kW * 64;
    constexpr int kQG = 1;        // query heads per wave
    using C = DCfg<D, kDThreads>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int n16 = lane & 15;     // query row
    const int g = lane >> 4;       // lane group: which 4 keys / which k-slice
    const int n_units = a.B * a.Hkv;
    const int unit = blockIdx.x % n_units;
    const int split = blockIdx.x / n_units;
    const int b = unit / a.Hkv;
    const int hk = unit % a.Hkv;
    const size_t kv_head = (size_t)b * a.Hkv + hk;

    int hq[kQG];
    bool hv[kQG];
#pragma unroll
    for (int j = 0; j < kQG; ++j) {
        const int gh = kW * j + wave;
        hv[j] = gh < a.G;
        hq[j] = hk * a.G + (hv[j] ? gh : 0);
    }
    const bool row_ok = n16 < a.Sq;
    const uint64_t row_mask = wave_ballot(row_ok);   // lanes of rows 0 .. Sq-1

    // tiles of this split; with a window the tiles before t_lo hold no visible key
    const int t_begin = split * a.tps;
    const int t_end = min(t_begin + a.tps, a.nT) - 1;
    int t_lo = 0;
    if (a.window > 0) {
        const int j = a.Skv - a.Sq - a.window + 1;
        t_lo = j <= 0 ? 0 : j / kTileKeys;
    }
    const int t_first = max(t_begin, t_lo);
    // mask bytes of the split's tiles collect in LDS (one row of tps bytes per
    // wave) and go out after the loop: no global store inside the loop, where
    // it would make the compiler wait for every outstanding load
    // mask bytes of the split's tiles.  D <= 128: lane i of mask_reg holds the
    // byte of tile t_first + 64 c + i; the 64 bytes of chunk c go out when the
    // loop leaves it (one global store per 64 tiles).  D = 256: one row of tps
    // bytes per wave in LDS, written out after the loop.  Either way no global
    // store in every iteration, where it would make the compiler wait for
    // every outstanding load.
    uint8_t* mask_lds = lds + C::kLdsBytes + wave * a.tps_pad;
    uint32_t mask_reg = 0;
    uint8_t* const mrow = a.mask && hv[0] ? a.mask + ((size_t)b * a.Hq + hq[0]) * a.nT : nullptr;

    // ---- prologue: Q operands and constants per query head -------------------------
    v8i qf[kQG][C::kKS];
    v8bf qb[C::kDC][kQG];
    float c8[kQG], inv_c8[kQG], a2[kQG];
    const float c16 = (float)a.l_d;
#pragma unroll
    for (int j = 0; j < kQG; ++j) {
        const size_t qh = (size_t)b * a.Hq + hq[j];
        const uint16_t* qrow = a.q16 + (qh * a.Sq + min(n16, a.Sq - 1)) * D;
        const bool use = hv[j] && row_ok;
#pragma unroll
        for (int ch = 0; ch < C::kDC; ++ch) {
            v8bf x = {};
            if (use) x = *reinterpret_cast<const v8bf*>(qrow + ch * 32 + g * 8);
            qb[ch][j] = x;
        }
        // Q8 = E4M3(fl32(q * inv)), the arithmetic of the quantisation pass, as
        // the FP8 operand: lane group g holds depth 32g .. 32g+31 of each step
        const float inv = a.q_inv[qh];
#pragma unroll
        for (int st = 0; st < C::kKS; ++st) {
            v8i x = {0, 0, 0, 0, 0, 0, 0, 0};
            if (use && (D >= 128 || g * 32 < D)) {
                const int gg = D >= 128 ? st * 4 + g : g;
                const uint16_t* src = qrow + 32 * gg;
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const u32x4 w = *reinterpret_cast<const u32x4*>(src + 8 * h);
                    float y[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        y[2 * e] = bf16_bits_to_float(w[e] & 0xFFFFu) * inv;
                        y[2 * e + 1] = bf16_bits_to_float(w[e] >> 16) * inv;
                    }
                    x[2 * h] = (int)cvt_pk_e4m3<true>(y[2], y[3], cvt_pk_e4m3<false>(y[0], y[1], 0u));
                    x[2 * h + 1] = (int)cvt_pk_e4m3<true>(y[6], y[7], cvt_pk_e4m3<false>(y[4], y[5], 0u));
                }
            }
            qf[j][st] = x;
        }
        c8[j] = (float)((double)a.q_scale[qh] * (double)a.k_scale[kv_head] * a.l_d);
        a2[j] = acc_threshold(a.t2, c8[j]);
        inv_c8[j] = 1.0f / c8[j];
    }
    const float k_inv = a.k_inv[kv_head];

    float m_run[kQG];
    v4f acc_o[kQG][C::kDB];
    v4f acc_l[kQG];
#pragma unroll
    for (int j = 0; j < kQG; ++j) {
        m_run[j] = -__builtin_inff();
        acc_l[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < C::kDB; ++db) acc_o[j][db] = v4f{0.f, 0.f, 0.f, 0.f};
    }

    // ---- staging: K and V rows through registers into LDS ---------------------------
    // Run u of a tile is keys kRun (u / kRowChunks) .. +kRun-1 at depth
    // 8 (u % kRowChunks) .. +7; thread tid stages runs tid + kDThreads r.
    const uint16_t* k_head = a.k16 + kv_head * (size_t)a.Skv * D;
    const uint16_t* v_head = a.v16 + kv_head * (size_t)a.Skv * D;
    // two register sets (D <= 128): tiles t+1 and t+2 are in flight while
    // tile t is computed
    u32x4 rkA[C::kCh], rvA[C::kCh];
    auto load = [&](int t, u32x4 (&rk)[C::kCh], u32x4 (&rv)[C::kCh]) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < C::kRuns; ++r) {
            const int u = tid + r * kDThreads;
            const int key0 = (u / C::kRowChunks) * C::kRun, col = u % C::kRowChunks;
#pragma unroll
            for (int e = 0; e < C::kRun; ++e) {
                // keys past the end reload the last key: they are masked out
                const unsigned gk = (unsigned)min(t * kTileKeys + key0 + e, a.Skv - 1);
                rk[r * C::kRun + e] = *reinterpret_cast<const u32x4*>(k_head + gk * D + col * 8);
                rv[r * C::kRun + e] = *reinterpret_cast<const u32x4*>(v_head + gk * D + col * 8);
            }
        }
    };
    uint8_t* k8l = lds + C::kK8Off;
    uint8_t* k16l = lds + C::kK16Off;
    uint8_t* vl = lds + C::kVOff;
    auto store = [&](const u32x4 (&rk)[C::kCh], const u32x4 (&rv)[C::kCh], const int so) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < C::kRuns; ++r) {
            const int u = tid + r * kDThreads;
            const int key0 = (u / C::kRowChunks) * C::kRun, col = u % C::kRowChunks;
#pragma unroll
            for (int e = 0; e < C::kRun; ++e) {
                const int key = key0 + e;
                const u32x4 w = rk[r * C::kRun + e];
                // K16 tile: logical chunk col of row key
                *reinterpret_cast<u32x4*>(k16l + so + lds_off<C::kK16Row>(key, col)) = w;
                // K8 tile: the 8 codes of depth 8col.. fill half of logical chunk col / 2
                // (|k| <= amax, so |k * k_inv| rounds to at most 448: no clamp)
                float y[8];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    y[2 * x] = bf16_bits_to_float(w[x] & 0xFFFFu) * k_inv;
                    y[2 * x + 1] = bf16_bits_to_float(w[x] >> 16) * k_inv;
                }
                const u32x2 o = {cvt_pk_e4m3_in_range<true>(y[2], y[3], cvt_pk_e4m3_in_range<false>(y[0], y[1], 0u)),
                                 cvt_pk_e4m3_in_range<true>(y[6], y[7], cvt_pk_e4m3_in_range<false>(y[4], y[5], 0u))};
                *reinterpret_cast<u32x2*>(k8l + so + lds_off<C::kK8Row>(key, col >> 1) + (col & 1) * 8) = o;
                // V tile: as loaded, at the K16 tile's offsets (the P.V reads transpose)
                *reinterpret_cast<u32x4*>(vl + so + lds_off<C::kVRow>(key, col)) = rv[r * C::kRun + e];
            }
        }
    };

    const v8bf ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                       (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
    constexpr float kNegInf = -__builtin_inff();

    auto tile = [&](const int t, const int so) __attribute__((always_inline)) {
        // waves without a query head only stage tiles
        if (hv[0]) {
            // ---- (1) 8-bit logits: s[j][kb][i] = key 16kb + 4g + i, query row n16
            v4f s[kQG][4];
#pragma unroll
            for (int st = 0; st < C::kKS; ++st)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const v8i ka = fp8_operand<D>(k8l + so, kb * 16 + n16, st, g);
#pragma unroll
                    for (int j = 0; j < kQG; ++j)
                        s[j][kb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            ka, qf[j][st], st == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : s[j][kb], 0, 0, 0, 0, 0, 0);
                }
            // visibility: an entry whose key its row does not see gets the logit
            // -inf, so that its exponential is 0 and the sub-block maxima ignore
            // it.  Tiles that every row sees whole (all but the causal, window
            // and Skv edges) skip this; there the rows past Sq (zero Q operands,
            // logits 0) are left out of the test by row_mask.
            const int j_last = t * kTileKeys + kTileKeys - 1;
            const bool all_rows_see_all = j_last < a.Skv && (!a.causal || j_last <= a.Skv - a.Sq) &&
                                          (a.window <= 0 || (a.Skv - 1) - t * kTileKeys < a.window);
            if (!all_rows_see_all) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool vv = dec_visible(n16, t * kTileKeys + kb * 16 + g * 4 + i, a.Sq, a.Skv, a.causal, a.window);
#pragma unroll
                        for (int j = 0; j < kQG; ++j) s[j][kb][i] = vv ? s[j][kb][i] : kNegInf;
                    }
            }

            // ---- (2)-(3) running max and 8-bit exponentials, per query head
            float alpha[kQG], m_use[kQG];
            float smax[kQG][4], smin[kQG][4];
            u32x2 P[kQG][4];
#pragma unroll
            for (int j = 0; j < kQG; ++j) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    float hi = kNegInf, lo = -kNegInf;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        hi = __builtin_fmaxf(hi, s[j][kb][i]);
                        if constexpr (kMode == 2)   // the minimum over seen keys only
                            lo = __builtin_fminf(lo, s[j][kb][i] == kNegInf ? -kNegInf : s[j][kb][i]);
                    }
                    smax[j][kb] = hi;
                    smin[j][kb] = lo;
                }
                float mx = __builtin_fmaxf(__builtin_fmaxf(smax[j][0], smax[j][1]),
                                           __builtin_fmaxf(smax[j][2], smax[j][3]));
                mx = max_over_lane_groups(mx);
                // rounding is monotone: the max of the fp32 logits is c8 times the
                // max accumulator, rounded
                const float mt = mx == kNegInf ? mx : mx * c8[j];
                const float mn = __builtin_fmaxf(m_run[j], mt);
                alpha[j] = mn == m_run[j] ? 1.0f : fast_exp2(m_run[j] - mn);
                m_use[j] = mn == kNegInf ? 0.0f : mn;
                m_run[j] = mn;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    float e[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)   // 2^-inf = 0 for unseen keys
                        e[i] = fast_exp2(__builtin_fmaf(s[j][kb][i], c8[j], -m_use[j]));
                    const uint32_t w = cvt_pk_e4m3_unit<true>(
                        e[2], e[3], cvt_pk_e4m3_unit<false>(e[0], e[1], __float_as_uint(e[0])));
                    P[j][kb] = u32x2{e4m3x2_to_bf16x2<false>(w), e4m3x2_to_bf16x2<true>(w)};
                }
            }

            // ---- (4) look-ahead test per query head: 4-bit flag sets (wave-uniform)
            // First stage: acc >= a1 = (x_delta + m) / c8; second: |acc| >= a2.  With
            // a1 > -a2 both hold iff acc >= max(a1, a2), so the sub-block maximum
            // decides; rows with a1 <= -a2 take the per-entry test.
            uint32_t flags[kQG];
#pragma unroll
            for (int j = 0; j < kQG; ++j) {
                uint64_t hit[4] = {0, 0, 0, 0};
                if constexpr (kMode == 1) {
                    const float a1 = (a.x_delta + m_use[j]) * inv_c8[j];
                    const float thr = __builtin_fmaxf(a1, a2[j]);
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) hit[kb] = wave_ballot(smax[j][kb] >= thr);
                    if (wave_ballot(row_ok && a1 <= -a2[j]) != 0) {
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) {
                            hit[kb] = 0;
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                // (x_delta may be -inf: unseen keys are excluded explicitly)
                                const float v = s[j][kb][i];
                                hit[kb] |= wave_ballot(__builtin_fmaf(v, c8[j], -m_use[j]) >= a.x_delta) &
                                           wave_ballot(__builtin_fabsf(v) >= a2[j]) &
                                           wave_ballot(v != kNegInf);
                            }
                        }
                    }
                } else if constexpr (kMode == 2) {
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
                        hit[kb] = wave_ballot(smax[j][kb] >= a2[j]) | wave_ballot(smin[j][kb] <= -a2[j]);
                }
                uint32_t f = 0;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) f |= ((hit[kb] & row_mask) != 0 ? 1u : 0u) << kb;
                flags[j] = hv[j] ? f : 0u;
            }

            // ---- (5) 16-bit recompute of the sub-blocks some head of the wave flagged;
            // each head takes the bf16 weights only where it flagged the sub-block
            uint32_t any = 0;
#pragma unroll
            for (int j = 0; j < kQG; ++j) any |= flags[j];
            any = __builtin_amdgcn_readfirstlane(any);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (!((any >> c) & 1u)) continue;
                v4f acc16[kQG];
#pragma unroll
                for (int ch = 0; ch < C::kDC; ++ch) {
                    const v8bf ka = *reinterpret_cast<const v8bf*>(k16l + so + lds_off<C::kK16Row>(c * 16 + n16, ch * 4 + g));
#pragma unroll
                    for (int j = 0; j < kQG; ++j)
                        acc16[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            ka, qb[ch][j], ch == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : acc16[j], 0, 0, 0);
                }
#pragma unroll
                for (int j = 0; j < kQG; ++j) {
                    if (!((flags[j] >> c) & 1u)) continue;
                    float e[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {   // unseen keys: 8-bit logit -inf
                        e[i] = fast_exp2(__builtin_fmaf(acc16[j][i], c16, -m_use[j]));
                        e[i] = s[j][c][i] == kNegInf ? 0.0f : e[i];
                    }
                    P[j][c] = u32x2{f32x2_to_bf16x2(e[0], e[1]), f32x2_to_bf16x2(e[2], e[3])};
                }
            }

            // ---- (6) online-softmax rescale, then P.V (row sums from an all-ones operand)
#pragma unroll
            for (int j = 0; j < kQG; ++j) {
                if (wave_ballot(alpha[j] != 1.0f) != 0) {
                    acc_l[j] *= alpha[j];
#pragma unroll
                    for (int db = 0; db < C::kDB; ++db) acc_o[j][db] *= alpha[j];
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                v8bf pb[kQG];
#pragma unroll
                for (int j = 0; j < kQG; ++j) {
                    const u32x4 w = {P[j][2 * h][0], P[j][2 * h][1], P[j][2 * h + 1][0], P[j][2 * h + 1][1]};
                    pb[j] = __builtin_bit_cast(v8bf, w);
                }
#pragma unroll
                for (int db = 0; db < C::kDB; ++db) {
                    const v8bf va = v_operand_tr<D>(vl + so, h, db, n16, g);
#pragma unroll
                    for (int j = 0; j < kQG; ++j)
                        acc_o[j][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[j], acc_o[j][db], 0, 0, 0);
                }
#pragma unroll
                for (int j = 0; j < kQG; ++j)
                    acc_l[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[j], acc_l[j], 0, 0, 0);
            }

            // ---- (7) mask byte
            if constexpr (D <= 128) {
                if (lane == ((t - t_first) & 63)) mask_reg = 0x80u | flags[0];
            } else {
                if (lane == 0) mask_lds[t - t_begin] = (uint8_t)(0x80u | flags[0]);
            }
        }
    };

    // Loads run every iteration; past the split's last tile they reload it
    // (from cache), which keeps the compiler from waiting on all loads at
    // the loop head.
    if constexpr (D <= 128) {
        // Two LDS slots.  The stores of tile t+1 go to the slot tile t does not
        // read, in the same block as tile t's work, and one barrier per tile
        // orders both: every wave has read a slot before it is refilled, and
        // the stores of t+1 are visible before t+1 is read.
        constexpr int kSlot = C::kLdsBytes;
        if (mrow)   // tiles before t_first (outside the window) hold no visible key
            for (int i = t_begin + lane; i < t_first; i += 64) mrow[i] = 0;
        if (t_first <= t_end) {
            load(t_first, rkA, rvA);
            store(rkA, rvA, 0);
            load(min(t_first + 1, t_end), rkA, rvA);
        }
        lds_barrier();
        for (int t = t_first; t <= t_end; ++t) {
            const int so = ((t - t_first) & 1) * kSlot;
            store(rkA, rvA, kSlot - so);
#ifdef LAMP_EXTRA_SYNC
            lds_barrier();   // test build: every wave's stores of t+1 before any reads of t
#endif
            load(min(t + 2, t_end), rkA, rvA);
            tile(t, so);
            if (((t - t_first) & 63) == 63 || t == t_end) {
                const int t0 = t - ((t - t_first) & 63);
                if (mrow && t0 + lane <= t) mrow[t0 + lane] = (uint8_t)mask_reg;
                mask_reg = 0;
            }
            lds_barrier();
        }
    } else {
        // D = 256: one slot, one register set (two would not fit next to the
        // accumulators); a barrier after the stores, one after the tile
        if (t_first <= t_end) load(t_first, rkA, rvA);
        for (int t = t_first; t <= t_end; ++t) {
            store(rkA, rvA, 0);
            lds_barrier();
            load(min(t + 1, t_end), rkA, rvA);
            tile(t, 0);
            lds_barrier();
        }
        if (mrow)
            for (int i = lane; i <= t_end - t_begin; i += 64)
                mrow[t_begin + i] = t_begin + i < t_first ? (uint8_t)0 : mask_lds[i];
    }

    // ---- the split's running max, row sum and unnormalised output ----------------------
#pragma unroll
    for (int j = 0; j < kQG; ++j) {
        if (!hv[j] || !row_ok) continue;
        const size_t prow = (((size_t)b * a.Hq + hq[j]) * a.n_split + split) * a.Sq + n16;
        float* dst = a.part_o + prow * D + g * 4;
#pragma unroll
        for (int db = 0; db < C::kDB; ++db) *reinterpret_cast<v4f*>(dst + db * 16) = acc_o[j][db];
        if (g == 0) {
            a.part_ml[prow * 2] = m_run[j];
            a.part_ml[prow * 2 + 1] = acc_l[j][0];
        }
    }
}

// out[row, d] = sum_s 2^(m_s - M) O_s[row, d] / sum_s 2^(m_s - M) l_s[row],
// M = max_s m_s; splits with m_s = -inf (no visible key) weigh 0.  A thread
// merges four consecutive columns of one row.
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           float* __restrict__ out, int rows, int Sq,
                                                           int n_split, int D) {
    const int D4 = D / 4;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * D4) return;
    const int row = idx / D4, d = (idx % D4) * 4;
    const int bh = row / Sq, i = row % Sq;
    const float* ml = part_ml + ((size_t)bh * n_split * Sq + i) * 2;   // split s at ml[2 s Sq]
    const size_t stride = (size_t)Sq * 2;
    float M = -__builtin_inff();
#pragma unroll 8
    for (int s = 0; s < n_split; ++s) M = __builtin_fmaxf(M, ml[s * stride]);
    v4f num = {0.f, 0.f, 0.f, 0.f};
    float den = 0.0f;
#pragma unroll 8
    for (int s = 0; s < n_split; ++s) {
        const float m = ml[s * stride];
        const float w = m == -__builtin_inff() ? 0.0f : fast_exp2(m - M);
        const size_t pr = ((size_t)bh * n_split + s) * Sq + i;
        num += w * *reinterpret_cast<const v4f*>(part_o + pr * D + d);
        den += w * ml[s * stride + 1];
    }
    *reinterpret_cast<v4f*>(out + (size_t)row * D + d) = num / den;
}

template <int D>
hipError_t launch_decode_d(const DecodeShape& sh, const DecodeParams& p, hipStream_t st) {
    DecodeArgs a;
    a.q16 = p.q16; a.k16 = p.k16; a.v16 = p.v16;
    a.q_scale = p.q_scale; a.q_inv = p.q_inv; a.k_scale = p.k_scale; a.k_inv = p.k_inv;
    a.part_o = p.part_o; a.part_ml = p.part_ml; a.mask = p.mask;
    a.l_d = p.log2e_over_sqrt_d; a.t2 = p.t2;
    a.x_delta = p.e_delta > 0.0f ? (float)std::log2((double)p.e_delta) : -__builtin_inff();
    const int mode = !(p.t2 < __builtin_inff()) || !(p.e_delta < __builtin_inff()) ? 0 : (p.e_delta > 0.0f ? 1 : 2);
    a.B = sh.B; a.Hq = sh.Hq; a.Hkv = sh.Hkv; a.Sq = sh.Sq; a.Skv = sh.Skv; a.nT = sh.nT;
    a.G = sh.Hq / sh.Hkv;
    a.causal = p.causal; a.window = p.window;
    a.tps = sh.tps; a.n_split = sh.n_split;
    a.tps_pad = (sh.tps + 15) / 16 * 16;
    using Fn = void (*)(DecodeArgs);
    // D = 256 always takes eight waves (their staging registers would not fit four)
    constexpr int kNarrow = D == 256 ? 8 : 4;
    static const Fn table[2][3] = {
        {lamp_decode_kernel<D, kNarrow, 0>, lamp_decode_kernel<D, kNarrow, 1>, lamp_decode_kernel<D, kNarrow, 2>},
        {lamp_decode_kernel<D, 8, 0>, lamp_decode_kernel<D, 8, 1>, lamp_decode_kernel<D, 8, 2>}};
    const bool wide = a.G > 4 || D == 256;
    const Fn fn = table[wide ? 1 : 0][mode];
    // D <= 128: two tile slots; D = 256: one slot and the mask bytes
    const int lds = D <= 128 ? 2 * DCfg<D, 256>::kLdsBytes : DCfg<D, 256>::kLdsBytes + 8 * a.tps_pad;
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(sh.B * sh.Hkv * sh.n_split), dim3(wide ? 512 : 256), lds, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeShape& sh, const DecodeParams& p, hipStream_t st) {
    if (sh.D == 64) return launch_decode_d<64>(sh, p, st);
    if (sh.D == 128) return launch_decode_d<128>(sh, p, st);
    if (sh.D == 256) return launch_decode_d<256>(sh, p, st);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const DecodeShape& sh, const DecodeParams& p, hipStream_t st) {
    const int rows = sh.B * sh.Hq * sh.Sq;
    hipLaunchKernelGGL(decode_merge_kernel, dim3((rows * (sh.D / 4) + 255) / 256), dim3(256), 0, st, p.part_o,
                       p.part_ml, p.out, rows, sh.Sq, sh.n_split, sh.D);
    return hipGetLastError();
}

}  // namespace lamp
