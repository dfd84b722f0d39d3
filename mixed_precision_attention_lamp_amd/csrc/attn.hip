// Fused LampAttention forward kernel for gfx950 (MI355X).
//
// Method: "LampAttention: Look-Ahead Mixed-Precision FlashAttention for
// Dedicated Accelerators" (abstract).  Per 64x64 tile of (query rows, keys):
//   1. 8-bit logits: e4m3 Q.K^T on the FP8 matrix cores, fp32 accumulation;
//   2. running row max over the 8-bit logits (log2 domain);
//   3. 8-bit exponentials: exp2 rounded to e4m3;
//   4. look-ahead test per 64x16 sub-block (figure 1-8 captions: delta, tau):
//      an entry is sensitive iff p8 >= delta (first stage, off for delta <= 0)
//      and |logit| >= 16 tau log2(e) (second stage); the wave ballots the
//      entries and ORs them into a 4-bit flag set, which is wave-uniform;
//   5. flagged sub-blocks, walked as a dense list of set bits (no divergence),
//      are recomputed from the bf16 inputs on the bf16 matrix cores and their
//      exponentials rounded to bf16 replace the 8-bit ones;
//   6. online-softmax rescale and P.V on the bf16 matrix cores (the row sums
//      come from the same instruction, with an all-ones operand);
//   7. a mask byte per tile records the flags ("16-bit sub-blocks per tile",
//      tables 1-6).
//
// Work decomposition: a workgroup of eight waves shares staged K/V tiles.  A
// pair of waves owns one 64-row query block of one query head (32 rows each,
// so that the fp32 output accumulator stays in architectural registers, where
// the per-row rescale is one multiply); the pair ORs its 4-bit sub-block flags
// through LDS.  The four pairs are four query heads of one GQA group (or fewer
// heads and consecutive row blocks when the group is smaller), so one staged
// K/V tile serves all of them.  Logits are held transposed (keys in rows,
// queries in columns): lane l keeps query l % 16 of each 16-query group, which
// makes the row max a register reduction plus two cross-lane steps and lets
// the exponentials feed the P.V operand in place.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace lamp {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kWaveRows = 32;            // query rows per wave
constexpr int kQG = kWaveRows / 16;      // 16-query groups per wave

struct AttnArgs {
    const uint8_t* q8;
    const uint8_t* k8;
    const uint16_t* q16;
    const uint16_t* k16;
    const uint16_t* vt;
    const float* q_scale;
    const float* k_scale;
    float* out;
    uint8_t* mask;
    float* dump_s;       // debug: [B, Hq, S, S] 8-bit accumulators (or null)
    uint16_t* dump_p;    // debug: [B, Hq, S, S] final bf16 weights (or null)
    double l_d;          // log2(e) / sqrt(D), fp64
    float e_delta;
    float t2;
    int B, Hq, Hkv, S, nT, S_pad;
    int causal, window;
    int G;               // Hq / Hkv
    int heads_per_wg;    // 4, 2 or 1
    int rows_per_wg;     // 4 / heads_per_wg
    int n_rg;            // row-block groups
    int xcd_remap;       // number of workgroups is a multiple of 8
    int n_wg;
};

template <int D>
struct Cfg {
    static constexpr int kK8Stride = D + 16;          // bytes per staged K8 row
    static constexpr int kK16Stride = 2 * D + 16;     // bytes per staged K16 / Q16 row
    static constexpr int kVtStride = 2 * kTileKeys + 16;  // bytes per staged V^T row (64 keys)
    static constexpr int kK8Bytes = kTileKeys * kK8Stride;
    static constexpr int kK16Bytes = kTileKeys * kK16Stride;
    static constexpr int kVtBytes = D * kVtStride;
    static constexpr int kBufBytes = kK8Bytes + kK16Bytes + kVtBytes;
    static constexpr int kQ16Bytes = kWaveRows * kK16Stride;   // per wave
    static constexpr int kLdsBytes = 2 * kBufBytes + kWaves * kQ16Bytes;
    // 16-byte chunks of one staged tile
    static constexpr int kK8Chunks = kTileKeys * D / 16;
    static constexpr int kK16Chunks = kTileKeys * D * 2 / 16;
    static constexpr int kVtChunks = D * kTileKeys * 2 / 16;
    static constexpr int kK8It = (kK8Chunks + kThreads - 1) / kThreads;
    static constexpr int kK16It = (kK16Chunks + kThreads - 1) / kThreads;
    static constexpr int kVtIt = (kVtChunks + kThreads - 1) / kThreads;
    static constexpr int kStage = kK8It + kK16It + kVtIt;
    static constexpr int kDB = D / 16;        // 16-wide output column blocks
    static constexpr int kDC = D / 32;        // 32-deep bf16 matrix-core steps
};

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

// Smallest fp32 a >= 0 with fl32(a * c8) >= t2: then |s| >= t2 for the
// log2-domain logit s = fl32(acc * c8) exactly when |acc| >= a (rounding is
// monotone).  0 when every logit passes, +inf when none can.
__device__ float acc_threshold(float t2, float c8) {
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

template <int D, bool kDump>
__global__ __launch_bounds__(kThreads, 1) void lamp_attn_kernel(AttnArgs a) {
    using C = Cfg<D>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int n16 = lane & 15;     // query column within a 16-query group
    const int g = lane >> 4;       // lane group: which 4 keys / which k-slice
    const int pair = wave >> 1;    // which (head, 64-row block) of the workgroup
    const int half = wave & 1;     // rows 32*half .. 32*half+31 of that block

    // ---- workgroup -> (batch, kv head, head group, row-block group) ----------
    int wg = blockIdx.x;
    if (a.xcd_remap) wg = (wg & 7) * (a.n_wg >> 3) + (wg >> 3);
    const int n_hg = a.G / a.heads_per_wg;
    int u = wg / a.n_rg;
    const int rg = a.n_rg - 1 - (wg % a.n_rg);   // longest (causal) rows first
    const int hg = u % n_hg;
    u /= n_hg;
    const int hk = u % a.Hkv;
    const int b = u / a.Hkv;
    const int hq = hk * a.G + hg * a.heads_per_wg + (pair % a.heads_per_wg);
    const int r = rg * a.rows_per_wg + pair / a.heads_per_wg;
    const bool active = r < a.nT;
    const int r_first = rg * a.rows_per_wg;
    const int r_last = min(r_first + a.rows_per_wg - 1, a.nT - 1);
    const int t_begin = tile_lo(r_first, a.window);
    const int t_end = tile_hi(r_last, a.nT, a.causal);
    const int row0 = r * kTileRows + half * kWaveRows;   // first query row of this wave

    const size_t kv_head = (size_t)b * a.Hkv + hk;
    const size_t q_head = (size_t)b * a.Hq + hq;

    uint8_t* q16_lds = lds + 2 * C::kBufBytes + wave * C::kQ16Bytes;
    __shared__ uint32_t flag_lds[kWaves];    // 4-bit flag sets exchanged by wave pairs

    // ---- prologue: Q16 rows into this wave's LDS, Q8 operand into registers -----
    v8i qf[kQG];
    float m_run[kQG], c8 = 0.0f, a2 = 0.0f;
    const float c16 = (float)a.l_d;
    if (active) {
        constexpr int kChunksPerRow = D / 8;
#pragma unroll
        for (int it = 0; it < kWaveRows * kChunksPerRow / 64; ++it) {
            const int c = lane + it * 64;
            const int row = c / kChunksPerRow, col = c % kChunksPerRow;
            const int gq = row0 + row;
            u32x4 w = {0u, 0u, 0u, 0u};
            if (gq < a.S) w = *reinterpret_cast<const u32x4*>(a.q16 + (q_head * a.S + gq) * D + col * 8);
            *reinterpret_cast<u32x4*>(q16_lds + row * C::kK16Stride + col * 16) = w;
        }
#pragma unroll
        for (int qg = 0; qg < kQG; ++qg) {
            const int row = row0 + qg * 16 + n16;
            const uint8_t* src = a.q8 + (q_head * a.S_pad + row) * D + g * 32;
            u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
            if (g * 32 < D) {
                lo = *reinterpret_cast<const u32x4*>(src);
                hi = *reinterpret_cast<const u32x4*>(src + 16);
            }
            qf[qg] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            m_run[qg] = -__builtin_inff();
        }
        c8 = (float)((double)a.q_scale[q_head] * (double)a.k_scale[kv_head] * a.l_d);
        a2 = acc_threshold(a.t2, c8);
        if (a.mask && half == 0) {
            uint8_t* mrow = a.mask + (q_head * a.nT + r) * a.nT;
            for (int t = lane; t < a.nT; t += 64)
                if (!tile_visited(r, t, a.S, a.causal, a.window)) mrow[t] = 0;
        }
    }

    v4f acc_o[kQG][C::kDB];
    v4f acc_l[kQG];
#pragma unroll
    for (int qg = 0; qg < kQG; ++qg) {
        acc_l[qg] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < C::kDB; ++db) acc_o[qg][db] = v4f{0.f, 0.f, 0.f, 0.f};
    }

    // ---- staging of one KV tile (all threads) ------------------------------------
    // Loads are unconditional (addresses clamped into the tensors) so that they
    // stay in flight together; rows past the end are zeroed when stored to LDS.
    u32x4 stage[C::kStage];
    uint32_t k16_valid = 0;    // bit it: chunk it of K16 lies inside the sequence
    auto stage_load = [&](int t) {
        const uint8_t* k8src = a.k8 + (kv_head * a.S_pad + (size_t)t * kTileKeys) * D;
#pragma unroll
        for (int it = 0; it < C::kK8It; ++it) {
            const int c = min(tid + it * kThreads, C::kK8Chunks - 1);
            stage[it] = *reinterpret_cast<const u32x4*>(k8src + (size_t)c * 16);
        }
        k16_valid = 0;
#pragma unroll
        for (int it = 0; it < C::kK16It; ++it) {
            const int c = min(tid + it * kThreads, C::kK16Chunks - 1);
            const int row = c / (D / 8), col = c % (D / 8);
            const int key = t * kTileKeys + row;
            k16_valid |= (key < a.S ? 1u : 0u) << it;
            const int kc = min(key, a.S - 1);
            stage[C::kK8It + it] = *reinterpret_cast<const u32x4*>(a.k16 + (kv_head * a.S + kc) * D + col * 8);
        }
        const uint16_t* vsrc = a.vt + (kv_head * a.nT + t) * (size_t)D * kTileKeys;
#pragma unroll
        for (int it = 0; it < C::kVtIt; ++it) {
            const int c = min(tid + it * kThreads, C::kVtChunks - 1);
            stage[C::kK8It + C::kK16It + it] = *reinterpret_cast<const u32x4*>(vsrc + (size_t)c * 8);
        }
    };
    auto stage_store = [&](int buf) {
        uint8_t* base = lds + buf * C::kBufBytes;
#pragma unroll
        for (int it = 0; it < C::kK8It; ++it) {
            const int c = tid + it * kThreads;
            const int row = c / (D / 16), col = c % (D / 16);
            if (c < C::kK8Chunks) *reinterpret_cast<u32x4*>(base + row * C::kK8Stride + col * 16) = stage[it];
        }
#pragma unroll
        for (int it = 0; it < C::kK16It; ++it) {
            const int c = tid + it * kThreads;
            const int row = c / (D / 8), col = c % (D / 8);
            u32x4 w = stage[C::kK8It + it];
            if (!((k16_valid >> it) & 1u)) w = u32x4{0u, 0u, 0u, 0u};
            if (c < C::kK16Chunks)
                *reinterpret_cast<u32x4*>(base + C::kK8Bytes + row * C::kK16Stride + col * 16) = w;
        }
#pragma unroll
        for (int it = 0; it < C::kVtIt; ++it) {
            const int c = tid + it * kThreads;
            const int row = c / 8, col = c % 8;
            if (c < C::kVtChunks)
                *reinterpret_cast<u32x4*>(base + C::kK8Bytes + C::kK16Bytes + row * C::kVtStride + col * 16) =
                    stage[C::kK8It + C::kK16It + it];
        }
    };

    // ---- per-tile state carried across the flag exchange ----------------------------
    u32x2 P[kQG][4];          // bf16 weights: keys 16kb + 4g + {0..3}, query 16qg + n16
    float alpha[kQG], m_use[kQG];
    uint32_t vis[kQG];        // masked tiles: bit kb*4+i = entry visible

    // (1)-(4): 8-bit logits, running max, 8-bit exponentials, two-stage test.
    // Returns this wave's 4-bit flag set (wave-uniform).
    auto first_pass = [&](int t, int buf, auto masked_tag) -> uint32_t {
        constexpr bool kMasked = decltype(masked_tag)::value;
        const uint8_t* k8l = lds + buf * C::kBufBytes;

        // (1) s[qg][kb][i] = 8-bit accumulator of key 16kb + 4g + i, query 16qg + n16
        v4f s[kQG][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            v8i ka = {0, 0, 0, 0, 0, 0, 0, 0};
            if (g * 32 < D) {
                const uint8_t* p = k8l + (kb * 16 + n16) * C::kK8Stride + g * 32;
                const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
                const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
                ka = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg)
                s[qg][kb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    ka, qf[qg], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        }

        if constexpr (kDump) {
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg) {
                const int qi = row0 + qg * 16 + n16;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int kj = t * kTileKeys + kb * 16 + g * 4 + i;
                        if (qi < a.S && kj < a.S) a.dump_s[(q_head * a.S + qi) * a.S + kj] = s[qg][kb][i];
                    }
            }
        }

        if constexpr (kMasked) {
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg) {
                vis[qg] = 0u;
                const int qi = row0 + qg * 16 + n16;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int kj = t * kTileKeys + kb * 16 + g * 4 + i;
                        if (pair_visible(qi, kj, a.S, a.causal, a.window)) vis[qg] |= 1u << (kb * 4 + i);
                    }
            }
        }

        // (2) running max in the log2 domain: rounding is monotone, so the max
        //     of the fp32 logits is c8 times the max accumulator, rounded
#pragma unroll
        for (int qg = 0; qg < kQG; ++qg) {
            float mx = -__builtin_inff();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = s[qg][kb][i];
                    if constexpr (kMasked) v = ((vis[qg] >> (kb * 4 + i)) & 1u) ? v : -__builtin_inff();
                    mx = __builtin_fmaxf(mx, v);
                }
            mx = max_over_lane_groups(mx);
            const float mt = mx == -__builtin_inff() ? mx : mx * c8;
            const float mn = __builtin_fmaxf(m_run[qg], mt);
            alpha[qg] = mn == m_run[qg] ? 1.0f : fast_exp2(m_run[qg] - mn);
            m_use[qg] = mn == -__builtin_inff() ? 0.0f : mn;
            m_run[qg] = mn;
        }

        // (3) 8-bit exponentials, (4) first and second stage of the test.  Each
        //     stage is one compare whose lane mask stays in scalar registers.
        uint64_t hit[4] = {0, 0, 0, 0};
#pragma unroll
        for (int qg = 0; qg < kQG; ++qg)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                float e[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e[i] = fast_exp2(__builtin_fmaf(s[qg][kb][i], c8, -m_use[qg]));
                    if constexpr (kMasked) {
                        const bool vv = (vis[qg] >> (kb * 4 + i)) & 1u;
                        e[i] = vv ? e[i] : 0.0f;
                        hit[kb] |= wave_ballot(e[i] >= a.e_delta) & wave_ballot(__builtin_fabsf(s[qg][kb][i]) >= a2) &
                                   wave_ballot(vv);
                    } else {
                        hit[kb] |= wave_ballot(e[i] >= a.e_delta) & wave_ballot(__builtin_fabsf(s[qg][kb][i]) >= a2);
                    }
                }
                const uint32_t w = cvt_pk_e4m3_unit<true>(e[2], e[3], cvt_pk_e4m3_unit<false>(e[0], e[1], 0u));
                P[qg][kb] = u32x2{e4m3x2_to_bf16x2<false>(w), e4m3x2_to_bf16x2<true>(w)};
            }
        uint32_t flags = 0;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) flags |= (hit[kb] != 0 ? 1u : 0u) << kb;
        return flags;
    };

    // (5)-(7): 16-bit recompute of the flagged sub-blocks, rescale, P.V, mask byte.
    auto second_pass = [&](int t, int buf, uint32_t flags, auto masked_tag) {
        constexpr bool kMasked = decltype(masked_tag)::value;
        const uint8_t* k16l = lds + buf * C::kBufBytes + C::kK8Bytes;
        const uint8_t* vtl = k16l + C::kK16Bytes;

        // (5) flagged sub-blocks.  The flag set is wave-uniform (scalar), so each
        //     sub-block is either skipped or recomputed by the whole wave with a
        //     scalar branch: no lane diverges, and the register tile P is
        //     addressed with compile-time indices.
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (!((flags >> c) & 1u)) continue;
            v8bf ka[C::kDC];
#pragma unroll
            for (int ch = 0; ch < C::kDC; ++ch)
                ka[ch] = *reinterpret_cast<const v8bf*>(k16l + (c * 16 + n16) * C::kK16Stride + (ch * 32 + g * 8) * 2);
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg) {
                v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ch = 0; ch < C::kDC; ++ch) {
                    const v8bf qb = *reinterpret_cast<const v8bf*>(q16_lds + (qg * 16 + n16) * C::kK16Stride + (ch * 32 + g * 8) * 2);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ch], qb, acc, 0, 0, 0);
                }
                float e[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e[i] = fast_exp2(__builtin_fmaf(acc[i], c16, -m_use[qg]));
                    if constexpr (kMasked) e[i] = ((vis[qg] >> (c * 4 + i)) & 1u) ? e[i] : 0.0f;
                }
                P[qg][c] = u32x2{f32x2_to_bf16x2(e[0], e[1]), f32x2_to_bf16x2(e[2], e[3])};
            }
        }

        if constexpr (kDump) {
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg) {
                const int qi = row0 + qg * 16 + n16;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int kj = t * kTileKeys + kb * 16 + g * 4 + i;
                        const uint32_t w = P[qg][kb][i / 2];
                        if (qi < a.S && kj < a.S)
                            a.dump_p[(q_head * a.S + qi) * a.S + kj] = (uint16_t)((i & 1) ? (w >> 16) : (w & 0xFFFFu));
                    }
            }
        }

        // (6) online-softmax rescale, then P.V and the row sums
        bool rescale = false;
#pragma unroll
        for (int qg = 0; qg < kQG; ++qg) rescale |= alpha[qg] != 1.0f;
        if (wave_ballot(rescale) != 0) {
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg) {
                acc_l[qg] *= alpha[qg];
#pragma unroll
                for (int db = 0; db < C::kDB; ++db) acc_o[qg][db] *= alpha[qg];
            }
        }
        const v8bf ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                           (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v8bf pb[kQG];
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg) {
                const u32x4 w = {P[qg][2 * h][0], P[qg][2 * h][1], P[qg][2 * h + 1][0], P[qg][2 * h + 1][1]};
                pb[qg] = __builtin_bit_cast(v8bf, w);
            }
#pragma unroll
            for (int db = 0; db < C::kDB; ++db) {
                const v8bf va = *reinterpret_cast<const v8bf*>(vtl + (db * 16 + n16) * C::kVtStride + h * 64 + g * 16);
#pragma unroll
                for (int qg = 0; qg < kQG; ++qg)
                    acc_o[qg][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[qg], acc_o[qg][db], 0, 0, 0);
            }
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg)
                acc_l[qg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[qg], acc_l[qg], 0, 0, 0);
        }

        // (7) mask byte
        if (a.mask && half == 0 && lane == 0)
            a.mask[(q_head * a.nT + r) * a.nT + t] = (uint8_t)(0x80u | flags);
    };

    // ---- main loop over the workgroup's KV tiles (double-buffered staging) -----
    stage_load(t_begin);
    stage_store(0);
    __syncthreads();
    for (int t = t_begin; t <= t_end; ++t) {
        const int buf = (t - t_begin) & 1;
        const bool has_next = t < t_end;
        if (has_next) stage_load(t + 1);
        const bool work = active && tile_visited(r, t, a.S, a.causal, a.window);
        const bool full = tile_full(r, t, a.S, a.causal, a.window);
        uint32_t flags = 0;
        if (work) {
            if (full) flags = first_pass(t, buf, std::integral_constant<bool, false>{});
            else flags = first_pass(t, buf, std::integral_constant<bool, true>{});
        }
        // the two waves of a 64-row block OR their flags
        if (lane == 0) flag_lds[wave] = flags;
        lds_barrier();
        flags |= flag_lds[wave ^ 1];
        if (work) {
            if (full) second_pass(t, buf, flags, std::integral_constant<bool, false>{});
            else second_pass(t, buf, flags, std::integral_constant<bool, true>{});
        }
        if (has_next) stage_store(buf ^ 1);
        lds_barrier();
    }

    // ---- epilogue: out = O / l ------------------------------------------------------
    if (active) {
#pragma unroll
        for (int qg = 0; qg < kQG; ++qg) {
            const int qi = row0 + qg * 16 + n16;
            if (qi < a.S) {
                const float inv_l = 1.0f / acc_l[qg][0];
                float* dst = a.out + (q_head * a.S + qi) * D + g * 4;
#pragma unroll
                for (int db = 0; db < C::kDB; ++db)
                    *reinterpret_cast<v4f*>(dst + db * 16) = acc_o[qg][db] * inv_l;
            }
        }
    }
}

template <int D>
hipError_t launch_d(const Shape& sh, const AttnParams& p, hipStream_t st) {
    AttnArgs a;
    a.q8 = p.q8; a.k8 = p.k8; a.q16 = p.q16; a.k16 = p.k16; a.vt = p.vt;
    a.q_scale = p.q_scale; a.k_scale = p.k_scale; a.out = p.out; a.mask = p.mask;
    a.dump_s = p.dump_s; a.dump_p = p.dump_p;
    a.l_d = p.log2e_over_sqrt_d; a.e_delta = p.e_delta; a.t2 = p.t2;
    a.B = sh.B; a.Hq = sh.Hq; a.Hkv = sh.Hkv; a.S = sh.S; a.nT = sh.nT; a.S_pad = sh.S_pad;
    a.causal = p.causal; a.window = p.window;
    a.G = sh.Hq / sh.Hkv;
    a.heads_per_wg = (a.G % 4 == 0) ? 4 : (a.G % 2 == 0) ? 2 : 1;
    a.rows_per_wg = 4 / a.heads_per_wg;
    a.n_rg = (sh.nT + a.rows_per_wg - 1) / a.rows_per_wg;
    a.n_wg = sh.B * sh.Hkv * (a.G / a.heads_per_wg) * a.n_rg;
    a.xcd_remap = (a.n_wg % 8 == 0) ? 1 : 0;
    const size_t lds = Cfg<D>::kLdsBytes;
    const bool dump = p.dump_s != nullptr && p.dump_p != nullptr;
    const void* fn = dump ? (const void*)lamp_attn_kernel<D, true> : (const void*)lamp_attn_kernel<D, false>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (dump)
        hipLaunchKernelGGL((lamp_attn_kernel<D, true>), dim3(a.n_wg), dim3(kThreads), lds, st, a);
    else
        hipLaunchKernelGGL((lamp_attn_kernel<D, false>), dim3(a.n_wg), dim3(kThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const Shape& sh, const AttnParams& p, hipStream_t st) {
    if (sh.D == 64) return launch_d<64>(sh, p, st);
    if (sh.D == 128) return launch_d<128>(sh, p, st);
    return hipErrorInvalidValue;
}

}  // namespace lamp
