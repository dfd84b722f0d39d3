// Fused LampAttention forward kernel for gfx950 (MI355X), head dimension 256:
// the variant with the 16-bit work deferred to after the tile loop.  (For
// D <= 128 the kernel in attn.hip recomputes flagged sub-blocks inside the
// loop; at D = 256 its LDS staging of the 16-bit operands does not fit.)
//
// Method: "LampAttention: Look-Ahead Mixed-Precision FlashAttention for
// Dedicated Accelerators" (abstract).  Per 64x64 tile of (query rows, keys):
//   1. 8-bit logits: e4m3 Q.K^T on the FP8 matrix cores, fp32 accumulation;
//   2. running row max over the 8-bit logits (log2 domain);
//   3. 8-bit exponentials: exp2 rounded to e4m3;
//   4. look-ahead test per 64x16 sub-block (figure 1-8 captions: delta, tau):
//      an entry is sensitive iff p8 >= delta (first stage, off for delta <= 0)
//      and |logit| >= 16 tau log2(e) (second stage); each wave ballots its
//      entries into a 4-bit flag set, and the waves of a 64-row block OR theirs;
//   5. flagged sub-blocks get bf16 logits from the bf16 inputs and exponentials
//      rounded to bf16 in place of the 8-bit ones;
//   6. online-softmax rescale and P.V on the bf16 matrix cores (the row sums
//      come from the same instruction, with an all-ones operand);
//   7. a mask byte per tile records the flags ("16-bit sub-blocks per tile",
//      tables 1-6).
//
// Step 5 is applied after the tile loop, as a correction.  The running max
// comes from the 8-bit logits alone, so the 8-bit weights, the flags and the
// max after every tile do not depend on step 5.  The loop therefore
// accumulates O and l from the 8-bit weights everywhere and records, for each
// flagged tile, the tile index, its flags and the max m_t of every row; after
// the loop each wave walks its block's records and adds, for every flagged
// sub-block, 2^(m_t - m_final) (P16 - P8).V and the matching row sums, where
// P8 is recomputed with the same instructions on the same operands (hence
// bit-identical to the loop's) and P16 comes from the bf16 matrix cores.  In
// exact arithmetic this is the same sum as splicing P16 in before the P.V of
// the tile; the fp32 rounding differs (order, and a relative 2^-17 on the
// scaled differences, which enter the matrix cores as two bf16 terms).  The point: the correction
// needs no LDS staging and no barrier, so waves whose rows flag different
// sub-blocks no longer wait for each other at every tile, and the tile loop
// has no data-dependent branch.
//
// Schedule of the tile loop: in the iteration of tile t a wave first issues
// the P.V products of tile t-1, which run on the matrix cores under the vector
// work of tile t (max, exponentials, 8-bit rounding); after the sub-block test
// it issues the Q.K^T products of tile t+1, which run under the rescale, the
// LDS stores and the barrier, the only one per tile.  K8 and V^T tiles are
// staged through registers into unpadded LDS layouts whose 16-byte chunks are
// XOR-swizzled by row (conflict-free operand reads), two slots each: K8 runs
// two tiles ahead, V^T zero.  Each wave keeps its Q8 rows in LDS.
//
// Work decomposition: a workgroup of eight waves shares the staged K/V tiles.
// A wave owns 32 query rows (16 when D = 256, so that the fp32 output
// accumulator stays in architectural registers, where the per-row rescale is
// one multiply); the 2 (or 4) waves of one 64-row query block exchange their
// flag sets through LDS at the next barrier.  The 4 (or 2) blocks of a
// workgroup are query heads of one GQA group (or fewer heads and consecutive
// row blocks when the group is smaller), so one staged K/V tile serves all of
// them.  Logits are held transposed (keys in rows, queries in columns): lane l
// keeps query l % 16 of each 16-query group, which makes the row max a
// register reduction plus two cross-lane steps and lets the exponentials feed
// the P.V operand in place.
#include <hip/hip_runtime.h>

#include <cmath>

#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace lamp {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

struct AttnArgs {
    const uint8_t* q8;
    const uint8_t* k8;
    const uint16_t* q16;
    const uint16_t* k16;
    const uint16_t* vt;
    const uint16_t* vsb;
    const float* q_scale;
    const float* k_scale;
    float* out;
    uint8_t* mask;
    float* rec_m;        // per-tile row maxima of flagged tiles (see rec_slot_base)
    float* dump_s;       // debug: [B, Hq, S, S] 8-bit accumulators (or null)
    uint16_t* dump_p;    // debug: [B, Hq, S, S] final bf16 weights (or null)
    double l_d;          // log2(e) / sqrt(D), fp64
    float x_delta;       // first stage: exp2 argument threshold (log2 of the e4m3 boundary)
    float t2;
    int test_mode;       // 0: no test (second stage off), 1: both stages, 2: second stage only
    int B, Hq, Hkv, S, nT, S_pad;
    int causal, window;
    int G;               // Hq / Hkv
    int heads_per_wg;    // query heads per workgroup
    int rows_per_wg;     // 64-row blocks per head and workgroup
    int n_rg;            // row-block groups
    int xcd_remap;       // number of workgroups is a multiple of 8
    int n_wg;
    int64_t rec_per_head;  // record slots per (batch, query head)
};

template <int D>
struct Cfg {
    static constexpr int kQG = D == 256 ? 1 : 2;          // 16-query groups per wave
    static constexpr int kWaveRows = 16 * kQG;
    static constexpr int kWavesPerBlock = kTileRows / kWaveRows;
    static constexpr int kBlocks = kWaves / kWavesPerBlock;   // 64-row blocks per workgroup
    static constexpr int kK8Row = D;                      // bytes per staged row
    static constexpr int kVtRow = 2 * kTileKeys;
    static constexpr int kK8Bytes = kTileKeys * kK8Row;
    static constexpr int kVtBytes = D * kVtRow;
    // Q8 rows stay in LDS, except for D = 256, where they stay in registers
    // (16 rows per wave leave room) and the LDS holds two 32 KB V^T slots
    static constexpr bool kQ8Lds = D != 256;
    static constexpr int kQ8Bytes = kQ8Lds ? kWaveRows * kK8Row : 0;   // per wave
    static constexpr int kK8Off = 0;                      // two slots each
    static constexpr int kVtOff = 2 * kK8Bytes;
    static constexpr int kQ8Off = kVtOff + 2 * kVtBytes;
    static constexpr int kListOff = kQ8Off + kWaves * kQ8Bytes;   // per-block record lists
    // after the tile loop the staging slots hold each wave's Q16 rows for the
    // 16-bit correction when they fit (D >= 128); for D = 64 they stay in registers
    static constexpr int kQ16Row = 2 * D;
    static constexpr int kQ16Bytes = kWaveRows * kQ16Row;   // per wave
    static constexpr bool kQ16Lds = kWaves * kQ16Bytes <= kQ8Off;
    static constexpr int kDB = D / 16;        // 16-wide output column blocks
    static constexpr int kDC = D / 32;        // 32-deep bf16 matrix-core steps
    static constexpr int kKS = D >= 128 ? D / 128 : 1;   // 128-deep FP8 matrix-core steps
};

typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

// kMode: 0 = no test (second stage off), 1 = both stages, 2 = second stage only.
template <int D, bool kDump, int kMode>
__global__ __launch_bounds__(kThreads, 1) void lamp_attn_kernel(AttnArgs a) {
    using C = Cfg<D>;
    constexpr int kQG = C::kQG;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ uint32_t flag_ring[2][kWaves];   // 4-bit flag sets of the last two tiles
    __shared__ int list_len[C::kBlocks];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int n16 = lane & 15;     // query column within a 16-query group
    const int g = lane >> 4;       // lane group: which 4 keys / which k-slice
    const int blk = wave / C::kWavesPerBlock;   // which (head, 64-row block) of the workgroup
    const int wib = wave % C::kWavesPerBlock;   // rows wib*kWaveRows .. of that block

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
    const int hq = hk * a.G + hg * a.heads_per_wg + (blk % a.heads_per_wg);
    const int r = rg * a.rows_per_wg + blk / a.heads_per_wg;
    const bool active = r < a.nT;
    const int r_first = rg * a.rows_per_wg;
    const int r_last = min(r_first + a.rows_per_wg - 1, a.nT - 1);
    const int t_begin = tile_lo(r_first, a.window);
    const int t_end = tile_hi(r_last, a.nT, a.causal);
    const int row0 = r * kTileRows + wib * C::kWaveRows;   // first query row of this wave

    const size_t kv_head = (size_t)b * a.Hkv + hk;
    const size_t q_head = (size_t)b * a.Hq + hq;

    uint8_t* q8_lds = lds + C::kQ8Off + wave * C::kQ8Bytes;
    uint16_t* list = reinterpret_cast<uint16_t*>(lds + C::kListOff) + blk * a.nT;
    // record slots of this block: one record of 64 row maxima per flagged tile
    float* rec = a.rec_m + ((int64_t)q_head * a.rec_per_head +
                            rec_slot_base(active ? r : 0, a.nT, a.causal, a.window)) * kTileRows;

    // ---- staging: register loads at the start of an iteration, LDS stores at its end
    // Thread tid owns the 16-byte chunks tid + kThreads*i of a tile, i.e. LDS
    // bytes [16 c, 16 c + 16) of the swizzled layout, and loads the global chunk
    // that belongs there.
    constexpr int kK8Ch = C::kK8Bytes / 16 / kThreads;     // chunks per thread and tile
    constexpr int kVtCh = C::kVtBytes / 16 / kThreads;
    static_assert(kVtCh >= 1, "tile smaller than one chunk per thread");
    constexpr int kK8ChMin = kK8Ch > 0 ? kK8Ch : 1;
    u32x4 st_k8[kK8ChMin], st_vt[kVtCh];
    auto load_k8 = [&](int t) __attribute__((always_inline)) {
        const uint8_t* src = a.k8 + (kv_head * a.S_pad + (size_t)t * kTileKeys) * D;
        constexpr int kNC = C::kK8Row / 16;
#pragma unroll
        for (int i = 0; i < kK8ChMin; ++i) {
            const int p = min((tid + i * kThreads) * 16, C::kK8Bytes - 16);
            const int row = p / C::kK8Row, slot = (p % C::kK8Row) >> 4;
            st_k8[i] = *reinterpret_cast<const u32x4*>(src + row * C::kK8Row + ((slot ^ swz<kNC>(row)) << 4));
        }
    };
    auto store_k8 = [&](int t) __attribute__((always_inline)) {
        uint8_t* base = lds + C::kK8Off + (t & 1) * C::kK8Bytes;
#pragma unroll
        for (int i = 0; i < kK8ChMin; ++i) {
            const int p = (tid + i * kThreads) * 16;
            if (p < C::kK8Bytes) *reinterpret_cast<u32x4*>(base + p) = st_k8[i];
        }
    };
    auto load_vt = [&](int t) __attribute__((always_inline)) {
        const uint8_t* src = reinterpret_cast<const uint8_t*>(a.vt + (kv_head * a.nT + t) * (size_t)D * kTileKeys);
        constexpr int kNC = C::kVtRow / 16;
#pragma unroll
        for (int i = 0; i < kVtCh; ++i) {
            const int p = (tid + i * kThreads) * 16;
            const int row = p / C::kVtRow, slot = (p % C::kVtRow) >> 4;
            st_vt[i] = *reinterpret_cast<const u32x4*>(src + row * C::kVtRow + ((slot ^ swz<kNC>(row)) << 4));
        }
    };
    auto store_vt = [&](int t) __attribute__((always_inline)) {
        uint8_t* base = lds + C::kVtOff + (t & 1) * C::kVtBytes;
#pragma unroll
        for (int i = 0; i < kVtCh; ++i) *reinterpret_cast<u32x4*>(base + (tid + i * kThreads) * 16) = st_vt[i];
    };

    // ---- prologue: this wave's Q8 rows into its LDS (or registers) -----------------
    float m_run[kQG], c8 = 0.0f, inv_c8 = 0.0f, a2 = 0.0f;
    const float c16 = (float)a.l_d;
    v8i qf_reg[C::kQ8Lds ? 1 : kQG][C::kKS];
    if constexpr (C::kQ8Lds) {
        constexpr int kNC = C::kK8Row / 16;
        const int qmax = a.S_pad - 1;
#pragma unroll
        for (int i = 0; i < C::kQ8Bytes / 1024; ++i) {
            const int p = i * 1024 + lane * 16;
            const int row = p / C::kK8Row, slot = (p % C::kK8Row) >> 4;
            const int gq = min(row0 + row, qmax);
            *reinterpret_cast<u32x4*>(q8_lds + p) = *reinterpret_cast<const u32x4*>(
                a.q8 + (q_head * a.S_pad + gq) * D + ((slot ^ swz<kNC>(row)) << 4));
        }
    } else {
#pragma unroll
        for (int qg = 0; qg < kQG; ++qg)
#pragma unroll
            for (int st = 0; st < C::kKS; ++st)
                qf_reg[qg][st] = fp8_operand_global<D>(
                    a.q8 + (q_head * a.S_pad + min(row0 + qg * 16 + n16, a.S_pad - 1)) * D, st, g);
    }
    // the Q8 operand of 16-query group qg, 128-deep step st
    auto q8_operand = [&](int qg, int st) __attribute__((always_inline)) -> v8i {
        if constexpr (C::kQ8Lds) return fp8_operand<D>(q8_lds, qg * 16 + n16, st, g);
        else return qf_reg[C::kQ8Lds ? 0 : qg][st];
    };
#pragma unroll
    for (int qg = 0; qg < kQG; ++qg) m_run[qg] = -__builtin_inff();
    if (active) {
        c8 = (float)((double)a.q_scale[q_head] * (double)a.k_scale[kv_head] * a.l_d);
        a2 = acc_threshold(a.t2, c8);
        inv_c8 = 1.0f / c8;
        if (a.mask && wib == 0) {
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

    auto work = [&](int t) __attribute__((always_inline)) {
        return active && t >= t_begin && t <= t_end && tile_visited(r, t, a.S, a.causal, a.window);
    };

    // ---- matrix-core phases ---------------------------------------------------------
    // Q.K^T of tile t: s[qg][kb][i] = 8-bit accumulator of key 16kb + 4g + i, query 16qg + n16
    auto qk = [&](v4f (&s)[kQG][4], int t) __attribute__((always_inline)) {
        const uint8_t* k8l = lds + C::kK8Off + (t & 1) * C::kK8Bytes;
#pragma unroll
        for (int st = 0; st < C::kKS; ++st) {
            v8i qf[kQG];
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg) qf[qg] = q8_operand(qg, st);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const v8i ka = fp8_operand<D>(k8l, kb * 16 + n16, st, g);
#pragma unroll
                for (int qg = 0; qg < kQG; ++qg)
                    s[qg][kb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        ka, qf[qg], st == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : s[qg][kb], 0, 0, 0, 0, 0, 0);
            }
        }
    };
    // P.V of the staged tile (and the row sums, with an all-ones operand)
    const v8bf ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                       (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
    auto pv = [&](const u32x2 (&P)[kQG][4], int t) __attribute__((always_inline)) {
        const uint8_t* vtl = lds + C::kVtOff + (t & 1) * C::kVtBytes;
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
                const v8bf va = *reinterpret_cast<const v8bf*>(vtl + lds_off<C::kVtRow>(db * 16 + n16, h * 4 + g));
#pragma unroll
                for (int qg = 0; qg < kQG; ++qg)
                    acc_o[qg][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[qg], acc_o[qg][db], 0, 0, 0);
            }
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg)
                acc_l[qg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[qg], acc_l[qg], 0, 0, 0);
        }
    };

    // ---- per-tile vector state ---------------------------------------------------------
    float alpha[kQG], m_use[kQG];
    float smax[kQG][4];                 // per (lane, sub-block) maxima of the 8-bit accumulators
    float smin[kMode == 2 ? kQG : 1][4];    // and minima, when the first stage is off
    uint32_t vis[kQG];                  // masked tiles: bit kb*4+i = entry visible
#pragma unroll
    for (int qg = 0; qg < kQG; ++qg) m_use[qg] = 0.0f;

    // (2)-(3): running max and 8-bit exponentials of tile t, straight-line code.
    auto softmax = [&](const v4f (&s)[kQG][4], u32x2 (&P)[kQG][4], int t, auto masked_tag) __attribute__((always_inline)) {
        constexpr bool kMasked = decltype(masked_tag)::value;
        constexpr float kNegInf = -__builtin_inff();
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
                        vis[qg] |= (pair_visible(qi, kj, a.S, a.causal, a.window) ? 1u : 0u) << (kb * 4 + i);
                    }
            }
        }
        // running max in the log2 domain: rounding is monotone, so the max of
        // the fp32 logits is c8 times the max accumulator, rounded
#pragma unroll
        for (int qg = 0; qg < kQG; ++qg) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                float v[4], w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[i] = w[i] = s[qg][kb][i];
                    if constexpr (kMasked) {
                        const bool vv = (vis[qg] >> (kb * 4 + i)) & 1u;
                        v[i] = vv ? v[i] : kNegInf;
                        w[i] = vv ? w[i] : -kNegInf;
                    }
                }
                smax[qg][kb] = __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), __builtin_fmaxf(v[2], v[3]));
                if constexpr (kMode == 2)
                    smin[qg][kb] = __builtin_fminf(__builtin_fminf(w[0], w[1]), __builtin_fminf(w[2], w[3]));
            }
            float mx = __builtin_fmaxf(__builtin_fmaxf(smax[qg][0], smax[qg][1]),
                                       __builtin_fmaxf(smax[qg][2], smax[qg][3]));
            mx = max_over_lane_groups(mx);
            const float mt = mx == kNegInf ? mx : mx * c8;
            const float mn = __builtin_fmaxf(m_run[qg], mt);
            alpha[qg] = mn == m_run[qg] ? 1.0f : fast_exp2(m_run[qg] - mn);
            m_use[qg] = mn == kNegInf ? 0.0f : mn;
            m_run[qg] = mn;
        }
        // 8-bit exponentials against the running max
#pragma unroll
        for (int qg = 0; qg < kQG; ++qg)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                float e[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e[i] = fast_exp2(__builtin_fmaf(s[qg][kb][i], c8, -m_use[qg]));
                    if constexpr (kMasked) e[i] = ((vis[qg] >> (kb * 4 + i)) & 1u) ? e[i] : 0.0f;
                }
                const uint32_t w = cvt_pk_e4m3_unit<true>(e[2], e[3], cvt_pk_e4m3_unit<false>(e[0], e[1], 0u));
                P[qg][kb] = u32x2{e4m3x2_to_bf16x2<false>(w), e4m3x2_to_bf16x2<true>(w)};
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
                        if (qi < a.S && kj < a.S) {
                            const size_t at = (q_head * a.S + qi) * a.S + kj;
                            a.dump_s[at] = s[qg][kb][i];
                            const uint32_t w = P[qg][kb][i / 2];
                            a.dump_p[at] = (uint16_t)((i & 1) ? (w >> 16) : (w & 0xFFFFu));
                        }
                    }
            }
        }
    };

    // (4): the look-ahead test on the accumulators of tile t; returns the wave's
    // 4-bit flag set (wave-uniform).  First stage: the 8-bit exponential is at
    // least delta, i.e. its argument x = acc c8 - m is at least x_delta, i.e.
    // acc >= a1 = (x_delta + m) / c8.  Second stage: |acc| >= a2.  When
    // a1 > -a2 both hold iff acc >= max(a1, a2), so a sub-block holds a
    // sensitive entry of this row iff its maximum does: one compare per (lane,
    // sub-block).  Rows with a1 <= -a2 (a very negative running max) fall back
    // to a per-entry test for the wave.
    auto test = [&](const v4f (&s)[kQG][4], bool masked) __attribute__((always_inline)) -> uint32_t {
        uint64_t hit[4] = {0, 0, 0, 0};
        if constexpr (kMode == 1) {
            bool slow = false;
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg) {
                const float a1 = (a.x_delta + m_use[qg]) * inv_c8;
                const float thr = __builtin_fmaxf(a1, a2);
                slow |= a1 <= -a2;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) hit[kb] |= wave_ballot(smax[qg][kb] >= thr);
            }
            if (wave_ballot(slow) != 0) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) hit[kb] = 0;
#pragma unroll
                for (int qg = 0; qg < kQG; ++qg)
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float v = s[qg][kb][i];
                            bool sens = __builtin_fmaf(v, c8, -m_use[qg]) >= a.x_delta;
                            sens = sens && __builtin_fabsf(v) >= a2;
                            if (masked) sens = sens && ((vis[qg] >> (kb * 4 + i)) & 1u);
                            hit[kb] |= wave_ballot(sens);
                        }
            }
        } else if constexpr (kMode == 2) {
            // first stage off: every visible entry is active; |acc| >= a2 holds
            // for some entry iff the sub-block maximum or minus its minimum does
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    hit[kb] |= wave_ballot(smax[qg][kb] >= a2) | wave_ballot(smin[qg][kb] <= -a2);
        }
        uint32_t flags = 0;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) flags |= (hit[kb] != 0 ? 1u : 0u) << kb;
        return flags;
    };

    // The flags of tile t, ORed over the waves of this block (read after the
    // barrier that follows their writes).  A flagged tile gets a record: its
    // index and flags in the block's LDS list, the row maxima it used (still
    // in m_use) in the block's global record slot.  The block's first wave
    // writes the mask byte.
    int n_rec = 0;
    auto finish_tile = [&](int t) __attribute__((always_inline)) {
        uint32_t f = 0;
#pragma unroll
        for (int w = 0; w < C::kWavesPerBlock; ++w) f |= flag_ring[t & 1][blk * C::kWavesPerBlock + w];
        if (f != 0) {
            float* dst = rec + (int64_t)n_rec * kTileRows + wib * C::kWaveRows;
            if (g == 0) {
#pragma unroll
                for (int qg = 0; qg < kQG; ++qg) dst[qg * 16 + n16] = m_use[qg];
            }
            if (wib == 0 && lane == 0) list[n_rec] = (uint16_t)(t | (f << 12));
            ++n_rec;
        }
        if (a.mask && wib == 0 && lane == 0) a.mask[(q_head * a.nT + r) * a.nT + t] = (uint8_t)(0x80u | f);
    };

    // ---- prologue staging and the first tile's Q.K^T ------------------------------
    v4f S[kQG][4];
    u32x2 P[kQG][4];
    load_k8(t_begin);
    store_k8(t_begin);
    if (t_begin + 1 <= t_end) {
        load_k8(t_begin + 1);
        store_k8(t_begin + 1);
    }
    lds_barrier();
    if (work(t_begin)) qk(S, t_begin);
    lds_barrier();   // every wave has read K8(t_begin) before its slot is refilled

    // ---- the pipelined loop ---------------------------------------------------------
    for (int t = t_begin; t <= t_end; ++t) {
        const bool ld_k8 = t + 2 <= t_end;
        const bool w_prev = work(t - 1), w_cur = work(t), w_next = work(t + 1);
        const bool full = tile_full(r, t, a.S, a.causal, a.window);
        // flags of tile t-1 (m_use still holds its row maxima)
        if (w_prev) finish_tile(t - 1);
        // P.V of tile t-1 is issued first (it reads P before the exponentials
        // of tile t overwrite it) and runs on the matrix cores under the
        // vector work of tile t
        if (w_prev) pv(P, t - 1);
        if (w_cur) {
            if (full) softmax(S, P, t, std::integral_constant<bool, false>{});
            else softmax(S, P, t, std::integral_constant<bool, true>{});
        }
        // loads for later tiles, stored to LDS before the barrier that ends this
        // iteration
        if (ld_k8) load_k8(t + 2);
        load_vt(t);
        const uint32_t flags = w_cur ? test(S, !full) : 0u;
        if (lane == 0) flag_ring[t & 1][wave] = flags;
        // Q.K^T of tile t+1 runs on the matrix cores under what follows
        if (w_next) qk(S, t + 1);
        if (w_cur) {
            // (6) online-softmax rescale of everything accumulated so far (the
            //     P.V of tile t-1 included), before the P.V of tile t
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg) {
                if (wave_ballot(alpha[qg] != 1.0f) != 0) {
                    acc_l[qg] *= alpha[qg];
#pragma unroll
                    for (int db = 0; db < C::kDB; ++db) acc_o[qg][db] *= alpha[qg];
                }
            }
        }
        // K8 of tile t+2 into the slot Q.K^T of tile t used, V^T of tile t into
        // the slot the P.V of tile t-2 used (both read before the previous
        // barrier); the other slots may still be in use by slower waves
        if (ld_k8) store_k8(t + 2);
        store_vt(t);
        lds_barrier();
    }
    // P.V and the flags of the last tile
    if (work(t_end)) {
        pv(P, t_end);
        finish_tile(t_end);
    }
    if (wib == 0 && lane == 0) list_len[blk] = n_rec;
    // this wave's record stores have landed, and the block's list is complete
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __syncthreads();

    // ---- (5) 16-bit correction of the flagged sub-blocks -------------------------------
    // The block's records expand into items (tile, sub-block), walked in
    // order with the K operands of the next item in flight while the current
    // one computes; every step is wave-uniform control flow, with no barrier.
    // Per item the wave adds scale * (P16 - P8).V to O and the row sums to l,
    // scale = 2^(m_t - m_final) per row.  The fp32 value scale * (P16 - P8)
    // enters the bf16 matrix cores as a sum of two bf16 terms (hi, and lo =
    // the rest, rounded), which carries it to a relative 2^-17 of itself (the
    // whole correction is at most about a sixteenth of the weight).
    const int n_list = active ? list_len[blk] : 0;
    if (n_list > 0) {
        const int smax_row = a.S - 1;
        // this wave's Q16 operand: LDS (the free staging slots) or registers
        uint8_t* q16_lds = lds + wave * C::kQ16Bytes;
        v8bf qb_reg[C::kQ16Lds ? 1 : C::kDC][kQG];
#pragma unroll
        for (int qg = 0; qg < kQG; ++qg) {
            const uint16_t* qrow = a.q16 + (q_head * a.S + min(row0 + qg * 16 + n16, smax_row)) * D;
#pragma unroll
            for (int ch = 0; ch < C::kDC; ++ch) {
                const v8bf x = *reinterpret_cast<const v8bf*>(qrow + ch * 32 + g * 8);
                if constexpr (C::kQ16Lds)
                    *reinterpret_cast<v8bf*>(q16_lds + lds_off<C::kQ16Row>(qg * 16 + n16, ch * 4 + g)) = x;
                else
                    qb_reg[ch][qg] = x;
            }
        }
        auto q16_operand = [&](int ch, int qg) __attribute__((always_inline)) -> v8bf {
            if constexpr (C::kQ16Lds)
                return *reinterpret_cast<const v8bf*>(q16_lds + lds_off<C::kQ16Row>(qg * 16 + n16, ch * 4 + g));
            else
                return qb_reg[C::kQ16Lds ? 0 : ch][qg];
        };
        const uint8_t* k8h = a.k8 + kv_head * a.S_pad * D;
        const uint16_t* k16h = a.k16 + kv_head * a.S * D;
        const uint16_t* vsh = a.vsb + kv_head * a.nT * (size_t)D * kTileKeys;
        const v4bf ones4 = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};

        // item cursor: record k and its remaining flag bits (scalar registers)
        struct Item { int k, t, c; };
        int cur_k = 0;
        uint32_t cur_e = __builtin_amdgcn_readfirstlane((uint32_t)list[0]);
        uint32_t cur_bits = cur_e >> 12;
        auto next_item = [&](Item& it) __attribute__((always_inline)) -> bool {
            while (cur_bits == 0 && cur_k + 1 < n_list) {
                ++cur_k;
                cur_e = __builtin_amdgcn_readfirstlane((uint32_t)list[cur_k]);
                cur_bits = cur_e >> 12;
            }
            if (cur_bits == 0) return false;
            it.k = cur_k;
            it.t = (int)(cur_e & 0xFFFu);
            it.c = __builtin_ctz(cur_bits);
            cur_bits &= cur_bits - 1;
            return true;
        };
        // the operands needed first: K8 (and, while registers allow, K16) rows of
        // the sub-block, record maxima
        constexpr bool kPreK16 = D <= 128;
        struct KOps {
            v8i k8[C::kKS];
            v8bf k16[kPreK16 ? C::kDC : 1];
            float m[kQG];
        };
        auto load_k = [&](const Item& it, KOps& o) __attribute__((always_inline)) {
            const int key = it.t * kTileKeys + it.c * 16 + n16;
#pragma unroll
            for (int st = 0; st < C::kKS; ++st) o.k8[st] = fp8_operand_global<D>(k8h + (size_t)key * D, st, g);
            if constexpr (kPreK16) {
                // keys past the end reload the last key: they are masked
                const uint16_t* krow = k16h + (size_t)min(key, smax_row) * D;
#pragma unroll
                for (int ch = 0; ch < C::kDC; ++ch)
                    o.k16[ch] = *reinterpret_cast<const v8bf*>(krow + ch * 32 + g * 8);
            }
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg)
                o.m[qg] = rec[(int64_t)it.k * kTileRows + wib * C::kWaveRows + qg * 16 + n16];
        };
        auto compute = [&](const Item& it, const KOps& o) __attribute__((always_inline)) {
            // V^T rows d of the sub-block, keys 4g .. 4g+3; their latency hides
            // under the products below
            v4bf vop[C::kDB];
            const uint16_t* vsub = vsh + ((size_t)(it.t * kSubBlocks + it.c) * D) * kSubKeys + g * 4;
#pragma unroll
            for (int db = 0; db < C::kDB; ++db)
                vop[db] = *reinterpret_cast<const v4bf*>(vsub + (db * 16 + n16) * kSubKeys);
            // 8-bit accumulators of the sub-block, as in the loop, and bf16 ones
            v4f s8[kQG], s16[kQG];
#pragma unroll
            for (int st = 0; st < C::kKS; ++st)
#pragma unroll
                for (int qg = 0; qg < kQG; ++qg)
                    s8[qg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        o.k8[st], q8_operand(qg, st), st == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : s8[qg],
                        0, 0, 0, 0, 0, 0);
            const uint16_t* krow = k16h + (size_t)min(it.t * kTileKeys + it.c * 16 + n16, smax_row) * D;
#pragma unroll
            for (int ch = 0; ch < C::kDC; ++ch) {
                v8bf kop;
                if constexpr (kPreK16) kop = o.k16[ch];
                else kop = *reinterpret_cast<const v8bf*>(krow + ch * 32 + g * 8);
#pragma unroll
                for (int qg = 0; qg < kQG; ++qg)
                    s16[qg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        kop, q16_operand(ch, qg), ch == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : s16[qg], 0, 0, 0);
            }
            const bool full = tile_full(r, it.t, a.S, a.causal, a.window);
            // weights of keys c*16 + 4g + i for query 16qg + n16, and the
            // scaled differences split into two bf16 terms
            u32x2 hi[kQG], lo[kQG];
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg) {
                const int qi = row0 + qg * 16 + n16;
                const float scale = m_run[qg] == -__builtin_inff() ? 0.0f : fast_exp2(o.m[qg] - m_run[qg]);
                float e8[4], e16[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e8[i] = fast_exp2(__builtin_fmaf(s8[qg][i], c8, -o.m[qg]));
                    e16[i] = fast_exp2(__builtin_fmaf(s16[qg][i], c16, -o.m[qg]));
                    if (!full && !pair_visible(qi, it.t * kTileKeys + it.c * 16 + g * 4 + i, a.S, a.causal, a.window)) {
                        e8[i] = 0.0f;
                        e16[i] = 0.0f;
                    }
                }
                const uint32_t w8 = cvt_pk_e4m3_unit<true>(e8[2], e8[3], cvt_pk_e4m3_unit<false>(e8[0], e8[1], 0u));
                const uint32_t p8b[2] = {e4m3x2_to_bf16x2<false>(w8), e4m3x2_to_bf16x2<true>(w8)};
                const uint32_t p16b[2] = {f32x2_to_bf16x2(e16[0], e16[1]), f32x2_to_bf16x2(e16[2], e16[3])};
                float x[4], h[4], l[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t b8 = (i & 1) ? (p8b[i / 2] >> 16) : (p8b[i / 2] & 0xFFFFu);
                    const uint32_t b16 = (i & 1) ? (p16b[i / 2] >> 16) : (p16b[i / 2] & 0xFFFFu);
                    // exact difference of two bf16-representable weights, then scaled
                    x[i] = scale * (bf16_bits_to_float(b16) - bf16_bits_to_float(b8));
                }
                hi[qg] = u32x2{f32x2_to_bf16x2(x[0], x[1]), f32x2_to_bf16x2(x[2], x[3])};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    h[i] = bf16_bits_to_float((i & 1) ? (hi[qg][i / 2] >> 16) : (hi[qg][i / 2] & 0xFFFFu));
                    l[i] = x[i] - h[i];
                }
                lo[qg] = u32x2{f32x2_to_bf16x2(l[0], l[1]), f32x2_to_bf16x2(l[2], l[3])};
                if constexpr (kDump) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int kj = it.t * kTileKeys + it.c * 16 + g * 4 + i;
                        if (qi < a.S && kj < a.S)
                            a.dump_p[(q_head * a.S + qi) * a.S + kj] =
                                (uint16_t)((i & 1) ? (p16b[i / 2] >> 16) : (p16b[i / 2] & 0xFFFFu));
                    }
                }
            }
            // O += V^T (hi + lo), l += 1^T (hi + lo)
#pragma unroll
            for (int db = 0; db < C::kDB; ++db)
#pragma unroll
                for (int qg = 0; qg < kQG; ++qg) {
                    acc_o[qg][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                        vop[db], __builtin_bit_cast(v4bf, hi[qg]), acc_o[qg][db], 0, 0, 0);
                    acc_o[qg][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                        vop[db], __builtin_bit_cast(v4bf, lo[qg]), acc_o[qg][db], 0, 0, 0);
                }
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg) {
                acc_l[qg] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones4, __builtin_bit_cast(v4bf, hi[qg]), acc_l[qg], 0, 0, 0);
                acc_l[qg] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones4, __builtin_bit_cast(v4bf, lo[qg]), acc_l[qg], 0, 0, 0);
            }
        };

        Item it;
        KOps nxt;
        bool valid = next_item(it);
        if (valid) load_k(it, nxt);
        while (valid) {
            const KOps cur = nxt;
            Item nx;
            const bool vn = next_item(nx);
            if (vn) load_k(nx, nxt);
            compute(it, cur);
            it = nx;
            valid = vn;
        }
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
size_t lds_bytes_d(int nT) {
    using C = Cfg<D>;
    return C::kListOff + (((size_t)C::kBlocks * nT * 2 + 15) / 16) * 16;
}

template <int D>
hipError_t launch_d(const Shape& sh, const AttnParams& p, hipStream_t st) {
    using C = Cfg<D>;
    AttnArgs a;
    a.q8 = p.q8; a.k8 = p.k8; a.q16 = p.q16; a.k16 = p.k16; a.vt = p.vt; a.vsb = p.vsb;
    a.q_scale = p.q_scale; a.k_scale = p.k_scale; a.out = p.out; a.mask = p.mask;
    a.rec_m = p.rec_m;
    a.dump_s = p.dump_s; a.dump_p = p.dump_p;
    a.l_d = p.log2e_over_sqrt_d; a.t2 = p.t2;
    a.x_delta = p.e_delta > 0.0f ? (float)std::log2((double)p.e_delta) : -__builtin_inff();
    a.test_mode = !(p.t2 < __builtin_inff()) || !(p.e_delta < __builtin_inff()) ? 0 : (p.e_delta > 0.0f ? 1 : 2);
    a.B = sh.B; a.Hq = sh.Hq; a.Hkv = sh.Hkv; a.S = sh.S; a.nT = sh.nT; a.S_pad = sh.S_pad;
    a.causal = p.causal; a.window = p.window;
    a.G = sh.Hq / sh.Hkv;
    a.heads_per_wg = 1;
    for (int h = C::kBlocks; h >= 1; h /= 2)
        if (a.G % h == 0) { a.heads_per_wg = h; break; }
    a.rows_per_wg = C::kBlocks / a.heads_per_wg;
    a.n_rg = (sh.nT + a.rows_per_wg - 1) / a.rows_per_wg;
    a.n_wg = sh.B * sh.Hkv * (a.G / a.heads_per_wg) * a.n_rg;
    a.xcd_remap = (a.n_wg % 8 == 0) ? 1 : 0;
    a.rec_per_head = rec_slot_base(sh.nT, sh.nT, p.causal, p.window);
    const size_t lds = lds_bytes_d<D>(sh.nT);
    const bool dump = p.dump_s != nullptr && p.dump_p != nullptr;
    using Fn = void (*)(AttnArgs);
    static const Fn table[2][3] = {
        {lamp_attn_kernel<D, false, 0>, lamp_attn_kernel<D, false, 1>, lamp_attn_kernel<D, false, 2>},
        {lamp_attn_kernel<D, true, 0>, lamp_attn_kernel<D, true, 1>, lamp_attn_kernel<D, true, 2>}};
    const Fn fn = table[dump ? 1 : 0][a.test_mode];
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(a.n_wg), dim3(kThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_deferred(const Shape& sh, const AttnParams& p, hipStream_t st) {
    if (sh.D == 256) return launch_d<256>(sh, p, st);
    return hipErrorInvalidValue;
}

}  // namespace lamp
