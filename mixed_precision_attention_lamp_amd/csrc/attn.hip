// Fused LampAttention forward kernel for gfx950 (MI355X), head dimensions 64,
// 128 and 256.
//
// Method: "LampAttention: Look-Ahead Mixed-Precision FlashAttention for
// Dedicated Accelerators" (abstract).  Per 64x64 tile of (query rows, keys):
//   1. 8-bit logits: e4m3 Q.K^T on the FP8 matrix cores, fp32 accumulation;
//   2. running row max over the 8-bit logits (log2 domain);
//   3. 8-bit exponentials: exp2 rounded to e4m3 (the hardware exp2, or in
//      the bit-reproducible variant a polynomial exp2 defined by its fp32
//      steps, poly_exp2);
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
// Schedule (D = 64, 128): two waves per SIMD run the same sequence of vector
// phases (max, exponentials, rescale, test) and matrix phases (recompute, P.V,
// the next tile's Q.K^T) one phase apart, so that each SIMD's matrix cores
// work under the other wave's vector work; the K8, K16 and V^T tiles are
// copied from global memory straight into LDS (buffer loads with an LDS
// destination, no registers) two tiles ahead, into three slots per array.
// D = 256 (no room for the ping-pong's slots): every wave runs one
// software-pipelined loop over two slots per array; the P.V products of tile
// t-1 run ahead of the vector work of tile t, with the copies of later tiles
// issued between them, and the Q.K^T products of tile t+1 under the rescale,
// the LDS stores and the barrier.  LDS layouts are unpadded, their 16-byte
// chunks XOR-swizzled by row (conflict-free operand reads).  Each wave
// quantises its Q rows in the prologue (the arithmetic of the quantisation
// pass) straight into its Q8 operand registers, and keeps its Q16 operand in
// registers too.
//
// Work decomposition: a workgroup of eight waves shares staged K/V tiles.  A
// wave owns 32 query rows (16 for D = 256), so that the fp32 output
// accumulator stays in architectural registers, where the per-row rescale is
// one multiply; the 2 (4) waves of one 64-row query block of one query head
// OR their 4-bit sub-block flags through LDS.  The 4 (2) blocks of a workgroup
// are query heads of one GQA group (or fewer heads and consecutive row blocks
// when the group is smaller), so one staged K/V tile serves all of them.
// Logits are held transposed (keys in rows, queries in columns): lane l keeps
// query l % 16 of each 16-query group, which makes the row max a register
// reduction plus two cross-lane steps and lets the exponentials feed the P.V
// operand in place.
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
    const uint8_t* k8;
    const uint16_t* q16;
    const uint16_t* k16;
    const uint16_t* vt;
    const float* q_scale;
    const float* q_inv;
    const float* k_scale;
    float* out;
    uint8_t* mask;
    float* dump_s;       // debug: [B, Hq, S, S] 8-bit accumulators (or null)
    uint16_t* dump_p;    // debug: [B, Hq, S, S] final bf16 weights (or null)
    double l_d;          // log2(e) / sqrt(D), fp64
    float x_delta;       // first stage: exp2 argument threshold (log2 of the e4m3 boundary)
    float t2;
    int test_mode;       // 0: no test (second stage off), 1: both stages, 2: second stage only
    int B, Hq, Hkv, S, nT, S_pad;
    int causal, window;
    int G;               // Hq / Hkv
    int heads_per_wg;    // kBlocks, ..., 1
    int rows_per_wg;     // kBlocks / heads_per_wg
    int n_rg;            // row-block groups
    int paired;          // 1: a workgroup runs row-block groups n_rg-1-level and level
    int n_wg;
    int rot_shift;       // unpaired: level l shifts the unit order by l >> rot_shift
};

template <int D, bool kPlain = false>
struct Cfg {
    // a wave owns 32 query rows (16 for D = 256, whose output accumulator is
    // twice as wide); 2 (or 4) waves form one 64-row block
    static constexpr int kQG = D == 256 ? 1 : 2;        // 16-query groups per wave
    static constexpr int kWaveRows = 16 * kQG;
    static constexpr int kWavesPerBlock = kTileRows / kWaveRows;
    static constexpr int kBlocks = kWaves / kWavesPerBlock;   // 64-row blocks per workgroup
    static constexpr int kKS = D >= 128 ? D / 128 : 1;       // 128-deep FP8 matrix-core steps
    static constexpr int kK8Row = D;                   // bytes per staged row
    static constexpr int kK16Row = 2 * D;
    static constexpr int kVtRow = 2 * kTileKeys;
    static constexpr int kK8Bytes = kTileKeys * kK8Row;
    static constexpr int kK16Bytes = kTileKeys * kK16Row;
    static constexpr int kVtBytes = D * kVtRow;
    // Every staged array is filled by direct global-to-LDS copies: three
    // slots each under the ping-pong schedule (D <= 128), two each otherwise
    // (D = 256: 160 KB, all of a CU's LDS)
    static constexpr bool kPP = D <= 128;
    static constexpr int kSlots16 = kPP ? 3 : 2;
    static constexpr int kSlotsQK = kPP ? 3 : 2;
    // The tiles Q.K^T reads: K8, or K16 in the plain bf16 mode (which then
    // needs no separate K16 slots).
    static constexpr int kQKRow = kPlain ? kK16Row : kK8Row;
    static constexpr int kQKBytes = kTileKeys * kQKRow;
    static constexpr int kK8Off = 0;
    static constexpr int kK16Off = kSlotsQK * kQKBytes;
    static constexpr int kVtOff = kK16Off + (kPlain ? 0 : kSlots16 * kK16Bytes);
    static constexpr int kLdsBytes = kVtOff + kSlots16 * kVtBytes;
    static constexpr int kDB = D / 16;        // 16-wide output column blocks
    static constexpr int kDC = D / 32;        // 32-deep bf16 matrix-core steps
};

// kMode: 0 = no test (second stage off), 1 = both stages, 2 = second stage
// only, 3 = plain bf16 FlashAttention (the 16-bit baseline: no 8-bit pass,
// Q.K^T of every sub-block on the bf16 matrix cores, exponentials rounded to
// bf16; at D = 256 its K16 tiles take the K8 slots); 4 + (0, 1, 2): the test modes 0-2 with
// 8-bit logits (the log2-domain logit c8 acc itself rounded to e4m3 before the
// running max, the exponentials and the test read it); 9: mode 1 with the
// per-entry test in vector form (for small tau, where most waves need it);
// 16 + (0, 1, 2): the test modes 0-2 with the 8-bit exponentials taken by
// the bit-reproducible polynomial exp2 (poly_exp2) instead of v_exp_f32.
template <int D, bool kDump, int kMode>
__global__ __launch_bounds__(kThreads, 1) void lamp_attn_kernel(AttnArgs a) {
    constexpr bool kPlain = kMode == 3;
    constexpr bool kLogit8 = (kMode & 4) != 0;
    constexpr bool kDense = (kMode & 8) != 0;
    constexpr bool kPoly = (kMode & 16) != 0;
    constexpr int kTest = kMode & 3;
    using C = Cfg<D, kPlain>;
    constexpr int kQG = C::kQG;
    constexpr int kWaveRows = C::kWaveRows;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int n16 = lane & 15;     // query column within a 16-query group
    const int g = lane >> 4;       // lane group: which 4 keys / which k-slice
    const int blk = wave / C::kWavesPerBlock;   // which (head, 64-row block) of the workgroup
    const int wib = wave % C::kWavesPerBlock;   // rows wib*kWaveRows .. of that block

    // ---- workgroup -> (batch, kv head, head group) unit and row-block group(s)
    // Workgroups are dispatched in index order, round-robin over the XCDs
    // (index i to XCD i mod 8), so each XCD receives a fixed eighth of them
    // whatever their cost.  Index order is longest (causal) rows first;
    // consecutive indices are consecutive units, so with 8 units per level
    // each XCD would keep to one unit and its K/V tiles would stay in that
    // XCD's L2 -- but units differ in how much they recompute (their keys
    // differ), and an XCD holding a heavy unit would finish last.  Unpaired
    // launches therefore shift the unit order by one every 2^rot_shift levels:
    // each XCD cycles through the units, a run of 2^rot_shift consecutive
    // row blocks of one unit at a time (those share most K/V tiles, in L2).
    const int wg = blockIdx.x;
    const int n_hg = a.G / a.heads_per_wg;
    const int n_lv = a.paired ? (a.n_rg + 1) / 2 : a.n_rg;
    const int n_u = a.n_wg / n_lv;
    const int level = wg / n_u;
    int u = (wg % n_u + (a.paired ? 0 : level >> a.rot_shift)) % n_u;
    const int hg = u % n_hg;
    u /= n_hg;
    const int hk = u % a.Hkv;
    const int b = u / a.Hkv;
    const int hq = hk * a.G + hg * a.heads_per_wg + (blk % a.heads_per_wg);
    const size_t kv_head = (size_t)b * a.Hkv + hk;
    const size_t q_head = (size_t)b * a.Hq + hq;

    // Paired launches: a workgroup runs two row-block groups back to back,
    // n_rg-1-level and level.  Under a causal mask they visit n_rg+1 tiles
    // together at every level, so all workgroups carry the same work and no
    // CU waits on a long last workgroup (it pays where there are only about
    // two workgroups per CU).  Otherwise a workgroup runs n_rg-1-level alone,
    // longest rows first.  Between the two runs every wave has passed the
    // last barrier of the first one's loop, after which no wave reads the LDS
    // staged for it (the one-slot loop's final P.V reads only V^T, which the
    // second one first writes after its prologue barrier).
    auto run_rows = [&](const int rg) __attribute__((always_inline)) {
    const int r = rg * a.rows_per_wg + blk / a.heads_per_wg;
    const bool active = r < a.nT;
    const int r_first = rg * a.rows_per_wg;
    const int r_last = min(r_first + a.rows_per_wg - 1, a.nT - 1);
    const int t_begin = tile_lo(r_first, a.window);
    const int t_end = tile_hi(r_last, a.nT, a.causal);
    const int row0 = r * kTileRows + wib * kWaveRows;   // first query row of this wave
    // The tiles this wave's row block visits, [tv_lo, tv_hi], and those all of
    // whose entries are visible, [tf_lo, tf_hi] (empty when lo > hi), as
    // wave-uniform bounds: the loop's per-tile decisions are scalar compares.
    const int r_u = __builtin_amdgcn_readfirstlane(r);
    const bool active_u = r_u < a.nT;
    const int tv_lo = active_u ? tile_lo(r_u, a.window) : 1;
    const int tv_hi = active_u ? tile_hi(r_u, a.nT, a.causal) : 0;
    int tf_lo = 1, tf_hi = 0;
    if (active_u && r_u * kTileRows + kTileRows <= a.S) {
        tf_hi = a.S / kTileKeys - 1;
        if (a.causal) tf_hi = min(tf_hi, r_u - 1);
        const int num = r_u * kTileRows + kTileRows - a.window;
        tf_lo = a.window > 0 && num > 0 ? (num + kTileKeys - 1) / kTileKeys : 0;
    }


    // ---- staging: K8, K16 and V^T tiles are copied from global memory straight
    // into swizzled LDS layouts.  Thread tid owns the 16-byte chunks
    // c = tid + kThreads*i of a tile, i.e. LDS bytes [16 c, 16 c + 16), and
    // copies the global chunk that belongs there.
    constexpr int kK8Ch = C::kQKBytes / 16 / kThreads;     // chunks per thread and tile
    constexpr int kK16Ch = C::kK16Bytes / 16 / kThreads;
    constexpr int kVtCh = C::kVtBytes / 16 / kThreads;
    static_assert(kK16Ch >= 1 && kVtCh >= 1, "tile smaller than one chunk per thread");
    constexpr int kK8ChMin = kK8Ch > 0 ? kK8Ch : 1;
    const uint8_t* k16_head = reinterpret_cast<const uint8_t*>(a.k16 + kv_head * a.S * D);
    // Copy i of wave w moves chunks i*kThreads + 64w .. +63 of a tile, lane l
    // the chunk i*kThreads + 64w + l.  Each array of the (batch, kv head) is one buffer: a lane's byte offset
    // (row and swizzled chunk) is fixed, the tile's is a scalar, and reads past
    // the buffer's end (keys past the last) return zeros.  A copy's LDS
    // destination is one wave-uniform address; lane l's 16 bytes land 16 l
    // bytes above it.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    constexpr int kBufWord3 = 0x00020000;    // raw 32-bit-format buffer
    const __amdgpu_buffer_rsrc_t rs_qk = __builtin_amdgcn_make_buffer_rsrc(
        kPlain ? (void*)k16_head : (void*)(a.k8 + kv_head * a.S_pad * D), (short)0,
        kPlain ? a.S * C::kK16Row : a.S_pad * D, kBufWord3);
    const __amdgpu_buffer_rsrc_t rs_k16 =
        __builtin_amdgcn_make_buffer_rsrc((void*)k16_head, (short)0, a.S * C::kK16Row, kBufWord3);
    const __amdgpu_buffer_rsrc_t rs_vt = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.vt + kv_head * a.nT * (size_t)D * kTileKeys), (short)0, a.nT * C::kVtBytes, kBufWord3);
    auto chunk_off = [&](int i, auto row_bytes) __attribute__((always_inline)) -> unsigned {
        constexpr int kRow = decltype(row_bytes)::value;
        const unsigned p = (tid + i * kThreads) * 16;
        const unsigned row = p / kRow, slot16 = (p % kRow) >> 4;
        return row * kRow + ((slot16 ^ swz<kRow / 16>(row)) << 4);
    };
    auto dma = [&](__amdgpu_buffer_rsrc_t rs, unsigned voff, int soff, uint8_t* dst) __attribute__((always_inline)) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
    };
    auto dma_qk_i = [&](int t, int slot, int i) __attribute__((always_inline)) {
        const int first = i * kThreads + wave_u * 64;
        if (first * 16 >= C::kQKBytes) return;    // D = 64: half the waves
        dma(rs_qk, chunk_off(i, std::integral_constant<int, C::kQKRow>{}), t * C::kQKBytes,
            lds + C::kK8Off + slot * C::kQKBytes + first * 16);
    };
    auto dma_k16_i = [&](int t, int slot, int i) __attribute__((always_inline)) {
        dma(rs_k16, chunk_off(i, std::integral_constant<int, C::kK16Row>{}), t * C::kK16Bytes,
            lds + C::kK16Off + slot * C::kK16Bytes + (i * kThreads + wave_u * 64) * 16);
    };
    auto dma_vt_i = [&](int t, int slot, int i) __attribute__((always_inline)) {
        dma(rs_vt, chunk_off(i, std::integral_constant<int, C::kVtRow>{}), t * C::kVtBytes,
            lds + C::kVtOff + slot * C::kVtBytes + (i * kThreads + wave_u * 64) * 16);
    };
    auto dma_qk = [&](int t, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kK8ChMin; ++i) dma_qk_i(t, slot, i);
    };
    auto dma_k16 = [&](int t, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kK16Ch; ++i) dma_k16_i(t, slot, i);
    };
    auto dma_vt = [&](int t, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kVtCh; ++i) dma_vt_i(t, slot, i);
    };
    // The copies one matrix phase issues, one per call: K16 and V^T of tile
    // t16 into slot s16, then K8 of tile t8 into slot s8.  Tiles past the end
    // copy the last one again: its destination slot is not read any more, and
    // the copies of a phase stay a fixed, branch-free sequence.
    constexpr int kDmaK16 = kPlain ? 0 : kK16Ch;
    constexpr int kDmaSteps = kDmaK16 + kVtCh + kK8ChMin;
    auto dma_step = [&](int k, int t16, int s16, int t8, int s8) __attribute__((always_inline)) {
        if (k < kDmaK16) {
            if constexpr (!kPlain) dma_k16_i(min(t16, t_end), s16, k);
        } else if (k < kDmaK16 + kVtCh) {
            dma_vt_i(min(t16, t_end), s16, k - kDmaK16);
        } else if (k < kDmaSteps) {
            dma_qk_i(min(t8, t_end), s8, k - kDmaK16 - kVtCh);
        }
    };

    // ---- prologue: this wave's Q16 and Q8 operands into registers ----------------------
    if constexpr (!C::kPP) {
        // one-loop schedule (D = 256): the first tile's copies go out before
        // the Q loads, so that their latencies overlap (measured slower in the
        // ping-pong schedule, whose prologue copies five tiles)
        dma_qk(t_begin, t_begin & 1);
        if constexpr (!kPlain) dma_k16(t_begin, t_begin & 1);
    }
    float m_run[kQG], c8 = 0.0f, inv_c8 = 0.0f, a2 = 0.0f, c8_log = 0.0f;
    const float c16 = (float)a.l_d;
    v8bf qb[C::kDC][kQG];     // bf16 operand of 16-query group qg, 32-deep step ch
#pragma unroll
    for (int qg = 0; qg < kQG; ++qg) {
        // rows past the end are never written out
        const uint16_t* qrow = a.q16 + (q_head * a.S + min(row0 + qg * 16 + n16, a.S - 1)) * D;
#pragma unroll
        for (int ch = 0; ch < C::kDC; ++ch) qb[ch][qg] = *reinterpret_cast<const v8bf*>(qrow + ch * 32 + g * 8);
    }
    // Q8 = E4M3(fl32(q * inv)) of this wave's rows (the arithmetic of the
    // quantisation pass), straight into the 8-bit operand registers: lane
    // (n16, g) holds depth 32g .. 32g+31 of 128-deep step st of row 16qg + n16
    // (D = 64: lane groups 2, 3 hold zeros); rows past the end are zero.
    v8i q8r[C::kKS][kQG];
    if constexpr (!kPlain) {
        const float inv = active ? a.q_inv[q_head] : 1.0f;
#pragma unroll
        for (int st = 0; st < C::kKS; ++st)
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg) {
                v8i x8 = {0, 0, 0, 0, 0, 0, 0, 0};
                const int gq = row0 + qg * 16 + n16;
                if (gq < a.S && (D >= 128 || g * 32 < D)) {
                    const uint16_t* src = a.q16 + (q_head * a.S + gq) * D + (D >= 128 ? st * 128 + 32 * g : 32 * g);
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const u32x4 w = *reinterpret_cast<const u32x4*>(src + 8 * h);
                        float x[8];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            x[2 * j] = bf16_bits_to_float(w[j] & 0xFFFFu) * inv;
                            x[2 * j + 1] = bf16_bits_to_float(w[j] >> 16) * inv;
                        }
                        x8[2 * h] = (int)cvt_pk_e4m3<true>(x[2], x[3], cvt_pk_e4m3<false>(x[0], x[1], 0u));
                        x8[2 * h + 1] = (int)cvt_pk_e4m3<true>(x[6], x[7], cvt_pk_e4m3<false>(x[4], x[5], 0u));
                    }
                }
                q8r[st][qg] = x8;
            }
    }
#pragma unroll
    for (int qg = 0; qg < kQG; ++qg) m_run[qg] = -__builtin_inff();
    if (active) {
        if constexpr (!kPlain) {
            c8 = (float)((double)a.q_scale[q_head] * (double)a.k_scale[kv_head] * a.l_d);
            // with 8-bit logits everything after the rounding reads logits
            // directly: the accumulator factor becomes 1
            if constexpr (kLogit8) {
                c8_log = c8;
                c8 = 1.0f;
            }
            a2 = acc_threshold(a.t2, c8);
            inv_c8 = 1.0f / c8;
        }
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

    auto work = [&](int t) __attribute__((always_inline)) { return t >= tv_lo && t <= tv_hi; };
    auto full_tile = [&](int t) __attribute__((always_inline)) { return t >= tf_lo && t <= tf_hi; };

    // ---- matrix-core phases ---------------------------------------------------------
    // Q.K^T of tile t: s[qg][kb][i] = 8-bit accumulator of key 16kb + 4g + i, query 16qg + n16
    auto qk = [&](v4f (&s)[kQG][4], int slot) __attribute__((always_inline)) {
        if constexpr (kPlain) {
            // bf16 logits of all four sub-blocks (the recompute's products)
            const uint8_t* kl = lds + C::kK8Off + slot * C::kQKBytes;
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int ch = 0; ch < C::kDC; ++ch) {
                    const v8bf ka = *reinterpret_cast<const v8bf*>(kl + lds_off<C::kK16Row>(c * 16 + n16, ch * 4 + g));
#pragma unroll
                    for (int qg = 0; qg < kQG; ++qg)
                        s[qg][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            ka, qb[ch][qg], ch == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : s[qg][c], 0, 0, 0);
                }
            return;
        }
        const uint8_t* k8l = lds + C::kK8Off + slot * C::kQKBytes;
#pragma unroll
        for (int st = 0; st < C::kKS; ++st) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const v8i ka = fp8_operand<D>(k8l, kb * 16 + n16, st, g);
#pragma unroll
                for (int qg = 0; qg < kQG; ++qg)
                    s[qg][kb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        ka, q8r[st][qg], st == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : s[qg][kb], 0, 0, 0, 0, 0, 0);
            }
        }
    };
    // P.V of tile t (and the row sums, with an all-ones operand)
    const v8bf ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                       (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
    // Ping-pong schedule: software-pipelined V^T operand reads.  The first
    // half's operands are read up front, and each read of the second half
    // reuses the registers of the first-half operand whose products were just
    // issued; the schedule is pinned (the scheduler would sink every read next
    // to its use).  The phase's copies into LDS (copy(k), k = 0, 1, ...) are
    // issued one after every second output block, between matrix products,
    // so that the memory unit takes them one at a time.
    auto pv = [&](const u32x2 (&P)[kQG][4], int slot, auto copy) __attribute__((always_inline)) {
        const uint8_t* vtl = lds + C::kVtOff + slot * C::kVtBytes;
        if constexpr (C::kPP) {
            v8bf va[C::kDB];
#pragma unroll
            for (int db = 0; db < C::kDB; ++db)
                va[db] = *reinterpret_cast<const v8bf*>(vtl + lds_off<C::kVtRow>(db * 16 + n16, g));
            __builtin_amdgcn_sched_group_barrier(0x100, C::kDB, 0);
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
#pragma unroll
                    for (int qg = 0; qg < kQG; ++qg)
                        acc_o[qg][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], pb[qg], acc_o[qg][db], 0, 0, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, kQG, 0);
                    if (h == 0) {
                        va[db] = *reinterpret_cast<const v8bf*>(vtl + lds_off<C::kVtRow>(db * 16 + n16, 4 + g));
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                    if ((db & 1) && h * (C::kDB / 2) + db / 2 < kDmaSteps) {
                        copy(h * (C::kDB / 2) + db / 2);
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                    }
                }
#pragma unroll
                for (int qg = 0; qg < kQG; ++qg)
                    acc_l[qg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[qg], acc_l[qg], 0, 0, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, kQG, 0);
            }
            return;
        }
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
                // one copy after every fourth output block
                if ((db & 3) == 3) copy((h * C::kDB + db) >> 2);
            }
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg)
                acc_l[qg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[qg], acc_l[qg], 0, 0, 0);
        }
    };

    // (2') 8-bit logits: s = e4m3(c8 acc), magnitudes clamped to 448 first
    // (e4m3fn saturates there), nearest even, back in fp32 exactly
    auto round_logits = [&](v4f (&s)[kQG][4]) __attribute__((always_inline)) {
        if constexpr (kLogit8) {
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    float y[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[i] = s[qg][kb][i] * c8_log;
                    const uint32_t w = cvt_pk_e4m3<true>(y[2], y[3], cvt_pk_e4m3<false>(y[0], y[1], __float_as_uint(y[0])));
                    const v2f lo = e4m3x2_to_f32x2<false>(w), hi = e4m3x2_to_f32x2<true>(w);
                    s[qg][kb] = v4f{lo[0], lo[1], hi[0], hi[1]};
                }
        }
    };

    // ---- per-tile vector state ---------------------------------------------------------
    float alpha[kQG], m_use[kQG];
    float smax[kQG][4];                 // per (lane, sub-block) maxima of the 8-bit accumulators
    float smin[kTest == 2 ? kQG : 1][4];    // and minima, when the first stage is off
    uint32_t vis[kQG];                  // masked tiles: bit kb*4+i = entry visible

    // (2): visibility, sub-block maxima (and minima) and the running max of
    // tile t, straight-line code.
    auto stats = [&](const v4f (&s)[kQG][4], int t, auto masked_tag) __attribute__((always_inline)) {
        constexpr bool kMasked = decltype(masked_tag)::value;
        constexpr float kNegInf = -__builtin_inff();
        if constexpr (kMasked) {
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg) {
                vis[qg] = 0u;
                const int qi = row0 + qg * 16 + n16;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    vis[qg] |= visible4(qi, t * kTileKeys + kb * 16 + g * 4, a.S, a.causal, a.window) << (kb * 4);
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
                if constexpr (kTest == 2)
                    smin[qg][kb] = __builtin_fminf(__builtin_fminf(w[0], w[1]), __builtin_fminf(w[2], w[3]));
            }
            float mx = __builtin_fmaxf(__builtin_fmaxf(smax[qg][0], smax[qg][1]),
                                       __builtin_fmaxf(smax[qg][2], smax[qg][3]));
            mx = max_over_lane_groups(mx);
            const float mt = mx == kNegInf ? mx : mx * (kPlain ? c16 : c8);
            const float mn = __builtin_fmaxf(m_run[qg], mt);
            alpha[qg] = mn == m_run[qg] ? 1.0f : fast_exp2(m_run[qg] - mn);
            m_use[qg] = mn == kNegInf ? 0.0f : mn;
            m_run[qg] = mn;
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
    };
    // (3): 8-bit exponentials of tile t against the running max.
    auto exps8 = [&](const v4f (&s)[kQG][4], u32x2 (&P)[kQG][4], auto masked_tag) __attribute__((always_inline)) {
        constexpr bool kMasked = decltype(masked_tag)::value;
#pragma unroll
        for (int qg = 0; qg < kQG; ++qg)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                float e[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = __builtin_fmaf(s[qg][kb][i], kPlain ? c16 : c8, -m_use[qg]);
                    e[i] = kPoly ? poly_exp2(x) : fast_exp2(x);
                    if constexpr (kMasked) e[i] = ((vis[qg] >> (kb * 4 + i)) & 1u) ? e[i] : 0.0f;
                }
                if constexpr (kPlain) {
                    P[qg][kb] = u32x2{f32x2_to_bf16x2(e[0], e[1]), f32x2_to_bf16x2(e[2], e[3])};
                } else {
                    // the high half of the first conversion's destination is
                    // overwritten by the second: any dead register serves as
                    // its initial value (a zero would cost a move per conversion)
                    const uint32_t w = cvt_pk_e4m3_unit<true>(
                        e[2], e[3], cvt_pk_e4m3_unit<false>(e[0], e[1], __float_as_uint(e[0])));
                    P[qg][kb] = u32x2{e4m3x2_to_bf16x2<false>(w), e4m3x2_to_bf16x2<true>(w)};
                }
            }
    };
    auto softmax = [&](const v4f (&s)[kQG][4], u32x2 (&P)[kQG][4], int t, auto masked_tag) __attribute__((always_inline)) {
        stats(s, t, masked_tag);
        exps8(s, P, masked_tag);
    };

    // (4): the look-ahead test on the accumulators of tile t; returns the wave's
    // 4-bit flag set (wave-uniform).  First stage: the 8-bit exponential is at
    // least delta, i.e. its argument x = acc c8 - m is at least x_delta, i.e.
    // acc >= a1 = (x_delta + m) / c8.  Second stage: |acc| >= a2.  When
    // a1 > -a2 both hold iff acc >= max(a1, a2), so a sub-block holds a
    // sensitive entry of this row iff its maximum does: one compare per (lane,
    // sub-block).  Rows with a1 <= -a2 (a very negative running max) fall back
    // to a per-entry test for the wave.
    auto test = [&](const v4f (&s)[kQG][4], auto masked_tag) __attribute__((always_inline)) -> uint32_t {
        constexpr bool kMasked = decltype(masked_tag)::value;
        uint64_t hit[4] = {0, 0, 0, 0};
        if constexpr (kTest == 1) {
            bool slow = false;
            float thr[kQG];
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg) {
                const float a1 = (a.x_delta + m_use[qg]) * inv_c8;
                thr[qg] = __builtin_fmaxf(a1, a2);
                slow |= a1 <= -a2;
            }
            if (wave_ballot(slow) == 0) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    uint64_t h = 0;
#pragma unroll
                    for (int qg = 0; qg < kQG; ++qg) h |= wave_ballot(smax[qg][kb] >= thr[qg]);
                    hit[kb] = h;
                }
            } else {
                if constexpr (kDense) {
                    // an entry is sensitive iff max(x_delta - x, a2 - |acc|) <= 0
                    // (each difference is exact in sign); the lane's minimum
                    // over a sub-block decides with one ballot
#pragma unroll
                    for (int qg = 0; qg < kQG; ++qg)
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) {
                            float dmin = __builtin_inff();
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float v = s[qg][kb][i];
                                float d = __builtin_fmaxf(a.x_delta - __builtin_fmaf(v, c8, -m_use[qg]),
                                                          a2 - __builtin_fabsf(v));
                                if constexpr (kMasked) d = ((vis[qg] >> (kb * 4 + i)) & 1u) ? d : __builtin_inff();
                                dmin = __builtin_fminf(dmin, d);
                            }
                            hit[kb] = (qg == 0 ? 0 : hit[kb]) | wave_ballot(dmin <= 0.0f);
                        }
                } else {
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) hit[kb] = 0;
#pragma unroll
                    for (int qg = 0; qg < kQG; ++qg)
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                // each ballot of a compare is that compare's lane
                                // mask; the masks combine in scalar registers
                                const float v = s[qg][kb][i];
                                uint64_t h = wave_ballot(__builtin_fmaf(v, c8, -m_use[qg]) >= a.x_delta) &
                                             wave_ballot(__builtin_fabsf(v) >= a2);
                                if constexpr (kMasked) h &= wave_ballot((vis[qg] >> (kb * 4 + i)) & 1u);
                                hit[kb] |= h;
                            }
                }
            }
        } else if constexpr (kTest == 2) {
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

    // (5): 16-bit recompute of tile t.  The flag set is wave-uniform (scalar):
    // the wave walks its set bits behind scalar branches, running the bf16
    // logits of each flagged sub-block on the matrix cores and rounding its
    // exponentials to bf16 into the compile-time-indexed register tile P.
    // The bf16 logits of flagged sub-block c (the matrix-core half of (5))
    auto recompute_mfma = [&](v4f (&acc16)[kQG], int c, int slot) __attribute__((always_inline)) {
        const uint8_t* k16l = lds + C::kK16Off + slot * C::kK16Bytes;
#pragma unroll
        for (int ch = 0; ch < C::kDC; ++ch) {
            const v8bf ka = *reinterpret_cast<const v8bf*>(k16l + lds_off<C::kK16Row>(c * 16 + n16, ch * 4 + g));
#pragma unroll
            for (int qg = 0; qg < kQG; ++qg)
                acc16[qg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    ka, qb[ch][qg], ch == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : acc16[qg], 0, 0, 0);
        }
    };
    // ... and their exponentials rounded to bf16, spliced into P
    auto recompute_exp = [&](u32x2 (&P)[kQG][4], const v4f (&acc16)[kQG], int c, auto masked_tag) __attribute__((always_inline)) {
        constexpr bool kMasked = decltype(masked_tag)::value;
#pragma unroll
        for (int qg = 0; qg < kQG; ++qg) {
            float e[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                e[i] = fast_exp2(__builtin_fmaf(acc16[qg][i], c16, -m_use[qg]));
                if constexpr (kMasked) e[i] = ((vis[qg] >> (c * 4 + i)) & 1u) ? e[i] : 0.0f;
            }
            P[qg][c] = u32x2{f32x2_to_bf16x2(e[0], e[1]), f32x2_to_bf16x2(e[2], e[3])};
        }
    };
    auto recompute = [&](u32x2 (&P)[kQG][4], uint32_t flags, auto masked_tag, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (!((flags >> c) & 1u)) continue;
            v4f acc16[kQG];
            recompute_mfma(acc16, c, slot);
            recompute_exp(P, acc16, c, masked_tag);
        }
    };

    // debug: the final weights of tile t
    auto dump_p = [&](const u32x2 (&P)[kQG][4], int t) __attribute__((always_inline)) {
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
    };
    // (6) online-softmax rescale of everything accumulated so far, before the
    //     P.V of tile t
    auto rescale = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int qg = 0; qg < kQG; ++qg) {
            if (wave_ballot(alpha[qg] != 1.0f) != 0) {
                acc_l[qg] *= alpha[qg];
#pragma unroll
                for (int db = 0; db < C::kDB; ++db) acc_o[qg][db] *= alpha[qg];
            }
        }
    };

    v4f S[kQG][4];
    u32x2 P[kQG][4];
    constexpr auto kFull = std::integral_constant<bool, false>{};
    constexpr auto kPart = std::integral_constant<bool, true>{};
    // waits for this wave's outstanding copies into LDS (and global stores)
    auto wait_copies = []() __attribute__((always_inline)) {
        __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory");
    };
    if constexpr (C::kPP) {
        // ---- ping-pong schedule ---------------------------------------------------------
        // Waves 0-3 (one per SIMD) and waves 4-7 run the same sequence of phases,
        // the second group one phase behind the first, so that on every SIMD one
        // wave is in a vector phase while the other is in a matrix phase:
        //   V(t): running max, exponentials, rescale and test of tile t, flags
        //         out;
        //   M(t): Q.K^T of tile t+1 (the logits of t are dead), 16-bit
        //         recompute and P.V of tile t, and the copies of K16(t+2),
        //         V^T(t+2) and K8(t+3) into LDS.
        // A workgroup barrier ends every phase.  Tile u lives in slot u % 3 of
        // each array.  Both groups read the K16 and V^T tiles of t and the K8
        // tile of t+1 in M(t), two consecutive phases; the copies a group issues
        // in M(t) overwrite tiles t-1 (K16, V^T) and t (K8), which both groups
        // finished reading in M(t-1), and they are complete (each wave waits
        // for its own before issuing the next ones, in M(t+1)) before the first
        // reader, the first group's M(t+2).  In the plain bf16 mode
        // the Q.K^T tiles are K16 tiles, staged like K8, and there is no test or
        // recompute.
        __shared__ uint32_t flag_lds[kWaves];    // 4-bit flag sets exchanged by the waves of a block
        const int grp = wave >> 2;
        int s_cur = t_begin % 3;                 // slot of tile t
        const int s_b1 = s_cur == 2 ? 0 : s_cur + 1;
        const int s_b2 = s_b1 == 2 ? 0 : s_b1 + 1;
        // the tiles the first two matrix phases read, and K8 of the third
        dma_qk(t_begin, s_cur);
        if (t_begin + 1 <= t_end) dma_qk(t_begin + 1, s_b1);
        if (t_begin + 2 <= t_end) dma_qk(t_begin + 2, s_b2);
        if constexpr (!kPlain) dma_k16(t_begin, s_cur);
        dma_vt(t_begin, s_cur);
        if (t_begin + 1 <= t_end) {
            if constexpr (!kPlain) dma_k16(t_begin + 1, s_b1);
            dma_vt(t_begin + 1, s_b1);
        }
        wait_copies();
        lds_barrier();
        if (grp == 1) lds_barrier();
        // M(t_begin - 1): the first Q.K^T
        if (work(t_begin)) qk(S, s_cur);
        lds_barrier();
        for (int t = t_begin; t <= t_end; ++t) {
            const bool w_cur = work(t), w_next = work(t + 1);
            const bool full = full_tile(t);
            const int s_n1 = s_cur == 2 ? 0 : s_cur + 1;   // slot of t+1
            const int s_n2 = s_n1 == 2 ? 0 : s_n1 + 1;     // slot of t+2 (and t-1)
            // ---- V(t)
            uint32_t flags = 0;
            if (w_cur) {
                round_logits(S);
                if (full) softmax(S, P, t, kFull);
                else softmax(S, P, t, kPart);
                rescale();
                if constexpr (!kPlain) flags = full ? test(S, kFull) : test(S, kPart);
            }
            if (lane == 0) flag_lds[wave] = flags;
            lds_barrier();
            // ---- M(t), at raised issue priority: the matrix-core work of this wave
            // goes first and the vector work of the other wave fills around it
            __builtin_amdgcn_s_setprio(1);
            flags = 0;
#pragma unroll
            for (int w = 0; w < C::kWavesPerBlock; ++w) flags |= flag_lds[blk * C::kWavesPerBlock + w];
            flags = __builtin_amdgcn_readfirstlane(flags);
            if (w_next) qk(S, s_n1);
            if (w_cur) {
                if constexpr (kPlain) {
                    flags = 0xFu;   // every sub-block in 16-bit
                } else if (flags != 0) {
                    if (full) recompute(P, flags, kFull, s_cur);
                    else recompute(P, flags, kPart, s_cur);
                }
                dump_p(P, t);
            }
            if (w_cur) pv(P, s_cur, [](int) {});
            // copies for later tiles, after this wave's previous ones have landed
            wait_copies();
#pragma unroll
            for (int k = 0; k < kDmaSteps; ++k) dma_step(k, t + 2, s_n2, t + 3, s_cur);
#ifdef LAMP_EXTRA_SYNC
            wait_copies();   // test build: the copies land within the phase that issues them
#endif
            if (w_cur && a.mask && wib == 0 && lane == 0)
                a.mask[(q_head * a.nT + r) * a.nT + t] = (uint8_t)(0x80u | flags);
            __builtin_amdgcn_s_setprio(0);
            lds_barrier();
            s_cur = s_n1;
        }
        if (grp == 0) lds_barrier();
    } else {
        // ---- one software-pipelined loop (D = 256) ----------------------------------------
        // Iteration t: copies of K8(t+1) into slot (t+1) & 1; P.V of tile t-1,
        // with the copies of K16(t+1) into slot (t+1) & 1 and of V^T(t) into
        // slot t & 1 issued between its products (one after every fourth output
        // block: issued together at the top, they held every wave at the
        // address unit); max, exponentials and test of tile t; flag barrier;
        // recompute of tile t; Q.K^T of tile t+1; rescale; barrier.
        // The copies overwrite K8(t-1), K16(t-1) and V^T(t-2), whose last
        // readers (Q.K^T in iteration t-2, the recompute and P.V in iteration
        // t-1) are behind the previous barrier.  Each wave waits for its K8 copy
        // before the flag barrier (Q.K^T of t+1 follows it) and for the rest
        // before the closing barrier.  The 4-bit flag sets go through the first
        // bytes of K8 slot t & 1: K8(t) has been read, and K8(t+2) is copied
        // there only after the closing barrier.  Waves 0-3 issue at a raised
        // priority, so that the wave sharing their SIMD falls behind and runs
        // its matrix products under their vector work rather than beside them.
        // (the plain bf16 mode stages its Q.K^T operand, K16, in the K8 slots
        // and copies no separate K16 tiles)
        constexpr int kK16Copies = kPlain ? 0 : kK16Ch;
        constexpr int kAfterK8 = kK16Copies + kVtCh;    // copies issued after a tile's K8 copies
        static_assert(kAfterK8 < 16, "vmcnt immediate");
        static_assert(kAfterK8 <= C::kDB / 2, "one copy per four output blocks of P.V");
        wait_copies();
        lds_barrier();
        if (work(t_begin)) qk(S, t_begin & 1);
        lds_barrier();   // every wave has read K8(t_begin): its slot takes the flags
        if (wave_u < C::kWavesPerBlock) __builtin_amdgcn_s_setprio(3);
        for (int t = t_begin; t <= t_end; ++t) {
            const int sc = t & 1, sn = sc ^ 1;
            if (t + 1 <= t_end) dma_qk(t + 1, sn);
#ifdef LAMP_EXTRA_SYNC
            wait_copies();   // test build: every copy lands where it is issued
#endif
            const bool w_prev = work(t - 1), w_cur = work(t), w_next = work(t + 1);
            const bool full = full_tile(t);
            auto copy = [&](int k) __attribute__((always_inline)) {
                if (k < kK16Copies) {
                    if constexpr (!kPlain)
                        if (t + 1 <= t_end) dma_k16_i(t + 1, sn, k);
                } else if (k < kAfterK8) {
                    dma_vt_i(t, sc, k - kK16Copies);
                }
            };
            // P.V of tile t-1 reads P before the exponentials of tile t overwrite it
            if (w_prev) {
                pv(P, sn, copy);
            } else {
#pragma unroll
                for (int k = 0; k < kAfterK8; ++k) copy(k);
            }
#ifdef LAMP_EXTRA_SYNC
            wait_copies();
#endif
            uint32_t flags = 0u;
            if (w_cur) {
                round_logits(S);
                if (full) softmax(S, P, t, kFull);
                else softmax(S, P, t, kPart);
                if constexpr (kPlain) flags = 0xFu;   // every sub-block in 16-bit
                else flags = full ? test(S, kFull) : test(S, kPart);
            }
            // the waves of a 64-row block OR their flags
            uint32_t* flag_slot = reinterpret_cast<uint32_t*>(lds + C::kK8Off + sc * C::kQKBytes);
            if (lane == 0) flag_slot[wave] = flags;
            // this wave's K8(t+1) copies have landed (at most kAfterK8 newer
            // copies outstanding; an iteration without them waits for nothing)
            __asm__ __volatile__("s_waitcnt vmcnt(%0)" ::"n"(kAfterK8) : "memory");
            lds_barrier();
            flags = 0;
#pragma unroll
            for (int w = 0; w < C::kWavesPerBlock; ++w) flags |= flag_slot[blk * C::kWavesPerBlock + w];
            flags = __builtin_amdgcn_readfirstlane(flags);
            if constexpr (!kPlain) {
                if (w_cur && flags != 0) {
                    if (full) recompute(P, flags, kFull, sc);
                    else recompute(P, flags, kPart, sc);
                }
            }
            // Q.K^T of tile t+1 runs on the matrix cores under what follows
            if (w_next) qk(S, sn);
            if (w_cur) {
                dump_p(P, t);
                rescale();
                // (7) mask byte
                if (a.mask && wib == 0 && lane == 0)
                    a.mask[(q_head * a.nT + r) * a.nT + t] = (uint8_t)(0x80u | flags);
            }
            wait_copies();
            lds_barrier();
        }
        __builtin_amdgcn_s_setprio(0);
        // P.V of the last tile
        if (work(t_end)) pv(P, t_end & 1, [](int) {});
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
    };
    run_rows(a.n_rg - 1 - level);
    // (D = 256 launches are never paired: they would carry the register cost
    // of the second run without the balance it buys at these grid sizes)
    if constexpr (C::kPP)
        if (a.paired && level != a.n_rg - 1 - level) run_rows(level);
}

template <int D>
hipError_t launch_d(const Shape& sh, const AttnParams& p, hipStream_t st) {
    AttnArgs a;
    a.k8 = p.k8; a.q16 = p.q16; a.k16 = p.k16; a.vt = p.vt;
    a.q_scale = p.q_scale; a.q_inv = p.q_inv; a.k_scale = p.k_scale; a.out = p.out; a.mask = p.mask;
    a.dump_s = p.dump_s; a.dump_p = p.dump_p;
    a.l_d = p.log2e_over_sqrt_d; a.t2 = p.t2;
    a.x_delta = p.e_delta > 0.0f ? (float)std::log2((double)p.e_delta) : -__builtin_inff();
    a.test_mode = !(p.t2 < __builtin_inff()) || !(p.e_delta < __builtin_inff()) ? 0 : (p.e_delta > 0.0f ? 1 : 2);
    a.B = sh.B; a.Hq = sh.Hq; a.Hkv = sh.Hkv; a.S = sh.S; a.nT = sh.nT; a.S_pad = sh.S_pad;
    a.causal = p.causal; a.window = p.window;
    a.G = sh.Hq / sh.Hkv;
    a.heads_per_wg = 1;
    for (int h = Cfg<D>::kBlocks; h >= 1; h /= 2)
        if (a.G % h == 0) { a.heads_per_wg = h; break; }
    a.rows_per_wg = Cfg<D>::kBlocks / a.heads_per_wg;
    a.n_rg = (sh.nT + a.rows_per_wg - 1) / a.rows_per_wg;
    // pair row-block groups where the unpaired grid gives at most two
    // workgroups per CU and the rows differ in length (causal, no window)
    const int n_u = sh.B * sh.Hkv * (a.G / a.heads_per_wg);
    a.paired = Cfg<D>::kPP && p.causal && p.window == 0 && n_u * a.n_rg <= 2 * cu_count() ? 1 : 0;
    a.n_wg = n_u * (a.paired ? (a.n_rg + 1) / 2 : a.n_rg);
    // the run length of one unit on an XCD (measured: 16 row blocks at D = 256
    // global and with few units, 4 with a window at D = 256, 1 with 16 units
    // or more, where an XCD holds several units at every level anyway)
    a.rot_shift = D == 256 ? (p.window > 0 ? 2 : 4) : (n_u >= 16 ? 0 : 4);
    size_t lds = Cfg<D>::kLdsBytes;
    const bool dump = p.dump_s != nullptr && p.dump_p != nullptr;
    using Fn = void (*)(AttnArgs);
    static const Fn table[2][2][3] = {
        {{lamp_attn_kernel<D, false, 0>, lamp_attn_kernel<D, false, 1>, lamp_attn_kernel<D, false, 2>},
         {lamp_attn_kernel<D, true, 0>, lamp_attn_kernel<D, true, 1>, lamp_attn_kernel<D, true, 2>}},
        {{lamp_attn_kernel<D, false, 4>, lamp_attn_kernel<D, false, 5>, lamp_attn_kernel<D, false, 6>},
         {lamp_attn_kernel<D, true, 4>, lamp_attn_kernel<D, true, 5>, lamp_attn_kernel<D, true, 6>}}};
    Fn fn = table[p.logit8 ? 1 : 0][dump ? 1 : 0][a.test_mode];
    // Small tau: rows whose running max is below -t2 - x_delta take the
    // per-entry test, and with t2 + x_delta <= -5 nearly every wave does;
    // there its vector form is faster (measured 256 against 275 us at
    // tau = 2^-3, qwen3-8b), elsewhere slower (240 against 221 at 2^-2).
    if (!p.logit8 && !p.plain && a.test_mode == 1 && a.t2 + a.x_delta <= -5.0f)
        fn = dump ? lamp_attn_kernel<D, true, 9> : lamp_attn_kernel<D, false, 9>;
    if (p.exp_poly && !p.logit8 && !p.plain) {
        static const Fn poly[2][3] = {
            {lamp_attn_kernel<D, false, 16>, lamp_attn_kernel<D, false, 17>, lamp_attn_kernel<D, false, 18>},
            {lamp_attn_kernel<D, true, 16>, lamp_attn_kernel<D, true, 17>, lamp_attn_kernel<D, true, 18>}};
        fn = poly[dump ? 1 : 0][a.test_mode];
    }
    if (p.plain) {
        fn = dump ? lamp_attn_kernel<D, true, 3> : lamp_attn_kernel<D, false, 3>;
        lds = Cfg<D, true>::kLdsBytes;
    }
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(a.n_wg), dim3(kThreads), lds, st, a);
    return hipGetLastError();
}

// Test hook: the 8-bit Q.K^T instruction of the attention kernel on given
// operand blocks.  One wave per block: a [16 rows][128] and b [16 rows][128]
// e4m3 codes, out [16][16] fp32 = a . b^T, with the operand arrangement of
// qk() (lane group g holds depth 32g .. 32g+31 of row n16 of each operand).
__global__ __launch_bounds__(64) void debug_fp8_dot_kernel(const uint8_t* __restrict__ a,
                                                           const uint8_t* __restrict__ b, float* out,
                                                           int n) {
    const int blk = blockIdx.x;
    if (blk >= n) return;
    const int lane = threadIdx.x, n16 = lane & 15, g = lane >> 4;
    const v8i ka = fp8_operand_global<128>(a + ((size_t)blk * 16 + n16) * 128, 0, g);
    const v8i qb = fp8_operand_global<128>(b + ((size_t)blk * 16 + n16) * 128, 0, g);
    const v4f s = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qb, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                                    0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[((size_t)blk * 16 + 4 * g + i) * 16 + n16] = s[i];
}

}  // namespace

hipError_t launch_debug_fp8_dot(const uint8_t* a, const uint8_t* b, float* out, int n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(debug_fp8_dot_kernel, dim3((unsigned)n), dim3(64), 0, st, a, b, out, n);
    return hipGetLastError();
}

hipError_t launch_attention(const Shape& sh, const AttnParams& p, hipStream_t st) {
    if (sh.D == 64) return launch_d<64>(sh, p, st);
    if (sh.D == 128) return launch_d<128>(sh, p, st);
    if (sh.D == 256) return launch_d<256>(sh, p, st);
    return hipErrorInvalidValue;
}

}  // namespace lamp
