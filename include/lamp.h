/*
 * lamp.h -- C ABI of the MI355X (gfx950) LampAttention forward pass.
 *
 * The method is the one of "LampAttention: Look-Ahead Mixed-Precision
 * FlashAttention for Dedicated Accelerators" (abstract): a FlashAttention that
 * sums key-query products and takes exponentials with 8-bit number formats,
 * finds the sensitive sub-blocks (look-ahead test with parameters delta and
 * tau, figure 1-8 captions) and redoes only those with 16-bit ones.  Tables
 * 1-6 count the 16-bit sub-blocks of each tile.
 *
 * Readings this library implements (the pages give no formula, format or size):
 *   - tiles of 64 query rows x 64 keys, four 64 x 16 sub-blocks per tile;
 *   - 8-bit = OCP e4m3fn with per-(batch, head) amax/448 scales for Q and K;
 *     products summed in fp32, exponentials rounded to e4m3;
 *   - 16-bit = bf16 operands, fp32 accumulation, exponentials rounded to bf16;
 *   - logits in the log2 domain; running row max from the 8-bit logits;
 *   - first stage: p8 >= delta (delta <= 0 disables it);
 *     second stage: |s| >= 16 * tau * log2(e) (log2-domain logit);
 *     a sub-block is recomputed iff some entry passes both stages.
 *
 * Conventions for every entry point
 *   - Tensors are caller-owned, contiguous, row-major.  Q is [B, Hq, S, D],
 *     K and V are [B, Hkv, S, D], all bf16 (raw 16-bit patterns).  Query head
 *     hq reads kv head hq / (Hq / Hkv).  Device pointers must be 16-byte aligned.
 *   - Calls are asynchronous on the library's current stream (lamp_set_stream);
 *     outputs are valid after that stream is synchronised.  A device fault
 *     surfaces at that synchronisation, not at the call.
 *   - Arguments are validated before any HIP call; on a validation error
 *     nothing is launched and nothing is written.  The return value is LAMP_OK
 *     or a negative error code; lamp_last_error() gives a message.
 *   - The library owns one device workspace per (device, stream) pair (K8, a
 *     transposed copy of V, scales, decode split results), allocated on the
 *     first call on that stream; it only grows (the old buffer is freed after
 *     that stream drains), and lamp_release_workspace() frees all of them.
 *     Calls on different streams use different workspaces and may overlap in
 *     time; calls on one stream run in order.  At most 64 (device, stream)
 *     pairs hold a workspace at a time (LAMP_ERR_UNSUPPORTED beyond that).
 *     LAMP_WORKSPACE_LIMIT_BYTES (environment, bytes) caps one workspace:
 *     a call that needs more returns LAMP_ERR_NOMEM and launches nothing.
 *   - Inputs must be finite, and every Q and K head whose largest magnitude
 *     is not 0 has it at least 2^-119, so that the inverse scale 448/amax is
 *     finite in fp32 (then no scaled value rounds beyond +-448).  The stream
 *     and the last error are per host thread; host threads may call
 *     concurrently on distinct streams.
 */
#ifndef LAMP_H
#define LAMP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    LAMP_OK = 0,
    LAMP_ERR_INVALID = -1,      /* bad pointer, size, flag or parameter */
    LAMP_ERR_UNSUPPORTED = -2,  /* valid request this build does not handle (e.g. D not in {64,128,256}) */
    LAMP_ERR_HIP = -3,          /* a HIP runtime call failed (message has hipGetErrorString) */
    LAMP_ERR_NOMEM = -4         /* workspace allocation failed or exceeded LAMP_WORKSPACE_LIMIT_BYTES */
};

/* Forward pass.  ("LampAttention", abstract; tables 1-6 for the mask.)
 *   q, k, v   bf16 device tensors as above.
 *   out       fp32 device tensor [B, Hq, S, D]: softmax(QK^T/sqrt(D)) V as computed
 *             by the method.
 *   causal    0 or 1: key j is visible to query i iff j <= i.
 *   window    0 = none; > 0 requires causal = 1 and additionally i - j < window.
 *   delta     first-stage threshold on the 8-bit exponential; <= 0 disables the stage.
 *   tau       second-stage parameter; +inf disables it (pure 8-bit attention);
 *             tau <= 0 with delta <= 0 sends every visited sub-block to 16-bit.
 *   subblock_mask_out  nullable; uint8 device tensor [B, Hq, nT, nT], nT = ceil(S/64).
 *             Byte (b, hq, r, t): bit 7 = tile (query rows 64r.., keys 64t..) visited,
 *             bit c (0..3) = sub-block c (keys 64t+16c .. 64t+16c+15) recomputed in
 *             16-bit; 0 for tiles that hold no visible entry.
 * Sizes: B, Hq, Hkv, S >= 1; Hq % Hkv == 0; D in {64, 128, 256}; per head
 * S_pad*D < 2^30 (S_pad = 64 nT); B*(Hq+2*Hkv)*nT < 2^29 (launch grids).  The
 * tensors themselves may exceed 2^31 elements. */
int lamp_attn_fwd(const void* q, const void* k, const void* v, float* out,
                  int B, int Hq, int Hkv, int S, int D,
                  int causal, int window, float delta, float tau,
                  uint8_t* subblock_mask_out);

/* lamp_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results, with the workspace in a fixed device array of
 * 64 MiB (67108864 bytes) per device instead of the per-stream workspace.
 * Nothing is allocated or freed by the call (no hipMalloc, hipFree or
 * allocating library routine); the array is part of the library's code object
 * and each device holds its copy until the process ends.  The workspace needs
 * about 3 * B * Hkv * ceil(S/64) * 64 * D bytes (K8 and the transposed V) plus
 * per-head scales; a call needing more than 64 MiB returns
 * LAMP_ERR_UNSUPPORTED and launches nothing.  Every call on a device shares
 * that device's array: calls that overlap in time on one device (different
 * streams, or host threads) race on it and must be serialised by the caller.
 * No timing events are recorded.  Arguments, layout, sizes and other errors
 * as lamp_attn_fwd. */
int lamp_attn_fwd_noalloc(const void* q, const void* k, const void* v, float* out,
                          int B, int Hq, int Hkv, int S, int D,
                          int causal, int window, float delta, float tau,
                          uint8_t* subblock_mask_out);

/* The forward pass under a literal reading of the 8-bit accumulation of
 * key-query products ("LampAttention", abstract): the log2-domain logit
 * c * acc (c = log2(e)/sqrt(D) times the Q and K scales) is itself rounded to
 * e4m3 (magnitudes clamped to 448, nearest even) before the running row max,
 * the 8-bit exponentials 2^(s8 - m) and the second stage |s8| >= 16 tau log2(e)
 * read it.  The 16-bit recompute is that of lamp_attn_fwd.  Arguments, layout,
 * sizes and errors as lamp_attn_fwd. */
int lamp_attn_fwd_logit8(const void* q, const void* k, const void* v, float* out,
                         int B, int Hq, int Hkv, int S, int D,
                         int causal, int window, float delta, float tau,
                         uint8_t* subblock_mask_out);

/* The forward pass with bit-reproducible 8-bit exponentials ("LampAttention",
 * abstract: exponentials taken in 8-bit formats; how they are evaluated is not
 * given).  Each 8-bit exponential is e4m3(P(x)), x = fma(acc, c, -m) as in
 * lamp_attn_fwd, where P is an exp2 defined by its fp32 steps, each rounded to
 * nearest even:
 *   x <- max(x, -30);  n = rint(x) (ties to even);  f = x - n;
 *   p = fma(fma(fma(fma(fma(c5, f, c4), f, c3), f, c2), f, c1), f, 1);
 *   P(x) = p * 2^n
 * with c1 = 0x1.62e42ap-1, c2 = 0x1.ebf9aep-3, c3 = 0x1.c6b64ep-5,
 * c4 = 0x1.3cee66p-7, c5 = 0x1.5c10d4p-10 (within 2^-22 of 2^x, relative), so
 * that a CPU evaluation of the same steps gives the same bits; lamp_attn_fwd
 * uses the hardware exp2 instead.  The 16-bit recompute is that of
 * lamp_attn_fwd.  Arguments, layout, sizes and errors as lamp_attn_fwd. */
int lamp_attn_fwd_exp2poly(const void* q, const void* k, const void* v, float* out,
                           int B, int Hq, int Hkv, int S, int D,
                           int causal, int window, float delta, float tau,
                           uint8_t* subblock_mask_out);

/* Decode: Sq query rows, the last positions (Skv - Sq .. Skv - 1) of a sequence,
 * against all Skv cached keys ("LampAttention", abstract: the method per tile as
 * in lamp_attn_fwd).  The Sq rows of a query head form the row block the
 * look-ahead test flags.  The KV tiles (64 keys each) are cut into contiguous
 * splits of tiles_per_split tiles; each split runs the tile loop from an empty
 * state (its own running max, row sum and output) and the splits are merged:
 * out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M the largest running max.
 * The split is part of the operation: the 8-bit exponentials of a split are taken
 * against that split's running max.
 *   q         bf16 device tensor [B, Hq, Sq, D]; k, v bf16 [B, Hkv, Skv, D].
 *   out       fp32 device tensor [B, Hq, Sq, D].
 *   causal, window, delta, tau as in lamp_attn_fwd, with query row i at
 *             position Skv - Sq + i.
 *   tiles_per_split  >= 1: KV tiles per split (clamped to the tile count; more
 *             than 8192 after clamping is LAMP_ERR_UNSUPPORTED);
 *             0: the library's choice, lamp_decode_tiles_per_split.
 *   subblock_mask_out  nullable; uint8 device tensor [B, Hq, nT], nT = ceil(Skv/64):
 *             byte (b, hq, t) as in lamp_attn_fwd for the one row block.
 * Sizes: 1 <= Sq <= 16, Sq <= Skv, Hq % Hkv == 0, Hq/Hkv <= 8, D in {64, 128, 256}
 * (LAMP_ERR_UNSUPPORTED otherwise).  Per call the library workspace also holds
 * B*Hq*n_split*Sq*(D+2) fp32 split results. */
int lamp_attn_decode(const void* q, const void* k, const void* v, float* out,
                     int B, int Hq, int Hkv, int Sq, int Skv, int D,
                     int causal, int window, float delta, float tau,
                     int tiles_per_split, uint8_t* subblock_mask_out);

/* lamp_attn_decode with the per-head K scales taken from kept maxima instead of
 * a pass over all Skv cached keys ("LampAttention", abstract: 8-bit formats
 * for the key-query products; the scale of a K head is its largest magnitude
 * over 448).  A serving loop keeps, per (batch, kv head), the largest bf16
 * magnitude of the keys in its cache, folding in each appended key with
 * lamp_kv_amax_update; the scales, and so the results, are then those of
 * lamp_attn_decode bit for bit.
 *   k_amax_state  uint32 device array [B * Hkv], 4-byte aligned: per (batch,
 *             kv head) the largest magnitude bits (bf16 bits & 0x7FFF) over all
 *             Skv cached keys, as lamp_kv_amax_update leaves it.  Read only.
 * Other arguments, layout, sizes and errors as lamp_attn_decode. */
int lamp_attn_decode_with_amax(const void* q, const void* k, const void* v, float* out,
                               int B, int Hq, int Hkv, int Sq, int Skv, int D,
                               int causal, int window, float delta, float tau,
                               int tiles_per_split, const uint32_t* k_amax_state,
                               uint8_t* subblock_mask_out);

/* Folds new keys into kept K maxima (the state lamp_attn_decode_with_amax
 * reads): k_amax_state[b * Hkv + h] becomes the larger of itself and the
 * largest bf16 magnitude bits (bits & 0x7FFF) of k_new[b, h, :, :].  The
 * caller zero-fills the state of an empty cache.  Integer maxima are exact and
 * independent of order, so passing a cache's keys in any number of pieces
 * leaves the amax of all of them.
 *   k_new     bf16 device tensor [B, Hkv, S_new, D], 16-byte aligned.
 *   k_amax_state  uint32 device array [B * Hkv], 4-byte aligned, updated in place.
 * Sizes: B, Hkv, S_new >= 1; D in {64, 128, 256}; S_new*D < 2^30; B*Hkv <= 65535
 * (LAMP_ERR_UNSUPPORTED otherwise).  Calls that update one state on different
 * streams race only in the order of their updates, not in the result. */
int lamp_kv_amax_update(const void* k_new, int B, int Hkv, int S_new, int D,
                        uint32_t* k_amax_state);

/* The tiles_per_split lamp_attn_decode uses when passed 0: the fewest tiles per
 * split that still give one workgroup slot of the current device a split (two
 * per compute unit, one when Hq/Hkv > 4 or D = 256); a negative error code for
 * sizes lamp_attn_decode rejects.  Launches nothing. */
int lamp_decode_tiles_per_split(int B, int Hq, int Hkv, int Sq, int Skv, int D);

/* The 16-bit baseline: plain bf16 FlashAttention on the same tiles ("16-bit"
 * column of tables 1-6 read as a kernel; no 8-bit pass).  Logits are the bf16
 * products accumulated in fp32 on the matrix cores, the running row max comes
 * from them, exponentials are rounded to bf16, and P.V runs in bf16 with fp32
 * accumulation.  Arguments, layout and errors as lamp_attn_fwd without delta
 * and tau; subblock_mask_out gets 0x8F for every visited tile (all four
 * sub-blocks in 16-bit).  Sizes as lamp_attn_fwd (D in {64, 128, 256}). */
int lamp_attn_fwd_bf16(const void* q, const void* k, const void* v, float* out,
                       int B, int Hq, int Hkv, int S, int D,
                       int causal, int window, uint8_t* subblock_mask_out);

/* Per-tile count of 16-bit sub-blocks, reduced on the device ("16-bit sub-blocks
 * per tile", tables 1-6).  mask is the output of lamp_attn_fwd for the same
 * B, Hq, S, causal, window.  stats_out: int64 device array of LAMP_STATS_LEN:
 *   [0..4] tiles with 0..4 sub-blocks in 16-bit (visited tiles only),
 *   [5] visited tiles, [6] visited sub-blocks (holding a visible entry),
 *   [7] sub-blocks in 16-bit, [8] visible entries, [9] visible entries in
 *   16-bit sub-blocks.  Overwritten, not accumulated.  A mask of 2^31 bytes
 * or more (B * Hq * ceil(S/64)^2) is LAMP_ERR_UNSUPPORTED. */
#define LAMP_STATS_LEN 10
int lamp_subblock_stats(const uint8_t* subblock_mask, int B, int Hq, int S,
                        int causal, int window, int64_t* stats_out);

/* The quantisation step on its own, for tests: Q and K brought to the 8-bit
 * format in which the key-query products are formed ("LampAttention", abstract:
 * 8-bit formats for the products).  Per (batch, head) the largest magnitude
 * amax of the bf16 slab gives the scale fl32(amax/448) and the inverse scale
 * fl32(448/amax) (both 1 for an all-zero head); each element x becomes the
 * e4m3fn code of fl32(x * inverse scale), nearest even.
 *   q [B,Hq,S,D], k [B,Hkv,S,D] bf16 device tensors as for lamp_attn_fwd.
 *   q8 [B,Hq,S,D], k8 [B,Hkv,S,D]: uint8 device outputs (e4m3fn codes, 16-byte
 *   aligned); q_scale [B*Hq], k_scale [B*Hkv]: fp32 device outputs (the scales).
 * Sizes and errors as lamp_attn_fwd, and B*(Hq+Hkv) <= 65535; uses the
 * workspace of the current stream. */
int lamp_quantize_qk(const void* q, const void* k, int B, int Hq, int Hkv, int S, int D,
                     uint8_t* q8, uint8_t* k8, float* q_scale, float* k_scale);

/* The device conversions the kernels use, applied elementwise, for tests:
 *   e4m3[i]  = e4m3fn code of x[i] (nearest even, magnitudes clamped to 448 first),
 *   e4m3_bf16[i] = bf16 pattern of the value of that code,
 *   bf16[i]  = bf16 pattern of x[i] (nearest even),
 *   exp2[i]  = the device fp32 exp2 of x[i].
 * All device pointers (any may be null), n elements. */
int lamp_debug_convert(const float* x, int64_t n, uint8_t* e4m3, uint16_t* e4m3_bf16,
                       uint16_t* bf16, float* exp2);

/* The exp2 of lamp_attn_fwd_exp2poly, P(x), applied elementwise on the device,
 * for tests: y[i] = P(x[i]) for n fp32 values (x finite; device pointers). */
int lamp_debug_exp2poly(const float* x, int64_t n, float* y);

/* The instruction that forms the 8-bit key-query products of lamp_attn_fwd
 * ("LampAttention", abstract: products in 8-bit formats), on given operands,
 * for tests of its accumulation: for each of n_blocks blocks,
 *   out[blk][i][j] = sum_{d<128} a[blk][i][d] * b[blk][j][d]
 * as the gfx950 FP8 matrix instruction of the attention kernel computes it
 * (e4m3fn operands, fp32 result; the hardware keeps a limited number of bits
 * below the largest product, so this is not the exactly rounded sum).
 *   a, b  uint8 device arrays [n_blocks, 16, 128] of e4m3fn codes (no NaN codes);
 *   out   fp32 device array [n_blocks, 16, 16].
 * 0 <= n_blocks <= 2^20; pointers 16-byte aligned. */
int lamp_debug_fp8_dot(const uint8_t* a, const uint8_t* b, float* out, int n_blocks);

/* lamp_attn_fwd plus a dump of its per-entry intermediates, for tests on small
 * shapes (S <= 2048).  For every visible (query i, key j) of head (b, hq):
 *   acc8_out [B, Hq, S, S] fp32: the 8-bit accumulator sum_d Q8[i,d] K8[j,d];
 *   p_out    [B, Hq, S, S] bf16 bits: the weight that entered P.V (the 8-bit
 *            exponential, or the 16-bit one for a recomputed sub-block), relative to
 *            the running row max at that tile.
 * Entries of tiles that are not visited are not written. */
int lamp_debug_attn_dump(const void* q, const void* k, const void* v, float* out,
                         int B, int Hq, int Hkv, int S, int D,
                         int causal, int window, float delta, float tau,
                         uint8_t* subblock_mask_out, float* acc8_out, uint16_t* p_out);

/* lamp_debug_attn_dump for lamp_attn_fwd_logit8: logit8_out [B, Hq, S, S] fp32
 * receives the 8-bit logit (an e4m3 value) of every visible entry instead of
 * the accumulator; p_out, sizes and errors as lamp_debug_attn_dump. */
int lamp_debug_attn_dump_logit8(const void* q, const void* k, const void* v, float* out,
                                int B, int Hq, int Hkv, int S, int D,
                                int causal, int window, float delta, float tau,
                                uint8_t* subblock_mask_out, float* logit8_out, uint16_t* p_out);

/* lamp_debug_attn_dump for lamp_attn_fwd_exp2poly: the same dump of the
 * 8-bit accumulators and of the weights that entered P.V; sizes and errors as
 * lamp_debug_attn_dump. */
int lamp_debug_attn_dump_exp2poly(const void* q, const void* k, const void* v, float* out,
                                  int B, int Hq, int Hkv, int S, int D,
                                  int causal, int window, float delta, float tau,
                                  uint8_t* subblock_mask_out, float* acc8_out, uint16_t* p_out);

/* Per-kernel timing with HIP events recorded on the library's stream, for
 * benches.  While enabled (enable = 1), every lamp_attn_fwd and
 * lamp_attn_decode call records one event before its preparation kernels
 * (quantisation and transpose; for decode the K amax and the scales), one
 * between them and the attention (decode) kernel and one right after that
 * kernel (the decode merge follows it, untimed).  lamp_read_timing waits for
 * those events, returns the summed milliseconds of the two phases and the
 * number of calls, and starts a new accumulation.  Event objects are created on first
 * use and reused; at most 4096 calls are recorded between two reads. */
int lamp_set_timing(int enable);
int lamp_read_timing(double* prep_ms, double* attn_ms, int* n_calls);

/* Stream for subsequent calls from this host thread (a hipStream_t; null = default). */
int lamp_set_stream(void* hip_stream);

/* Message of the last non-OK return on this host thread ("" if none). */
const char* lamp_last_error(void);

/* Free every workspace (synchronises each device that holds one first). */
void lamp_release_workspace(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int lamp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LAMP_H */
