// Host side of the C ABI declared in include/lamp.h: argument validation,
// workspace, stream and launch order of the LampAttention forward pass.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>

#include "kernels.hpp"
#include "lamp.h"

namespace {

constexpr double kLog2e = 1.4426950408889634;   // fp64 nearest to log2(e)
constexpr int kMaxDevices = 64;

thread_local hipStream_t g_stream = nullptr;
thread_local std::string g_error;

// One workspace per (device, stream): kernels of calls on different streams
// never share scratch memory, so such calls may overlap in time.
struct Workspace {
    int dev = -1;
    hipStream_t stream = nullptr;
    void* ptr = nullptr;
    size_t bytes = 0;
};
constexpr int kMaxWorkspaces = 64;
std::mutex g_ws_mutex;
Workspace g_ws[kMaxWorkspaces];

// Event timing of lamp_attn_fwd phases (lamp_set_timing / lamp_read_timing).
constexpr int kMaxTimed = 4096;
thread_local bool g_timing = false;
thread_local int g_n_timed = 0;
thread_local hipEvent_t g_events[kMaxTimed][3];

// The next free slot of three events, or null when timing is off or every
// slot is taken.  The slot counts as used only after timing_commit, which a
// call reaches once all of its launches have been enqueued: a call that fails
// part way leaves no half-recorded slot behind.
hipEvent_t* timing_slot() {
    if (!g_timing || g_n_timed >= kMaxTimed) return nullptr;
    hipEvent_t* ev = g_events[g_n_timed];
    for (int i = 0; i < 3; ++i)
        if (!ev[i] && hipEventCreate(&ev[i]) != hipSuccess) return nullptr;
    return ev;
}

void timing_commit(hipEvent_t* ev) {
    if (hipEventRecord(ev[2], g_stream) == hipSuccess) ++g_n_timed;
}

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(LAMP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t workspace_limit() {
    const char* s = std::getenv("LAMP_WORKSPACE_LIMIT_BYTES");
    if (!s || !*s) return SIZE_MAX;
    return (size_t)std::strtoull(s, nullptr, 10);
}

// Returns LAMP_OK and a device pointer to at least `bytes` of workspace for
// the current device and the calling thread's stream.  Grows only; the old
// buffer is freed after that stream has drained, since only kernels on it
// read that buffer.
int get_workspace(size_t bytes, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(LAMP_ERR_UNSUPPORTED, "device index %d", dev);
    if (bytes > workspace_limit())
        return fail(LAMP_ERR_NOMEM, "workspace of %zu bytes exceeds LAMP_WORKSPACE_LIMIT_BYTES", bytes);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace* slot = nullptr;
    for (auto& w : g_ws)
        if (w.dev == dev && w.stream == g_stream) { slot = &w; break; }
    if (!slot)
        for (auto& w : g_ws)
            if (w.dev < 0) { slot = &w; w.dev = dev; w.stream = g_stream; break; }
    if (!slot)
        return fail(LAMP_ERR_UNSUPPORTED, "more than %d (device, stream) pairs hold a workspace; "
                    "call lamp_release_workspace", kMaxWorkspaces);
    Workspace& ws = *slot;
    if (ws.bytes < bytes) {
        if (ws.ptr) {
            e = hipStreamSynchronize(g_stream);
            if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
            (void)hipFree(ws.ptr);
            ws.ptr = nullptr;
            ws.bytes = 0;
        }
        void* p = nullptr;
        e = hipMalloc(&p, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(LAMP_ERR_NOMEM, "hipMalloc(%zu): %s", bytes, hipGetErrorString(e));
        }
        ws.ptr = p;
        ws.bytes = bytes;
    }
    *out = ws.ptr;
    return LAMP_OK;
}

// Whether the product of positive factors (each below 2^32) reaches `limit`
// (at most 2^31): the running product is checked after every factor, so it
// never overflows.
bool product_reaches(std::initializer_list<int64_t> factors, int64_t limit) {
    int64_t p = 1;
    for (int64_t f : factors) {
        p *= f;
        if (p >= limit) return true;
    }
    return false;
}

int check_sizes(int B, int Hq, int Hkv, int S, int D) {
    if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || D < 1)
        return fail(LAMP_ERR_INVALID, "sizes must be >= 1 (B=%d Hq=%d Hkv=%d S=%d D=%d)", B, Hq, Hkv, S, D);
    if (Hq % Hkv != 0) return fail(LAMP_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (D != 64 && D != 128 && D != 256)
        return fail(LAMP_ERR_UNSUPPORTED, "head dimension D=%d (supported: 64, 128, 256)", D);
    const int64_t nT = ((int64_t)S + 63) / 64;   // 64-bit: S may be INT_MAX
    // Addresses across heads are 64-bit everywhere; within one (batch, head)
    // slab the kernels use 32-bit offsets and buffer sizes of S_pad * 2D bytes,
    // and the launches have at most B (Hq + 2 Hkv) nT (D / 64) workgroups.
    if (product_reaches({nT * 64, D}, (int64_t)1 << 30))
        return fail(LAMP_ERR_UNSUPPORTED, "S*D (S padded to 64) reaches 2^30 per head (S=%d D=%d)", S, D);
    if (product_reaches({B, (int64_t)Hq + 2 * (int64_t)Hkv, nT}, (int64_t)1 << 29))
        return fail(LAMP_ERR_UNSUPPORTED, "B*(Hq+2*Hkv)*ceil(S/64) reaches 2^29 (B=%d Hq=%d Hkv=%d S=%d)",
                    B, Hq, Hkv, S);
    return LAMP_OK;
}

lamp::Shape make_shape(int B, int Hq, int Hkv, int S, int D) {
    lamp::Shape sh;
    sh.B = B; sh.Hq = Hq; sh.Hkv = Hkv; sh.S = S; sh.D = D;
    sh.nT = (S + 63) / 64;
    sh.S_pad = sh.nT * 64;
    return sh;
}

// Positive finite e4m3fn values by code 1..126.
double e4m3_value(int code) {
    const int ef = code >> 3, m = code & 7;
    return ef == 0 ? m * std::ldexp(1.0, -9) : (1.0 + m / 8.0) * std::ldexp(1.0, ef - 7);
}

// Smallest fp32 e such that rounding e to e4m3 (nearest, ties to even) gives a
// value >= delta.  The first stage compares the fp32 exponential against it,
// which is the same as comparing its 8-bit rounding against delta.
float exponential_threshold(float delta) {
    if (!(delta > 0.0f)) return -INFINITY;
    int c = 1;
    while (c <= 126 && e4m3_value(c) < (double)delta) ++c;
    if (c > 126) return INFINITY;
    const double below = c == 1 ? 0.0 : e4m3_value(c - 1);
    const float mid = (float)((below + e4m3_value(c)) * 0.5);   // exact: 5 significant bits
    return (c % 2 == 0) ? mid : std::nextafter(mid, INFINITY);
}

struct Layout {
    size_t partial, q_scale, k_scale, q_inv, k8, vt, total;
};

Layout workspace_layout(const lamp::Shape& sh) {
    Layout L;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = round_up(off + bytes, 256); return o; };
    const size_t nslab = (size_t)sh.B * (sh.Hq + sh.Hkv);
    L.partial = take(nslab * lamp::amax_chunks(sh.S, sh.D) * sizeof(uint32_t));
    L.q_scale = take((size_t)sh.B * sh.Hq * sizeof(float));
    L.q_inv = take((size_t)sh.B * sh.Hq * sizeof(float));
    L.k_scale = take((size_t)sh.B * sh.Hkv * sizeof(float));
    L.k8 = take((size_t)sh.B * sh.Hkv * sh.S_pad * sh.D);
    L.vt = take((size_t)sh.B * sh.Hkv * sh.nT * sh.D * 64 * sizeof(uint16_t));
    L.total = off;
    return L;
}

// KV tiles per split of a decode call: enough splits that one round of
// workgroups fills the device (two four-wave or one eight-wave workgroup per
// compute unit: eight waves of two per SIMD), each split at least one tile.
// The decode kernel keeps a split's mask bytes in LDS: at most this many
// tiles per split.
constexpr int kMaxTilesPerSplit = 8192;

int decode_tiles_per_split(int B, int Hq, int Hkv, int Skv, int D) {
    const int nT = (Skv + 63) / 64;
    const int units = B * Hkv;
    const bool wide = Hq / Hkv > 4 || D == 256;
    const int want = (wide ? 1 : 2) * lamp::cu_count();
    int n_split = (want + units - 1) / units;
    if (n_split > nT) n_split = nT;
    if (n_split < (nT + kMaxTilesPerSplit - 1) / kMaxTilesPerSplit)
        n_split = (nT + kMaxTilesPerSplit - 1) / kMaxTilesPerSplit;
    if (n_split < 1) n_split = 1;
    return (nT + n_split - 1) / n_split;
}

int check_decode(int B, int Hq, int Hkv, int Sq, int Skv, int D) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1)
        return fail(LAMP_ERR_INVALID, "sizes must be >= 1 (B=%d Hq=%d Hkv=%d Sq=%d Skv=%d)", B, Hq, Hkv, Sq, Skv);
    if (Hq % Hkv != 0) return fail(LAMP_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (Sq > Skv) return fail(LAMP_ERR_INVALID, "Sq (%d) must not exceed Skv (%d)", Sq, Skv);
    if (D != 64 && D != 128 && D != 256)
        return fail(LAMP_ERR_UNSUPPORTED, "head dimension D=%d (supported: 64, 128, 256)", D);
    if (Sq > 16) return fail(LAMP_ERR_UNSUPPORTED, "decode needs Sq <= 16 (got %d)", Sq);
    if (Hq / Hkv > 8) return fail(LAMP_ERR_UNSUPPORTED, "decode needs Hq/Hkv <= 8 (got %d)", Hq / Hkv);
    const int64_t nT = ((int64_t)Skv + 63) / 64;   // 64-bit: Skv may be INT_MAX
    if (product_reaches({B, Hkv, nT * 64, D}, (int64_t)1 << 31) ||
        product_reaches({B, Hq, Sq, D, nT}, (int64_t)1 << 31))
        return fail(LAMP_ERR_UNSUPPORTED, "decode sizes exceed 2^31 elements");
    return LAMP_OK;
}

}  // namespace

namespace lamp {

int cu_count() {
    static int cached[kMaxDevices] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 256;
    }
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cached[dev] = n;
    }
    return cached[dev];
}

}  // namespace lamp

// plain = 1: plain bf16 FlashAttention (delta and tau unused).
// Workspace of lamp_attn_fwd_noalloc: a fixed device array, one copy per
// device, held until the process ends.  Host code never passes `scratch`
// itself to a kernel or a copy (in host code the name is a host-side stand-in,
// not a device address); it uses the address hipGetSymbolAddress returns for
// the current device.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

// The current device's address of `scratch`, looked up on the first call on
// that device (with that device current).
int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(LAMP_ERR_UNSUPPORTED, "device index %d", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(LAMP_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return LAMP_OK;
}

}  // namespace

// use_scratch = 1: the workspace is the device's fixed scratch array (nothing
// is allocated; sizes beyond it are rejected), and no timing events are used.
static int attn_fwd_impl(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                         int S, int D, int causal, int window, float delta, float tau,
                         uint8_t* subblock_mask_out, float* dump_s, uint16_t* dump_p, int plain,
                         int logit8, int use_scratch = 0, int exp_poly = 0) {
    if (!q || !k || !v || !out) return fail(LAMP_ERR_INVALID, "q, k, v and out must be non-null");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(LAMP_ERR_INVALID, "q, k, v and out must be 16-byte aligned");
    int rc = check_sizes(B, Hq, Hkv, S, D);
    if (rc != LAMP_OK) return rc;
    if (causal != 0 && causal != 1) return fail(LAMP_ERR_INVALID, "causal must be 0 or 1 (got %d)", causal);
    if (window < 0) return fail(LAMP_ERR_INVALID, "window must be >= 0 (got %d)", window);
    if (window > 0 && !causal) return fail(LAMP_ERR_INVALID, "a sliding window requires causal = 1");
    if (!plain && (std::isnan(delta) || std::isnan(tau)))
        return fail(LAMP_ERR_INVALID, "delta and tau must not be NaN");

    const lamp::Shape sh = make_shape(B, Hq, Hkv, S, D);
    const Layout L = workspace_layout(sh);
    void* ws = nullptr;
    if (use_scratch) {
        if (L.total > kScratchBytes)
            return fail(LAMP_ERR_UNSUPPORTED,
                        "lamp_attn_fwd_noalloc: this call needs %zu bytes of workspace, more than the "
                        "fixed %zu-byte scratch array (B*Hkv*ceil(S/64)*64*D*3 bytes plus scales)",
                        L.total, kScratchBytes);
        rc = scratch_address(&ws);
    } else {
        rc = get_workspace(L.total, &ws);
    }
    if (rc != LAMP_OK) return rc;
    uint8_t* base = static_cast<uint8_t*>(ws);

    const uint16_t* q16 = static_cast<const uint16_t*>(q);
    const uint16_t* k16 = static_cast<const uint16_t*>(k);
    const uint16_t* v16 = static_cast<const uint16_t*>(v);
    auto* partial = reinterpret_cast<uint32_t*>(base + L.partial);
    auto* q_scale = reinterpret_cast<float*>(base + L.q_scale);
    auto* k_scale = reinterpret_cast<float*>(base + L.k_scale);
    auto* k8 = base + L.k8;
    auto* vt = reinterpret_cast<uint16_t*>(base + L.vt);

    hipEvent_t* ev = use_scratch ? nullptr : timing_slot();
    if (ev) (void)hipEventRecord(ev[0], g_stream);
    auto* q_inv = reinterpret_cast<float*>(base + L.q_inv);
    // amax partial maxima and the V transpose, then scales and K8 (the
    // attention kernel quantises its Q rows itself); the plain bf16 mode
    // needs only the transpose
    hipError_t e = lamp::launch_amax_transpose(sh, q16, k16, partial, v16, vt, !plain, g_stream);
    if (e != hipSuccess) return hip_fail(e, "amax/transpose launch");
    if (!plain) {
        e = lamp::launch_quantize_codes(sh, q16, k16, partial, q_scale, k_scale, q_inv, nullptr, k8, sh.S_pad,
                                        g_stream);
        if (e != hipSuccess) return hip_fail(e, "quantise launch");
    }
    if (ev) (void)hipEventRecord(ev[1], g_stream);

    lamp::AttnParams p;
    p.k8 = k8; p.q16 = q16; p.k16 = k16; p.vt = vt;
    p.q_scale = q_scale; p.k_scale = k_scale; p.q_inv = q_inv;
    p.out = out; p.mask = subblock_mask_out;
    p.log2e_over_sqrt_d = kLog2e / std::sqrt((double)D);
    p.e_delta = exponential_threshold(delta);
    p.t2 = (float)(16.0 * (double)tau * kLog2e);
    p.causal = causal; p.window = window;
    p.dump_s = dump_s; p.dump_p = dump_p;
    p.plain = plain;
    p.logit8 = logit8;
    p.exp_poly = exp_poly;
    e = lamp::launch_attention(sh, p, g_stream);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    if (ev) timing_commit(ev);
    return LAMP_OK;
}

// lamp_attn_decode, with the K scales from kept maxima (k_amax, B*Hkv values)
// instead of a pass over K when k_amax is not null.
static int decode_impl(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                       int Sq, int Skv, int D, int causal, int window, float delta, float tau,
                       int tiles_per_split, const uint32_t* k_amax, uint8_t* subblock_mask_out) {
    if (!q || !k || !v || !out) return fail(LAMP_ERR_INVALID, "q, k, v and out must be non-null");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(LAMP_ERR_INVALID, "q, k, v and out must be 16-byte aligned");
    int rc = check_decode(B, Hq, Hkv, Sq, Skv, D);
    if (rc != LAMP_OK) return rc;
    if (causal != 0 && causal != 1) return fail(LAMP_ERR_INVALID, "causal must be 0 or 1 (got %d)", causal);
    if (window < 0) return fail(LAMP_ERR_INVALID, "window must be >= 0 (got %d)", window);
    if (window > 0 && !causal) return fail(LAMP_ERR_INVALID, "a sliding window requires causal = 1");
    if (std::isnan(delta) || std::isnan(tau)) return fail(LAMP_ERR_INVALID, "delta and tau must not be NaN");
    if (tiles_per_split < 0)
        return fail(LAMP_ERR_INVALID, "tiles_per_split must be >= 0 (got %d)", tiles_per_split);

    lamp::DecodeShape sh;
    sh.B = B; sh.Hq = Hq; sh.Hkv = Hkv; sh.Sq = Sq; sh.Skv = Skv; sh.D = D;
    sh.nT = (Skv + 63) / 64;
    sh.tps = tiles_per_split > 0 ? (tiles_per_split < sh.nT ? tiles_per_split : sh.nT)
                                 : decode_tiles_per_split(B, Hq, Hkv, Skv, D);
    if (sh.tps > kMaxTilesPerSplit)
        return fail(LAMP_ERR_UNSUPPORTED, "tiles_per_split %d exceeds %d", sh.tps, kMaxTilesPerSplit);
    sh.n_split = (sh.nT + sh.tps - 1) / sh.tps;

    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = round_up(off + bytes, 256); return o; };
    const size_t o_partial = take(k_amax ? 0 : (size_t)B * Hkv * lamp::decode_amax_chunks(Skv, D) * sizeof(uint32_t));
    const size_t o_qs = take((size_t)B * Hq * sizeof(float));
    const size_t o_qi = take((size_t)B * Hq * sizeof(float));
    const size_t o_ks = take((size_t)B * Hkv * sizeof(float));
    const size_t o_ki = take((size_t)B * Hkv * sizeof(float));
    const size_t o_po = take((size_t)B * Hq * sh.n_split * Sq * D * sizeof(float));
    const size_t o_ml = take((size_t)B * Hq * sh.n_split * Sq * 2 * sizeof(float));
    void* ws = nullptr;
    rc = get_workspace(off, &ws);
    if (rc != LAMP_OK) return rc;
    uint8_t* base = static_cast<uint8_t*>(ws);

    lamp::DecodeParams p;
    p.q16 = static_cast<const uint16_t*>(q);
    p.k16 = static_cast<const uint16_t*>(k);
    p.v16 = static_cast<const uint16_t*>(v);
    p.q_scale = reinterpret_cast<float*>(base + o_qs);
    p.q_inv = reinterpret_cast<float*>(base + o_qi);
    p.k_scale = reinterpret_cast<float*>(base + o_ks);
    p.k_inv = reinterpret_cast<float*>(base + o_ki);
    p.part_o = reinterpret_cast<float*>(base + o_po);
    p.part_ml = reinterpret_cast<float*>(base + o_ml);
    p.out = out;
    p.mask = subblock_mask_out;
    p.log2e_over_sqrt_d = kLog2e / std::sqrt((double)D);
    p.e_delta = exponential_threshold(delta);
    p.t2 = (float)(16.0 * (double)tau * kLog2e);
    p.causal = causal;
    p.window = window;

    hipEvent_t* ev = timing_slot();
    if (ev) (void)hipEventRecord(ev[0], g_stream);
    hipError_t e =
        k_amax ? lamp::launch_decode_scales_kept(sh, p.q16, k_amax, reinterpret_cast<float*>(base + o_qs),
                                                 reinterpret_cast<float*>(base + o_qi),
                                                 reinterpret_cast<float*>(base + o_ks),
                                                 reinterpret_cast<float*>(base + o_ki), g_stream)
               : lamp::launch_decode_scales(sh, p.q16, p.k16, reinterpret_cast<uint32_t*>(base + o_partial),
                                            reinterpret_cast<float*>(base + o_qs),
                                            reinterpret_cast<float*>(base + o_qi),
                                            reinterpret_cast<float*>(base + o_ks),
                                            reinterpret_cast<float*>(base + o_ki), g_stream);
    if (e != hipSuccess) return hip_fail(e, "decode scale launch");
    if (ev) (void)hipEventRecord(ev[1], g_stream);
    e = lamp::launch_decode(sh, p, g_stream);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    if (ev) timing_commit(ev);
    e = lamp::launch_decode_merge(sh, p, g_stream);
    if (e != hipSuccess) return hip_fail(e, "decode merge launch");
    return LAMP_OK;
}


extern "C" {

int lamp_attn_fwd(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                  int S, int D, int causal, int window, float delta, float tau,
                  uint8_t* subblock_mask_out) {
    return attn_fwd_impl(q, k, v, out, B, Hq, Hkv, S, D, causal, window, delta, tau, subblock_mask_out,
                         nullptr, nullptr, 0, 0);
}

int lamp_attn_fwd_noalloc(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                          int S, int D, int causal, int window, float delta, float tau,
                          uint8_t* subblock_mask_out) {
    return attn_fwd_impl(q, k, v, out, B, Hq, Hkv, S, D, causal, window, delta, tau, subblock_mask_out,
                         nullptr, nullptr, 0, 0, 1);
}

int lamp_attn_fwd_logit8(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                         int S, int D, int causal, int window, float delta, float tau,
                         uint8_t* subblock_mask_out) {
    return attn_fwd_impl(q, k, v, out, B, Hq, Hkv, S, D, causal, window, delta, tau, subblock_mask_out,
                         nullptr, nullptr, 0, 1);
}

int lamp_attn_fwd_exp2poly(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                           int S, int D, int causal, int window, float delta, float tau,
                           uint8_t* subblock_mask_out) {
    return attn_fwd_impl(q, k, v, out, B, Hq, Hkv, S, D, causal, window, delta, tau, subblock_mask_out,
                         nullptr, nullptr, 0, 0, 0, 1);
}

int lamp_attn_fwd_bf16(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                       int S, int D, int causal, int window, uint8_t* subblock_mask_out) {
    return attn_fwd_impl(q, k, v, out, B, Hq, Hkv, S, D, causal, window, 0.0f, 0.0f, subblock_mask_out,
                         nullptr, nullptr, 1, 0);
}

static int attn_dump_impl(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                          int S, int D, int causal, int window, float delta, float tau,
                          uint8_t* subblock_mask_out, float* acc8_out, uint16_t* p_out, int logit8,
                          int exp_poly = 0) {
    if (!acc8_out || !p_out) return fail(LAMP_ERR_INVALID, "acc8_out and p_out must be non-null");
    if (S > 2048) return fail(LAMP_ERR_UNSUPPORTED, "debug dump needs S <= 2048 (got %d)", S);
    return attn_fwd_impl(q, k, v, out, B, Hq, Hkv, S, D, causal, window, delta, tau, subblock_mask_out,
                         acc8_out, p_out, 0, logit8, 0, exp_poly);
}

int lamp_debug_attn_dump(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                         int S, int D, int causal, int window, float delta, float tau,
                         uint8_t* subblock_mask_out, float* acc8_out, uint16_t* p_out) {
    return attn_dump_impl(q, k, v, out, B, Hq, Hkv, S, D, causal, window, delta, tau, subblock_mask_out,
                          acc8_out, p_out, 0);
}

int lamp_debug_attn_dump_logit8(const void* q, const void* k, const void* v, float* out, int B, int Hq,
                                int Hkv, int S, int D, int causal, int window, float delta, float tau,
                                uint8_t* subblock_mask_out, float* logit8_out, uint16_t* p_out) {
    return attn_dump_impl(q, k, v, out, B, Hq, Hkv, S, D, causal, window, delta, tau, subblock_mask_out,
                          logit8_out, p_out, 1);
}

int lamp_debug_attn_dump_exp2poly(const void* q, const void* k, const void* v, float* out, int B, int Hq,
                                  int Hkv, int S, int D, int causal, int window, float delta, float tau,
                                  uint8_t* subblock_mask_out, float* acc8_out, uint16_t* p_out) {
    return attn_dump_impl(q, k, v, out, B, Hq, Hkv, S, D, causal, window, delta, tau, subblock_mask_out,
                          acc8_out, p_out, 0, 1);
}

int lamp_decode_tiles_per_split(int B, int Hq, int Hkv, int Sq, int Skv, int D) {
    const int rc = check_decode(B, Hq, Hkv, Sq, Skv, D);
    if (rc != LAMP_OK) return rc;
    return decode_tiles_per_split(B, Hq, Hkv, Skv, D);
}

int lamp_attn_decode(const void* q, const void* k, const void* v, float* out, int B, int Hq, int Hkv,
                     int Sq, int Skv, int D, int causal, int window, float delta, float tau,
                     int tiles_per_split, uint8_t* subblock_mask_out) {
    return decode_impl(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, causal, window, delta, tau, tiles_per_split,
                       nullptr, subblock_mask_out);
}

int lamp_attn_decode_with_amax(const void* q, const void* k, const void* v, float* out, int B, int Hq,
                               int Hkv, int Sq, int Skv, int D, int causal, int window, float delta,
                               float tau, int tiles_per_split, const uint32_t* k_amax_state,
                               uint8_t* subblock_mask_out) {
    if (!k_amax_state) return fail(LAMP_ERR_INVALID, "k_amax_state must be non-null");
    if (reinterpret_cast<uintptr_t>(k_amax_state) % 4 != 0)
        return fail(LAMP_ERR_INVALID, "k_amax_state must be 4-byte aligned");
    return decode_impl(q, k, v, out, B, Hq, Hkv, Sq, Skv, D, causal, window, delta, tau, tiles_per_split,
                       k_amax_state, subblock_mask_out);
}

int lamp_kv_amax_update(const void* k_new, int B, int Hkv, int S_new, int D, uint32_t* k_amax_state) {
    if (!k_new || !k_amax_state) return fail(LAMP_ERR_INVALID, "k_new and k_amax_state must be non-null");
    if (!aligned16(k_new)) return fail(LAMP_ERR_INVALID, "k_new must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(k_amax_state) % 4 != 0)
        return fail(LAMP_ERR_INVALID, "k_amax_state must be 4-byte aligned");
    if (B < 1 || Hkv < 1 || S_new < 1)
        return fail(LAMP_ERR_INVALID, "sizes must be >= 1 (B=%d Hkv=%d S_new=%d)", B, Hkv, S_new);
    if (D != 64 && D != 128 && D != 256)
        return fail(LAMP_ERR_UNSUPPORTED, "head dimension D=%d (supported: 64, 128, 256)", D);
    if (product_reaches({S_new, D}, (int64_t)1 << 30))
        return fail(LAMP_ERR_UNSUPPORTED, "S_new*D reaches 2^30 (S_new=%d D=%d)", S_new, D);
    // one grid row per (batch, kv head)
    if ((int64_t)B * Hkv > 65535)
        return fail(LAMP_ERR_UNSUPPORTED, "B*Hkv must be <= 65535 (B=%d Hkv=%d)", B, Hkv);
    hipError_t e = lamp::launch_kv_amax_update(static_cast<const uint16_t*>(k_new), B * Hkv, S_new * D,
                                               k_amax_state, g_stream);
    if (e != hipSuccess) return hip_fail(e, "amax update launch");
    return LAMP_OK;
}

int lamp_set_timing(int enable) {
    if (enable != 0 && enable != 1) return fail(LAMP_ERR_INVALID, "enable must be 0 or 1");
    g_timing = enable != 0;
    return LAMP_OK;
}

int lamp_read_timing(double* prep_ms, double* attn_ms, int* n_calls) {
    if (!prep_ms || !attn_ms || !n_calls) return fail(LAMP_ERR_INVALID, "outputs must be non-null");
    double a = 0.0, b = 0.0;
    const int n = g_n_timed;
    // the slots are released whatever happens below, so that one failed read
    // does not make every later one fail too
    g_n_timed = 0;
    for (int i = 0; i < n; ++i) {
        hipEvent_t* ev = g_events[i];
        hipError_t e = hipEventSynchronize(ev[2]);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        float x = 0.f, y = 0.f;
        e = hipEventElapsedTime(&x, ev[0], ev[1]);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        e = hipEventElapsedTime(&y, ev[1], ev[2]);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        a += x;
        b += y;
    }
    *prep_ms = a;
    *attn_ms = b;
    *n_calls = n;
    return LAMP_OK;
}

int lamp_subblock_stats(const uint8_t* subblock_mask, int B, int Hq, int S, int causal, int window,
                        int64_t* stats_out) {
    if (!subblock_mask || !stats_out) return fail(LAMP_ERR_INVALID, "mask and stats_out must be non-null");
    if (B < 1 || Hq < 1 || S < 1) return fail(LAMP_ERR_INVALID, "sizes must be >= 1");
    const int64_t nT = ((int64_t)S + 63) / 64;
    if (product_reaches({B, Hq, nT, nT}, (int64_t)1 << 31))
        return fail(LAMP_ERR_UNSUPPORTED, "a mask of B*Hq*nT*nT bytes reaches 2^31 (B=%d Hq=%d S=%d)", B, Hq, S);
    if (causal != 0 && causal != 1) return fail(LAMP_ERR_INVALID, "causal must be 0 or 1");
    if (window < 0 || (window > 0 && !causal)) return fail(LAMP_ERR_INVALID, "bad window");
    if ((reinterpret_cast<uintptr_t>(stats_out) & 7u) != 0) return fail(LAMP_ERR_INVALID, "stats_out must be 8-byte aligned");
    hipError_t e = lamp::launch_subblock_stats(subblock_mask, B, Hq, S, causal, window, stats_out, g_stream);
    if (e != hipSuccess) return hip_fail(e, "stats launch");
    return LAMP_OK;
}

int lamp_quantize_qk(const void* q, const void* k, int B, int Hq, int Hkv, int S, int D, uint8_t* q8,
                     uint8_t* k8, float* q_scale, float* k_scale) {
    if (!q || !k || !q8 || !k8 || !q_scale || !k_scale)
        return fail(LAMP_ERR_INVALID, "all pointers must be non-null");
    if (!aligned16(q) || !aligned16(k) || !aligned16(q8) || !aligned16(k8))
        return fail(LAMP_ERR_INVALID, "q, k, q8 and k8 must be 16-byte aligned");
    int rc = check_sizes(B, Hq, Hkv, S, D);
    if (rc != LAMP_OK) return rc;
    // the maxima pass of this entry point runs one grid row per (batch, head)
    if ((int64_t)B * ((int64_t)Hq + Hkv) > 65535)
        return fail(LAMP_ERR_UNSUPPORTED, "lamp_quantize_qk needs B*(Hq+Hkv) <= 65535 (B=%d Hq=%d Hkv=%d)", B, Hq,
                    Hkv);
    const lamp::Shape sh = make_shape(B, Hq, Hkv, S, D);
    const Layout L = workspace_layout(sh);
    void* ws = nullptr;
    rc = get_workspace(L.total, &ws);
    if (rc != LAMP_OK) return rc;
    auto* partial = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + L.partial);
    hipError_t e = lamp::launch_quantize(sh, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                         partial, q_scale, k_scale, nullptr, q8, k8, S, g_stream);
    if (e != hipSuccess) return hip_fail(e, "quantise launch");
    return LAMP_OK;
}

int lamp_debug_convert(const float* x, int64_t n, uint8_t* e4m3, uint16_t* e4m3_bf16, uint16_t* bf16,
                       float* exp2) {
    if (n < 0) return fail(LAMP_ERR_INVALID, "n must be >= 0");
    if (n == 0) return LAMP_OK;
    if (!x) return fail(LAMP_ERR_INVALID, "x must be non-null");
    hipError_t e = lamp::launch_debug_convert(x, n, e4m3, e4m3_bf16, bf16, exp2, g_stream);
    if (e != hipSuccess) return hip_fail(e, "convert launch");
    return LAMP_OK;
}

int lamp_debug_exp2poly(const float* x, int64_t n, float* y) {
    if (n < 0) return fail(LAMP_ERR_INVALID, "n must be >= 0");
    if (n == 0) return LAMP_OK;
    if (!x || !y) return fail(LAMP_ERR_INVALID, "x and y must be non-null");
    hipError_t e = lamp::launch_debug_poly_exp2(x, n, y, g_stream);
    if (e != hipSuccess) return hip_fail(e, "exp2 launch");
    return LAMP_OK;
}

int lamp_debug_fp8_dot(const uint8_t* a, const uint8_t* b, float* out, int n_blocks) {
    if (n_blocks < 0 || n_blocks > (1 << 20))
        return fail(LAMP_ERR_INVALID, "n_blocks must be in [0, 2^20] (got %d)", n_blocks);
    if (n_blocks == 0) return LAMP_OK;
    if (!a || !b || !out) return fail(LAMP_ERR_INVALID, "a, b and out must be non-null");
    if (!aligned16(a) || !aligned16(b) || !aligned16(out))
        return fail(LAMP_ERR_INVALID, "a, b and out must be 16-byte aligned");
    hipError_t e = lamp::launch_debug_fp8_dot(a, b, out, n_blocks, g_stream);
    if (e != hipSuccess) return hip_fail(e, "fp8 dot launch");
    return LAMP_OK;
}

int lamp_set_stream(void* hip_stream) {
    g_stream = static_cast<hipStream_t>(hip_stream);
    return LAMP_OK;
}

const char* lamp_last_error(void) { return g_error.c_str(); }

void lamp_release_workspace(void) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    bool any = false;
    for (auto& ws : g_ws) any |= ws.dev >= 0;
    if (!any) return;
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto& ws : g_ws) {
        if (ws.dev < 0) continue;
        if (ws.ptr) {
            (void)hipSetDevice(ws.dev);
            (void)hipDeviceSynchronize();
            (void)hipFree(ws.ptr);
        }
        ws = Workspace{};
    }
    (void)hipSetDevice(cur);
}

int lamp_version(void) { return 100; }

}  // extern "C"
