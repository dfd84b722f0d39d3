"""ctypes binding of liblamp.so (include/lamp.h): argument marshalling only.

Every function here has the name of the C entry point it calls.  Tensors are
torch tensors on the GPU; torch provides device memory and the current
stream, nothing else.  There is no fallback: if the HIP library is not built,
or a call fails, a RuntimeError is raised.
"""
import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblamp.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "lamp.h")

LAMP_OK = 0
LAMP_ERR_INVALID = -1
LAMP_ERR_UNSUPPORTED = -2
LAMP_ERR_HIP = -3
LAMP_ERR_NOMEM = -4
LAMP_STATS_LEN = 10

_lib = None


class LampError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"lamp error {code}: {msg}")
        self.code = code


def load():
    """Load liblamp.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def load_library(path):
    """A ctypes handle on a built copy of the library at `path` (liblamp.so,
    or the test build liblamp_sync.so), with the entry points' signatures set;
    raises if the file is missing."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m mixed_precision_attention_lamp_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64
    lib.lamp_attn_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, f32, vp]
    lib.lamp_attn_fwd.restype = i32
    lib.lamp_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, f32, vp]
    lib.lamp_attn_fwd_noalloc.restype = i32
    lib.lamp_attn_fwd_logit8.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, f32, vp]
    lib.lamp_attn_fwd_logit8.restype = i32
    lib.lamp_attn_fwd_exp2poly.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, f32, vp]
    lib.lamp_attn_fwd_exp2poly.restype = i32
    lib.lamp_attn_fwd_bf16.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.lamp_attn_decode.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, f32,
                                     i32, vp]
    lib.lamp_attn_decode.restype = i32
    lib.lamp_attn_decode_with_amax.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32,
                                               f32, i32, vp, vp]
    lib.lamp_attn_decode_with_amax.restype = i32
    lib.lamp_kv_amax_update.argtypes = [vp, i32, i32, i32, i32, vp]
    lib.lamp_kv_amax_update.restype = i32
    lib.lamp_decode_tiles_per_split.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.lamp_decode_tiles_per_split.restype = i32
    lib.lamp_attn_fwd_bf16.restype = i32
    lib.lamp_debug_attn_dump.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, f32,
                                         vp, vp, vp]
    lib.lamp_debug_attn_dump.restype = i32
    lib.lamp_debug_attn_dump_logit8.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                                f32, vp, vp, vp]
    lib.lamp_debug_attn_dump_logit8.restype = i32
    lib.lamp_debug_attn_dump_exp2poly.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                                  f32, vp, vp, vp]
    lib.lamp_debug_attn_dump_exp2poly.restype = i32
    lib.lamp_debug_exp2poly.argtypes = [vp, i64, vp]
    lib.lamp_debug_exp2poly.restype = i32
    lib.lamp_subblock_stats.argtypes = [vp, i32, i32, i32, i32, i32, vp]
    lib.lamp_subblock_stats.restype = i32
    lib.lamp_quantize_qk.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.lamp_quantize_qk.restype = i32
    lib.lamp_debug_fp8_dot.argtypes = [vp, vp, vp, i32]
    lib.lamp_debug_fp8_dot.restype = i32
    lib.lamp_debug_convert.argtypes = [vp, i64, vp, vp, vp, vp]
    lib.lamp_debug_convert.restype = i32
    lib.lamp_set_timing.argtypes = [i32]
    lib.lamp_set_timing.restype = i32
    lib.lamp_read_timing.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int)]
    lib.lamp_read_timing.restype = i32
    lib.lamp_set_stream.argtypes = [vp]
    lib.lamp_set_stream.restype = i32
    lib.lamp_last_error.argtypes = []
    lib.lamp_last_error.restype = ctypes.c_char_p
    lib.lamp_release_workspace.argtypes = []
    lib.lamp_release_workspace.restype = None
    lib.lamp_version.argtypes = []
    lib.lamp_version.restype = i32
    return lib


def declared_symbols():
    """Names of the functions include/lamp.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(lamp_\w+)\s*\(", text, re.M)))


def _check(rc):
    if rc != LAMP_OK:
        raise LampError(rc, load().lamp_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _invalid(msg):
    raise LampError(LAMP_ERR_INVALID, msg)


def _expect(t, name, dtypes, shape, device=None):
    """Check one tensor argument before its pointer reaches the library:
    dtype, shape and contiguity.  ``dtypes`` is a torch dtype or a tuple of
    them; ``shape`` a tuple of ints.  The device is checked by _on_gpu once
    every argument has passed these checks."""
    import torch
    if t is None:
        _invalid(f"{name} must not be None")
    if not isinstance(t, torch.Tensor):
        _invalid(f"{name} must be a torch tensor (got {type(t).__name__})")
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        _invalid(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        _invalid(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        _invalid(f"{name} must be contiguous")


def _on_gpu(named):
    """Every (name, tensor) pair (None tensors skipped) on the first one's GPU."""
    named = [(n, t) for n, t in named if t is not None]
    n0, t0 = named[0]
    if t0.device.type != "cuda":
        _invalid(f"{n0} must be on a GPU (got {t0.device})")
    for n, t in named[1:]:
        if t.device != t0.device:
            _invalid(f"{n} must be on {t0.device} (got {t.device})")


def _attn_shapes(q, k, v):
    """(B, Hq, Hkv, S, D) of a forward call, after checking q, k and v."""
    import torch
    if q is None or not isinstance(q, torch.Tensor) or q.dim() != 4:
        _invalid("q must be a 4-d tensor [B, Hq, S, D]")
    B, Hq, S, D = q.shape
    if k is None or not isinstance(k, torch.Tensor) or k.dim() != 4:
        _invalid("k must be a 4-d tensor [B, Hkv, S, D]")
    Hkv = k.shape[1]
    _expect(q, "q", torch.bfloat16, (B, Hq, S, D))
    _expect(k, "k", torch.bfloat16, (B, Hkv, S, D))
    _expect(v, "v", torch.bfloat16, (B, Hkv, S, D))
    if Hkv < 1 or Hq % Hkv != 0:
        _invalid(f"Hq ({Hq}) must be a multiple of Hkv ({Hkv})")
    return B, Hq, Hkv, S, D


def _n_tiles(S):
    return (S + 63) // 64


def _check_fwd_outputs(q, k, v, out, mask, B, Hq, S, D, extra=()):
    """Outputs of a forward call, then the devices of every argument."""
    import torch
    _expect(out, "out", torch.float32, (B, Hq, S, D))
    if mask is not None:
        nT = _n_tiles(S)
        _expect(mask, "subblock_mask_out", torch.uint8, (B, Hq, nT, nT))
    _on_gpu([("q", q), ("k", k), ("v", v), ("out", out), ("subblock_mask_out", mask), *extra])


def _sync_stream(lib):
    import torch
    lib.lamp_set_stream(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def lamp_version():
    return load().lamp_version()


def lamp_last_error():
    return load().lamp_last_error().decode()


def lamp_release_workspace():
    load().lamp_release_workspace()


def lamp_set_stream(stream):
    """stream: a torch.cuda.Stream (or None for the default stream)."""
    _check(load().lamp_set_stream(None if stream is None else ctypes.c_void_p(stream.cuda_stream)))


def lamp_set_timing(enable):
    _check(load().lamp_set_timing(int(enable)))


def lamp_read_timing():
    """(prep_ms_total, attn_ms_total, n_calls) since the last read."""
    a, b, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int()
    _check(load().lamp_read_timing(ctypes.byref(a), ctypes.byref(b), ctypes.byref(n)))
    return a.value, b.value, n.value


def lamp_attn_fwd(q, k, v, out, causal=1, window=0, delta=2.0 ** -8, tau=2.0 ** -1,
                  subblock_mask_out=None):
    """q [B,Hq,S,D], k/v [B,Hkv,S,D] bf16; out [B,Hq,S,D] fp32; optional uint8 mask."""
    lib = load()
    B, Hq, Hkv, S, D = _attn_shapes(q, k, v)
    _check_fwd_outputs(q, k, v, out, subblock_mask_out, B, Hq, S, D)
    _sync_stream(lib)
    _check(lib.lamp_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, S, D,
                             int(causal), int(window), float(delta), float(tau),
                             _ptr(subblock_mask_out)))


def lamp_attn_fwd_noalloc(q, k, v, out, causal=1, window=0, delta=2.0 ** -8, tau=2.0 ** -1,
                          subblock_mask_out=None):
    """lamp_attn_fwd on the library's fixed scratch array (allocates nothing);
    arguments as lamp_attn_fwd."""
    lib = load()
    B, Hq, Hkv, S, D = _attn_shapes(q, k, v)
    _check_fwd_outputs(q, k, v, out, subblock_mask_out, B, Hq, S, D)
    _sync_stream(lib)
    _check(lib.lamp_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, S, D,
                                     int(causal), int(window), float(delta), float(tau),
                                     _ptr(subblock_mask_out)))


def lamp_attn_fwd_logit8(q, k, v, out, causal=1, window=0, delta=2.0 ** -8, tau=2.0 ** -1,
                         subblock_mask_out=None):
    """The variant with e4m3 logits; arguments as lamp_attn_fwd."""
    lib = load()
    B, Hq, Hkv, S, D = _attn_shapes(q, k, v)
    _check_fwd_outputs(q, k, v, out, subblock_mask_out, B, Hq, S, D)
    _sync_stream(lib)
    _check(lib.lamp_attn_fwd_logit8(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, S, D,
                                    int(causal), int(window), float(delta), float(tau),
                                    _ptr(subblock_mask_out)))


def lamp_attn_fwd_exp2poly(q, k, v, out, causal=1, window=0, delta=2.0 ** -8, tau=2.0 ** -1,
                           subblock_mask_out=None):
    """The variant with the polynomial exp2 for the 8-bit exponentials;
    arguments as lamp_attn_fwd."""
    lib = load()
    B, Hq, Hkv, S, D = _attn_shapes(q, k, v)
    _check_fwd_outputs(q, k, v, out, subblock_mask_out, B, Hq, S, D)
    _sync_stream(lib)
    _check(lib.lamp_attn_fwd_exp2poly(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, S, D,
                                      int(causal), int(window), float(delta), float(tau),
                                      _ptr(subblock_mask_out)))


def lamp_attn_decode(q, k, v, out, causal=1, window=0, delta=2.0 ** -8, tau=2.0 ** -1,
                     tiles_per_split=0, subblock_mask_out=None):
    """q [B,Hq,Sq,D] (the last Sq positions), k/v [B,Hkv,Skv,D] bf16; out
    [B,Hq,Sq,D] fp32; optional uint8 mask [B,Hq,ceil(Skv/64)]."""
    import torch
    lib = load()
    if q is None or not isinstance(q, torch.Tensor) or q.dim() != 4:
        _invalid("q must be a 4-d tensor [B, Hq, Sq, D]")
    if k is None or not isinstance(k, torch.Tensor) or k.dim() != 4:
        _invalid("k must be a 4-d tensor [B, Hkv, Skv, D]")
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    _expect(q, "q", torch.bfloat16, (B, Hq, Sq, D))
    _expect(k, "k", torch.bfloat16, (B, Hkv, Skv, D))
    _expect(v, "v", torch.bfloat16, (B, Hkv, Skv, D))
    if Hkv < 1 or Hq % Hkv != 0:
        _invalid(f"Hq ({Hq}) must be a multiple of Hkv ({Hkv})")
    _expect(out, "out", torch.float32, (B, Hq, Sq, D))
    if subblock_mask_out is not None:
        _expect(subblock_mask_out, "subblock_mask_out", torch.uint8, (B, Hq, _n_tiles(Skv)))
    _on_gpu([("q", q), ("k", k), ("v", v), ("out", out), ("subblock_mask_out", subblock_mask_out)])
    _sync_stream(lib)
    _check(lib.lamp_attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, Sq, Skv, D,
                                int(causal), int(window), float(delta), float(tau),
                                int(tiles_per_split), _ptr(subblock_mask_out)))


def lamp_attn_decode_with_amax(q, k, v, out, k_amax_state, causal=1, window=0, delta=2.0 ** -8,
                               tau=2.0 ** -1, tiles_per_split=0, subblock_mask_out=None):
    """lamp_attn_decode with the K scales from kept maxima: k_amax_state is an
    int32 (uint32 bits) device tensor [B, Hkv] as lamp_kv_amax_update leaves it."""
    import torch
    lib = load()
    if q is None or not isinstance(q, torch.Tensor) or q.dim() != 4:
        _invalid("q must be a 4-d tensor [B, Hq, Sq, D]")
    if k is None or not isinstance(k, torch.Tensor) or k.dim() != 4:
        _invalid("k must be a 4-d tensor [B, Hkv, Skv, D]")
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    _expect(q, "q", torch.bfloat16, (B, Hq, Sq, D))
    _expect(k, "k", torch.bfloat16, (B, Hkv, Skv, D))
    _expect(v, "v", torch.bfloat16, (B, Hkv, Skv, D))
    if Hkv < 1 or Hq % Hkv != 0:
        _invalid(f"Hq ({Hq}) must be a multiple of Hkv ({Hkv})")
    _expect(out, "out", torch.float32, (B, Hq, Sq, D))
    _expect(k_amax_state, "k_amax_state", torch.int32, (B, Hkv))
    if subblock_mask_out is not None:
        _expect(subblock_mask_out, "subblock_mask_out", torch.uint8, (B, Hq, _n_tiles(Skv)))
    _on_gpu([("q", q), ("k", k), ("v", v), ("out", out), ("k_amax_state", k_amax_state),
             ("subblock_mask_out", subblock_mask_out)])
    _sync_stream(lib)
    _check(lib.lamp_attn_decode_with_amax(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, Sq, Skv, D,
                                          int(causal), int(window), float(delta), float(tau),
                                          int(tiles_per_split), _ptr(k_amax_state), _ptr(subblock_mask_out)))


def lamp_kv_amax_update(k_new, k_amax_state):
    """Fold new keys k_new [B, Hkv, S_new, D] (bf16) into the kept maxima
    k_amax_state [B, Hkv] (int32 device tensor holding uint32 bits)."""
    import torch
    lib = load()
    if k_new is None or not isinstance(k_new, torch.Tensor) or k_new.dim() != 4:
        _invalid("k_new must be a 4-d tensor [B, Hkv, S_new, D]")
    B, Hkv, S_new, D = k_new.shape
    _expect(k_new, "k_new", torch.bfloat16, (B, Hkv, S_new, D))
    _expect(k_amax_state, "k_amax_state", torch.int32, (B, Hkv))
    _on_gpu([("k_new", k_new), ("k_amax_state", k_amax_state)])
    _sync_stream(lib)
    _check(lib.lamp_kv_amax_update(_ptr(k_new), B, Hkv, S_new, D, _ptr(k_amax_state)))


def lamp_decode_tiles_per_split(B, Hq, Hkv, Sq, Skv, D):
    rc = load().lamp_decode_tiles_per_split(B, Hq, Hkv, Sq, Skv, D)
    _check(min(rc, 0))
    return rc


def lamp_attn_fwd_bf16(q, k, v, out, causal=1, window=0, subblock_mask_out=None):
    """The plain bf16 FlashAttention baseline; arguments as lamp_attn_fwd."""
    lib = load()
    B, Hq, Hkv, S, D = _attn_shapes(q, k, v)
    _check_fwd_outputs(q, k, v, out, subblock_mask_out, B, Hq, S, D)
    _sync_stream(lib)
    _check(lib.lamp_attn_fwd_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, S, D,
                                  int(causal), int(window), _ptr(subblock_mask_out)))


def lamp_debug_attn_dump(q, k, v, out, causal, window, delta, tau, subblock_mask_out,
                         acc8_out, p_out):
    import torch
    lib = load()
    B, Hq, Hkv, S, D = _attn_shapes(q, k, v)
    _expect(acc8_out, "acc8_out", torch.float32, (B, Hq, S, S))
    _expect(p_out, "p_out", (torch.int16, torch.bfloat16), (B, Hq, S, S))
    _check_fwd_outputs(q, k, v, out, subblock_mask_out, B, Hq, S, D, (("acc8_out", acc8_out), ("p_out", p_out)))
    _sync_stream(lib)
    _check(lib.lamp_debug_attn_dump(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, S, D,
                                    int(causal), int(window), float(delta), float(tau),
                                    _ptr(subblock_mask_out), _ptr(acc8_out), _ptr(p_out)))


def lamp_debug_attn_dump_logit8(q, k, v, out, causal, window, delta, tau, subblock_mask_out,
                                logit8_out, p_out):
    import torch
    lib = load()
    B, Hq, Hkv, S, D = _attn_shapes(q, k, v)
    _expect(logit8_out, "logit8_out", torch.float32, (B, Hq, S, S))
    _expect(p_out, "p_out", (torch.int16, torch.bfloat16), (B, Hq, S, S))
    _check_fwd_outputs(q, k, v, out, subblock_mask_out, B, Hq, S, D, (("logit8_out", logit8_out), ("p_out", p_out)))
    _sync_stream(lib)
    _check(lib.lamp_debug_attn_dump_logit8(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, S, D,
                                           int(causal), int(window), float(delta), float(tau),
                                           _ptr(subblock_mask_out), _ptr(logit8_out), _ptr(p_out)))


def lamp_debug_attn_dump_exp2poly(q, k, v, out, causal, window, delta, tau, subblock_mask_out,
                                  acc8_out, p_out):
    import torch
    lib = load()
    B, Hq, Hkv, S, D = _attn_shapes(q, k, v)
    _expect(acc8_out, "acc8_out", torch.float32, (B, Hq, S, S))
    _expect(p_out, "p_out", (torch.int16, torch.bfloat16), (B, Hq, S, S))
    _check_fwd_outputs(q, k, v, out, subblock_mask_out, B, Hq, S, D, (("acc8_out", acc8_out), ("p_out", p_out)))
    _sync_stream(lib)
    _check(lib.lamp_debug_attn_dump_exp2poly(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, S, D,
                                             int(causal), int(window), float(delta), float(tau),
                                             _ptr(subblock_mask_out), _ptr(acc8_out), _ptr(p_out)))


def lamp_subblock_stats(subblock_mask, B, Hq, S, causal, window, stats_out):
    import torch
    lib = load()
    nT = _n_tiles(S)
    _expect(subblock_mask, "subblock_mask", torch.uint8, (B, Hq, nT, nT))
    _expect(stats_out, "stats_out", torch.int64, (LAMP_STATS_LEN,))
    _on_gpu([("subblock_mask", subblock_mask), ("stats_out", stats_out)])
    _sync_stream(lib)
    _check(lib.lamp_subblock_stats(_ptr(subblock_mask), B, Hq, S, int(causal), int(window),
                                   _ptr(stats_out)))


def lamp_quantize_qk(q, k, q8, k8, q_scale, k_scale):
    import torch
    lib = load()
    if q is None or not isinstance(q, torch.Tensor) or q.dim() != 4:
        _invalid("q must be a 4-d tensor [B, Hq, S, D]")
    if k is None or not isinstance(k, torch.Tensor) or k.dim() != 4:
        _invalid("k must be a 4-d tensor [B, Hkv, S, D]")
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    _expect(q, "q", torch.bfloat16, (B, Hq, S, D))
    _expect(k, "k", torch.bfloat16, (B, Hkv, S, D))
    _expect(q8, "q8", torch.uint8, (B, Hq, S, D))
    _expect(k8, "k8", torch.uint8, (B, Hkv, S, D))
    _expect(q_scale, "q_scale", torch.float32, (B * Hq,))
    _expect(k_scale, "k_scale", torch.float32, (B * Hkv,))
    _on_gpu([("q", q), ("k", k), ("q8", q8), ("k8", k8), ("q_scale", q_scale), ("k_scale", k_scale)])
    _sync_stream(lib)
    _check(lib.lamp_quantize_qk(_ptr(q), _ptr(k), B, Hq, Hkv, S, D, _ptr(q8), _ptr(k8),
                                _ptr(q_scale), _ptr(k_scale)))


def lamp_debug_convert(x, e4m3=None, e4m3_bf16=None, bf16=None, exp2=None):
    import torch
    lib = load()
    if x is None or not isinstance(x, torch.Tensor):
        _invalid("x must be a torch tensor")
    n = x.numel()
    _expect(x, "x", torch.float32, (n,))
    for t, name, dt in ((e4m3, "e4m3", torch.uint8), (e4m3_bf16, "e4m3_bf16", (torch.int16, torch.bfloat16)),
                        (bf16, "bf16", (torch.int16, torch.bfloat16)), (exp2, "exp2", torch.float32)):
        if t is not None:
            _expect(t, name, dt, (n,))
    _on_gpu([("x", x), ("e4m3", e4m3), ("e4m3_bf16", e4m3_bf16), ("bf16", bf16), ("exp2", exp2)])
    _sync_stream(lib)
    _check(lib.lamp_debug_convert(_ptr(x), x.numel(), _ptr(e4m3), _ptr(e4m3_bf16), _ptr(bf16),
                                  _ptr(exp2)))


def lamp_debug_exp2poly(x, y):
    """y[i] = the polynomial exp2 of lamp_attn_fwd_exp2poly at x[i] (fp32, same length)."""
    import torch
    lib = load()
    if x is None or not isinstance(x, torch.Tensor):
        _invalid("x must be a torch tensor")
    n = x.numel()
    _expect(x, "x", torch.float32, (n,))
    _expect(y, "y", torch.float32, (n,))
    _on_gpu([("x", x), ("y", y)])
    _sync_stream(lib)
    _check(lib.lamp_debug_exp2poly(_ptr(x), n, _ptr(y)))


def lamp_debug_fp8_dot(a, b, out):
    """a, b uint8 [n, 16, 128] e4m3 codes; out fp32 [n, 16, 16] = a . b^T per block."""
    import torch
    lib = load()
    if a is None or not isinstance(a, torch.Tensor) or a.dim() != 3:
        _invalid("a must be a 3-d tensor [n, 16, 128]")
    n = a.shape[0]
    _expect(a, "a", torch.uint8, (n, 16, 128))
    _expect(b, "b", torch.uint8, (n, 16, 128))
    _expect(out, "out", torch.float32, (n, 16, 16))
    _on_gpu([("a", a), ("b", b), ("out", out)])
    _sync_stream(lib)
    _check(lib.lamp_debug_fp8_dot(_ptr(a), _ptr(b), _ptr(out), n))
