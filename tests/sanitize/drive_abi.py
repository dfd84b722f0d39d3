"""Drives every entry point of a sanitized liblamp build through ctypes.

Run in a child process with the sanitizer runtime preloaded (see
tests/test_sanitized_host.py).  Host buffers stand in for device pointers:
the host has no GPU, so calls that pass validation end in a HIP error code.
Any sanitizer report aborts the process with a non-zero exit code.
"""
import ctypes as C
import math
import sys

lib = C.CDLL(sys.argv[1])
VP, F, I, I64 = C.c_void_p, C.c_float, C.c_int, C.c_int64
CODES = {0, -1, -2, -3, -4}
INT_MAX = 2 ** 31 - 1

lib.lamp_last_error.restype = C.c_char_p
buf = C.create_string_buffer(1 << 20)
b0 = C.addressof(buf)
b0 += (-b0) % 256                      # 256-byte aligned host address
mis = b0 + 2                           # misaligned


def call(name, *args, expect=None):
    fn = getattr(lib, name)
    rc = fn(*args)
    assert rc in CODES, (name, args, rc)
    if expect == "fail":
        assert rc != 0, (name, args)
    if rc != 0:
        msg = lib.lamp_last_error()
        assert msg, (name, "no error message")
    return rc


fwd_names = ["lamp_attn_fwd", "lamp_attn_fwd_noalloc", "lamp_attn_fwd_logit8", "lamp_attn_fwd_exp2poly"]
sizes_bad = [(0, 1, 1, 64, 128), (1, 0, 1, 64, 128), (1, 1, 0, 64, 128), (1, 1, 1, 0, 128),
             (1, 3, 2, 64, 128), (1, 1, 1, 64, 96), (-1, 1, 1, 64, 128), (1, 1, 1, -5, 64),
             (1, 1, 1, INT_MAX, 128), (INT_MAX, INT_MAX, 1, INT_MAX, 256), (1, 8, 1, 1 << 24, 256),
             (65536, 65536, 1, 64, 64)]
for name in fwd_names:
    for (B, Hq, Hkv, S, D) in sizes_bad:
        call(name, VP(b0), VP(b0), VP(b0), VP(b0), I(B), I(Hq), I(Hkv), I(S), I(D), I(1), I(0),
             F(2 ** -8), F(0.5), VP(b0), expect="fail")
    # null and misaligned pointers, bad flags, NaN parameters
    for args in [(None, b0, b0, b0), (b0, None, b0, b0), (b0, b0, None, b0), (b0, b0, b0, None),
                 (mis, b0, b0, b0), (b0, mis, b0, b0), (b0, b0, mis, b0), (b0, b0, b0, mis)]:
        call(name, *[VP(x) for x in args], I(1), I(2), I(1), I(100), I(128), I(1), I(0),
             F(2 ** -8), F(0.5), VP(b0), expect="fail")
    for causal, window, delta, tau in [(2, 0, 2 ** -8, 0.5), (-1, 0, 2 ** -8, 0.5), (0, 16, 2 ** -8, 0.5),
                                       (1, -3, 2 ** -8, 0.5), (1, 0, math.nan, 0.5), (1, 0, 2 ** -8, math.nan)]:
        call(name, VP(b0), VP(b0), VP(b0), VP(b0), I(1), I(2), I(1), I(100), I(128), I(causal), I(window),
             F(delta), F(tau), VP(b0), expect="fail")
    # valid requests: end in a HIP error without a device
    for (B, Hq, Hkv, S, D, causal, window, delta, tau) in [
            (1, 2, 1, 100, 128, 1, 0, 2 ** -8, 0.5), (2, 8, 2, 4096, 64, 0, 0, 0.0, math.inf),
            (1, 4, 4, 1, 256, 1, 64, 2 ** -4, 0.0), (1, 1, 1, 65, 128, 1, 0, math.inf, 2 ** -5)]:
        call(name, VP(b0), VP(b0), VP(b0), VP(b0), I(B), I(Hq), I(Hkv), I(S), I(D), I(causal), I(window),
             F(delta), F(tau), VP(None))

# plain bf16 baseline
for (B, Hq, Hkv, S, D) in sizes_bad + [(1, 2, 1, 100, 256)]:
    call("lamp_attn_fwd_bf16", VP(b0), VP(b0), VP(b0), VP(b0), I(B), I(Hq), I(Hkv), I(S), I(D), I(1), I(0),
         VP(b0), expect="fail")
call("lamp_attn_fwd_bf16", VP(b0), VP(b0), VP(b0), VP(b0), I(1), I(2), I(1), I(100), I(128), I(1), I(0), VP(b0))

# decode
for (B, Hq, Hkv, Sq, Skv, D, tps) in [(1, 4, 1, 0, 100, 128, 0), (1, 4, 1, 17, 100, 128, 0),
                                      (1, 4, 1, 8, 4, 128, 0), (1, 16, 1, 8, 100, 128, 0),
                                      (1, 4, 1, 8, INT_MAX, 128, 0), (1, 4, 1, 8, 100, 128, -2),
                                      (1, 4, 1, 8, 100, 96, 0), (INT_MAX, 4, 1, 8, 100, 128, 0),
                                      (1, 4, 1, 8, 1 << 30, 128, 0)]:
    call("lamp_attn_decode", VP(b0), VP(b0), VP(b0), VP(b0), I(B), I(Hq), I(Hkv), I(Sq), I(Skv), I(D),
         I(1), I(0), F(2 ** -8), F(0.5), I(tps), VP(b0), expect="fail")
call("lamp_attn_decode", VP(b0), VP(b0), VP(b0), VP(b0), I(2), I(8), I(2), I(16), I(3000), I(128),
     I(1), I(0), F(2 ** -8), F(0.5), I(0), VP(b0))
for args in [(1, 4, 1, 16, 16384, 128), (0, 4, 1, 16, 100, 128), (1, 4, 1, 16, INT_MAX, 128),
             (INT_MAX, INT_MAX, 1, 16, INT_MAX, 256)]:
    lib.lamp_decode_tiles_per_split(*[I(x) for x in args])

# kept K maxima and decode with them
for (B, Hkv, S, D) in [(0, 1, 64, 128), (1, 0, 64, 128), (1, 1, 0, 128), (1, 1, 64, 96), (1, 1, INT_MAX, 128),
                       (INT_MAX, INT_MAX, 64, 128), (300, 300, 64, 128)]:
    call("lamp_kv_amax_update", VP(b0), I(B), I(Hkv), I(S), I(D), VP(b0), expect="fail")
call("lamp_kv_amax_update", VP(None), I(1), I(1), I(64), I(128), VP(b0), expect="fail")
call("lamp_kv_amax_update", VP(b0), I(1), I(1), I(64), I(128), VP(b0 + 2), expect="fail")
call("lamp_kv_amax_update", VP(b0), I(2), I(4), I(100), I(128), VP(b0))
for state in [None, b0 + 2]:
    call("lamp_attn_decode_with_amax", VP(b0), VP(b0), VP(b0), VP(b0), I(1), I(4), I(1), I(8), I(100), I(128),
         I(1), I(0), F(2 ** -8), F(0.5), I(0), VP(state), VP(b0), expect="fail")
call("lamp_attn_decode_with_amax", VP(b0), VP(b0), VP(b0), VP(b0), I(1), I(4), I(1), I(17), I(100), I(128),
     I(1), I(0), F(2 ** -8), F(0.5), I(0), VP(b0), VP(b0), expect="fail")
call("lamp_attn_decode_with_amax", VP(b0), VP(b0), VP(b0), VP(b0), I(2), I(8), I(2), I(16), I(3000), I(128),
     I(1), I(0), F(2 ** -8), F(0.5), I(0), VP(b0), VP(b0))

# statistics, quantisation, hooks
for (B, Hq, S) in [(0, 1, 64), (1, 1, 0), (1, 1, INT_MAX), (INT_MAX, INT_MAX, 64)]:
    call("lamp_subblock_stats", VP(b0), I(B), I(Hq), I(S), I(1), I(0), VP(b0), expect="fail")
call("lamp_subblock_stats", VP(None), I(1), I(1), I(64), I(1), I(0), VP(b0), expect="fail")
call("lamp_subblock_stats", VP(b0), I(1), I(2), I(128), I(1), I(0), VP(b0))
for (B, Hq, Hkv, S, D) in sizes_bad:
    call("lamp_quantize_qk", VP(b0), VP(b0), I(B), I(Hq), I(Hkv), I(S), I(D), VP(b0), VP(b0), VP(b0), VP(b0),
         expect="fail")
call("lamp_quantize_qk", VP(b0), VP(b0), I(1), I(2), I(1), I(64), I(128), VP(b0), VP(b0), VP(b0), VP(b0))
for n in [-1, 1 << 40]:
    call("lamp_debug_convert", VP(b0), I64(n), VP(b0), VP(b0), VP(b0), VP(b0), expect="fail")
call("lamp_debug_convert", VP(b0), I64(100), VP(b0), VP(b0), VP(b0), VP(b0))
for n in [-1, (1 << 20) + 1]:
    call("lamp_debug_fp8_dot", VP(b0), VP(b0), VP(b0), I(n), expect="fail")
call("lamp_debug_fp8_dot", VP(mis), VP(b0), VP(b0), I(1), expect="fail")
call("lamp_debug_fp8_dot", VP(b0), VP(b0), VP(b0), I(4))
for n in [-1, 1 << 40]:
    call("lamp_debug_exp2poly", VP(b0), I64(n), VP(b0), expect="fail")
call("lamp_debug_exp2poly", VP(None), I64(4), VP(b0), expect="fail")
call("lamp_debug_exp2poly", VP(b0), I64(100), VP(b0))
for name in ["lamp_debug_attn_dump", "lamp_debug_attn_dump_logit8", "lamp_debug_attn_dump_exp2poly"]:
    for S in [0, 4096, INT_MAX]:
        call(name, VP(b0), VP(b0), VP(b0), VP(b0), I(1), I(1), I(1), I(S), I(64), I(1), I(0), F(2 ** -8),
             F(0.5), VP(b0), VP(b0), VP(b0), expect="fail")
    call(name, VP(b0), VP(b0), VP(b0), VP(b0), I(1), I(1), I(1), I(100), I(64), I(1), I(0), F(2 ** -8),
         F(0.5), VP(b0), VP(b0), VP(b0))

# stream, timing, workspace, version
call("lamp_set_timing", I(1))
pm, am, n = C.c_double(), C.c_double(), C.c_int()
call("lamp_read_timing", C.byref(pm), C.byref(am), C.byref(n))
call("lamp_read_timing", None, None, None)
call("lamp_set_timing", I(0))
call("lamp_set_stream", VP(None))
lib.lamp_release_workspace()
assert lib.lamp_version() > 0
print("driven: all entry points")
