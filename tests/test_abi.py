"""The C ABI library loads, exports what include/lamp.h declares, and rejects
bad arguments before touching HIP.  No GPU and no compute call."""
import ctypes
import math
import subprocess

import pytest
import torch

import mixed_precision_attention_lamp_amd as lamp
from mixed_precision_attention_lamp_amd import _lib

ALIGNED = 1 << 20          # any 16-byte aligned non-null address: never dereferenced


@pytest.fixture(scope="module")
def lib():
    return lamp.load()


def test_exports_every_declared_symbol(lib):
    names = lamp.declared_symbols()
    assert {"lamp_attn_fwd", "lamp_subblock_stats", "lamp_quantize_qk", "lamp_set_stream",
            "lamp_last_error", "lamp_release_workspace", "lamp_version",
            "lamp_debug_convert", "lamp_set_timing", "lamp_read_timing",
            "lamp_debug_attn_dump", "lamp_attn_fwd_bf16", "lamp_attn_fwd_logit8",
            "lamp_debug_attn_dump_logit8", "lamp_attn_fwd_exp2poly", "lamp_debug_attn_dump_exp2poly",
            "lamp_debug_exp2poly"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_version(lib):
    assert lib.lamp_version() == 100


def _fwd(lib, **kw):
    args = dict(q=ALIGNED, k=ALIGNED, v=ALIGNED, out=ALIGNED, B=1, Hq=2, Hkv=1, S=128, D=128,
                causal=1, window=0, delta=2.0 ** -8, tau=0.5, mask=None)
    args.update(kw)
    return lib.lamp_attn_fwd(args["q"], args["k"], args["v"], args["out"], args["B"], args["Hq"],
                             args["Hkv"], args["S"], args["D"], args["causal"], args["window"],
                             args["delta"], args["tau"], args["mask"])


@pytest.mark.parametrize("kw,code,text", [
    (dict(q=None), -1, "non-null"),
    (dict(out=None), -1, "non-null"),
    (dict(k=ALIGNED + 2), -1, "aligned"),
    (dict(B=0), -1, ">= 1"),
    (dict(S=-5), -1, ">= 1"),
    (dict(Hq=3, Hkv=2), -1, "multiple"),
    (dict(D=96), -2, "D=96"),
    (dict(D=512), -2, "D=512"),
    (dict(causal=2), -1, "causal"),
    (dict(window=-1), -1, "window"),
    (dict(window=16, causal=0), -1, "window"),
    (dict(delta=math.nan), -1, "NaN"),
    (dict(tau=math.nan), -1, "NaN"),
    (dict(Hq=1, Hkv=1, S=1 << 23, D=128), -2, "2^30"),        # one head: S*D = 2^30
    (dict(B=1 << 20, Hq=512, Hkv=1, S=64, D=64), -2, "2^29"),  # launch grid
])
def test_attn_validation(lib, kw, code, text):
    assert _fwd(lib, **kw) == code
    assert text in lamp.lamp_last_error()


def test_other_entry_points_validate(lib):
    assert lib.lamp_quantize_qk(None, ALIGNED, 1, 1, 1, 64, 64, ALIGNED, ALIGNED, ALIGNED, ALIGNED) == -1
    # the quantisation export's maxima pass: one grid row per (batch, head), at most 65535
    assert lib.lamp_quantize_qk(ALIGNED, ALIGNED, 1000, 64, 8, 64, 64, ALIGNED, ALIGNED, ALIGNED, ALIGNED) == -2
    assert "65535" in lamp.lamp_last_error()
    assert lib.lamp_subblock_stats(None, 1, 1, 64, 1, 0, ALIGNED) == -1
    assert lib.lamp_subblock_stats(ALIGNED, 1, 1, 64, 0, 8, ALIGNED) == -1
    assert lib.lamp_debug_convert(None, 10, None, None, None, None) == -1
    # kept K maxima: null or misaligned state, bad sizes (before any HIP call)
    assert lib.lamp_kv_amax_update(ALIGNED, 1, 1, 64, 128, None) == -1
    assert lib.lamp_kv_amax_update(ALIGNED, 1, 1, 64, 128, ALIGNED + 2) == -1
    assert lib.lamp_kv_amax_update(ALIGNED + 2, 1, 1, 64, 128, ALIGNED) == -1
    assert lib.lamp_kv_amax_update(ALIGNED, 0, 1, 64, 128, ALIGNED) == -1
    assert lib.lamp_kv_amax_update(ALIGNED, 1, 1, 64, 96, ALIGNED) == -2
    assert lib.lamp_kv_amax_update(ALIGNED, 1, 1, 1 << 23, 128, ALIGNED) == -2
    assert lib.lamp_kv_amax_update(ALIGNED, 300, 300, 64, 128, ALIGNED) == -2
    assert lib.lamp_attn_decode_with_amax(ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1, 4, 1, 8, 100, 128, 1, 0,
                                          2.0 ** -8, 0.5, 0, None, None) == -1
    assert lib.lamp_attn_decode_with_amax(ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1, 4, 1, 17, 100, 128, 1, 0,
                                          2.0 ** -8, 0.5, 0, ALIGNED, None) == -2
    assert lib.lamp_debug_convert(None, 0, None, None, None, None) == 0
    assert lib.lamp_set_stream(None) == 0


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device error path")
def test_valid_call_without_device_reports_hip_error(lib):
    assert _fwd(lib) == -3
    assert "hip" in lamp.lamp_last_error().lower()


def test_binding_raises_on_error():
    class Fake:
        shape = (1, 1, 64, 96)

        def data_ptr(self):
            return ALIGNED
    with pytest.raises(lamp.LampError) as ei:
        lamp.lamp_attn_fwd.__wrapped__ if hasattr(lamp.lamp_attn_fwd, "__wrapped__") else None
        _lib._check(_fwd(lamp.load(), D=96))
    assert ei.value.code == -2


def test_bf16_baseline_rejects_before_hip(lib):
    # bad sizes are rejected as for lamp_attn_fwd, before any HIP call
    assert lib.lamp_attn_fwd_bf16(ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1, 2, 1, 128, 96, 1, 0, None) == -2
    assert "D=96" in lib.lamp_last_error().decode()
    assert lib.lamp_attn_fwd_bf16(ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1, 3, 2, 128, 128, 1, 0, None) == -1


def test_logit8_variant_rejects_before_hip(lib):
    # the 8-bit-logit variant validates its arguments as lamp_attn_fwd does
    f = lib.lamp_attn_fwd_logit8
    assert f(ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1, 2, 1, 128, 96, 1, 0, 0.0039, 0.5, None) == -2
    assert f(ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1, 2, 1, 128, 128, 1, 0, math.nan, 0.5, None) == -1
    assert "NaN" in lamp.lamp_last_error()
    assert f(None, ALIGNED, ALIGNED, ALIGNED, 1, 2, 1, 128, 128, 1, 0, 0.0039, 0.5, None) == -1
    d = lib.lamp_debug_attn_dump_logit8
    assert d(ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1, 1, 1, 64, 64, 1, 0, 0.0, 0.5, None, None, ALIGNED) == -1
    assert d(ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1, 1, 1, 4096, 64, 1, 0, 0.0, 0.5, None, ALIGNED,
             ALIGNED) == -2


def test_exp2poly_variant_rejects_before_hip(lib):
    # the bit-reproducible variant validates its arguments as lamp_attn_fwd does
    f = lib.lamp_attn_fwd_exp2poly
    assert f(ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1, 2, 1, 128, 96, 1, 0, 0.0039, 0.5, None) == -2
    assert f(ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1, 2, 1, 128, 128, 1, 0, 0.0039, math.nan, None) == -1
    assert f(ALIGNED, None, ALIGNED, ALIGNED, 1, 2, 1, 128, 128, 1, 0, 0.0039, 0.5, None) == -1
    d = lib.lamp_debug_attn_dump_exp2poly
    assert d(ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1, 1, 1, 4096, 64, 1, 0, 0.0, 0.5, None, ALIGNED,
             ALIGNED) == -2
    e = lib.lamp_debug_exp2poly
    assert e(ALIGNED, -1, ALIGNED) == -1
    assert e(None, 4, ALIGNED) == -1
    assert e(None, 0, None) == 0


def test_decode_rejects_before_hip(lib):
    f = lib.lamp_attn_decode
    A = ALIGNED
    # Sq > 16, Sq > Skv, G > 8, D = 96: unsupported or invalid, nothing launched
    assert f(A, A, A, A, 1, 2, 1, 17, 64, 128, 1, 0, 0.0039, 0.5, 0, None) == -2
    assert "Sq <= 16" in lamp.lamp_last_error()
    assert f(A, A, A, A, 1, 2, 1, 8, 4, 128, 1, 0, 0.0039, 0.5, 0, None) == -1
    assert f(A, A, A, A, 1, 16, 1, 8, 64, 128, 1, 0, 0.0039, 0.5, 0, None) == -2
    assert f(A, A, A, A, 1, 2, 1, 8, 64, 96, 1, 0, 0.0039, 0.5, 0, None) == -2
    assert f(A, A, A, A, 1, 2, 1, 8, 64, 128, 0, 8, 0.0039, 0.5, 0, None) == -1
    assert f(A, A, A, A, 1, 2, 1, 8, 64, 128, 1, 0, math.nan, 0.5, 0, None) == -1
    assert f(A, A, A, A, 1, 2, 1, 8, 64, 128, 1, 0, 0.0039, 0.5, -1, None) == -1
    assert f(None, A, A, A, 1, 2, 1, 8, 64, 128, 1, 0, 0.0039, 0.5, 0, None) == -1
    # a split of more than 8192 tiles (Skv = 1M keys in one split)
    assert f(A, A, A, A, 1, 2, 1, 8, 1 << 20, 64, 1, 0, 0.0039, 0.5, 9000, None) == -2
    assert "tiles_per_split" in lamp.lamp_last_error()
    assert lib.lamp_decode_tiles_per_split(1, 2, 1, 17, 64, 128) == -2


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the default compute-unit count")
def test_decode_split_choice_without_device(lib):
    # 256 compute units assumed: 512 four-wave workgroups; 64 (batch, kv head)
    # units of 256 tiles give 8 splits of 32 tiles; G = 8 takes eight-wave
    # workgroups, 256 of them; few tiles give 1 per split
    assert lib.lamp_decode_tiles_per_split(8, 32, 8, 16, 16384, 128) == 32
    assert lib.lamp_decode_tiles_per_split(8, 64, 8, 16, 16384, 128) == 64
    assert lib.lamp_decode_tiles_per_split(1, 4, 1, 1, 300, 64) == 1
    assert lib.lamp_decode_tiles_per_split(64, 64, 16, 16, 4096, 128) == 64
    # one unit (G = 8: eight-wave workgroups) and 1M keys: 256 splits of 64 tiles
    assert lib.lamp_decode_tiles_per_split(1, 8, 1, 16, 1 << 20, 128) == 64
