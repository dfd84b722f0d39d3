"""The Python binding rejects malformed tensor arguments before any pointer
reaches the library (CPU: nothing here launches a kernel).  A short K/V, a
strided view, a wrong dtype or an undersized output would otherwise make a
kernel read or write out of bounds on the device."""
import pytest
import torch

import mixed_precision_attention_lamp_amd as lamp
from mixed_precision_attention_lamp_amd import LampError
from mixed_precision_attention_lamp_amd._lib import LAMP_ERR_INVALID

B, HQ, HKV, S, D = 1, 4, 2, 70, 64
NT = (S + 63) // 64


def _args(**over):
    a = dict(q=torch.zeros(B, HQ, S, D, dtype=torch.bfloat16),
             k=torch.zeros(B, HKV, S, D, dtype=torch.bfloat16),
             v=torch.zeros(B, HKV, S, D, dtype=torch.bfloat16),
             out=torch.zeros(B, HQ, S, D, dtype=torch.float32),
             subblock_mask_out=torch.zeros(B, HQ, NT, NT, dtype=torch.uint8))
    a.update(over)
    return a


def _rejects(fn, match, **over):
    a = _args(**over)
    with pytest.raises(LampError, match=match) as e:
        fn(a["q"], a["k"], a["v"], a["out"], 1, 0, subblock_mask_out=a["subblock_mask_out"]) \
            if fn is lamp.lamp_attn_fwd_bf16 else \
            fn(a["q"], a["k"], a["v"], a["out"], 1, 0, 2.0 ** -8, 0.5, a["subblock_mask_out"])
    assert e.value.code == LAMP_ERR_INVALID


FWD = [lamp.lamp_attn_fwd, lamp.lamp_attn_fwd_logit8, lamp.lamp_attn_fwd_exp2poly, lamp.lamp_attn_fwd_bf16]


@pytest.mark.parametrize("fn", FWD, ids=lambda f: f.__name__)
def test_forward_rejections(fn):
    _rejects(fn, "q must have dtype", q=torch.zeros(B, HQ, S, D, dtype=torch.float16))
    _rejects(fn, "k must have dtype", k=torch.zeros(B, HKV, S, D, dtype=torch.float32))
    _rejects(fn, "k must have shape", k=torch.zeros(B, HKV, S - 1, D, dtype=torch.bfloat16))
    _rejects(fn, "v must have shape", v=torch.zeros(B, HKV, S, D // 2, dtype=torch.bfloat16))
    _rejects(fn, "v must have shape", v=torch.zeros(B, HKV + 1, S, D, dtype=torch.bfloat16))
    _rejects(fn, "k must be contiguous",
             k=torch.zeros(B, HKV, D, S, dtype=torch.bfloat16).transpose(2, 3))
    _rejects(fn, "multiple of Hkv", k=torch.zeros(B, 3, S, D, dtype=torch.bfloat16),
             v=torch.zeros(B, 3, S, D, dtype=torch.bfloat16))
    _rejects(fn, "out must have dtype", out=torch.zeros(B, HQ, S, D, dtype=torch.bfloat16))
    _rejects(fn, "out must have shape", out=torch.zeros(B, HQ, S - 1, D, dtype=torch.float32))
    _rejects(fn, "subblock_mask_out must have shape",
             subblock_mask_out=torch.zeros(B, HQ, NT, NT - 1, dtype=torch.uint8))
    _rejects(fn, "subblock_mask_out must have dtype",
             subblock_mask_out=torch.zeros(B, HQ, NT, NT, dtype=torch.int8))
    _rejects(fn, "q must be a 4-d", q=torch.zeros(HQ, S, D, dtype=torch.bfloat16))
    # well-formed CPU tensors: rejected for their device, before any launch
    _rejects(fn, "must be on a GPU")


def test_decode_rejections():
    sq, skv = 3, 200
    good = dict(q=torch.zeros(B, HQ, sq, D, dtype=torch.bfloat16),
                k=torch.zeros(B, HKV, skv, D, dtype=torch.bfloat16),
                v=torch.zeros(B, HKV, skv, D, dtype=torch.bfloat16),
                out=torch.zeros(B, HQ, sq, D, dtype=torch.float32),
                mask=torch.zeros(B, HQ, (skv + 63) // 64, dtype=torch.uint8))

    def call(**over):
        a = dict(good, **over)
        lamp.lamp_attn_decode(a["q"], a["k"], a["v"], a["out"], 1, 0, 2.0 ** -8, 0.5, 0, a["mask"])

    for over, match in ((dict(v=torch.zeros(B, HKV, skv - 1, D, dtype=torch.bfloat16)), "v must have shape"),
                        (dict(out=torch.zeros(B, HQ, sq, D, dtype=torch.float16)), "out must have dtype"),
                        (dict(mask=torch.zeros(B, HQ, 3, dtype=torch.uint8)), "subblock_mask_out must have shape"),
                        ({}, "must be on a GPU")):
        with pytest.raises(LampError, match=match):
            call(**over)


def test_dump_stats_quantize_convert_rejections():
    a = _args()
    with pytest.raises(LampError, match="acc8_out must have shape"):
        lamp.lamp_debug_attn_dump(a["q"], a["k"], a["v"], a["out"], 1, 0, 2.0 ** -8, 0.5,
                                  a["subblock_mask_out"], torch.zeros(B, HQ, S, S - 1), torch.zeros(B, HQ, S, S, dtype=torch.int16))
    with pytest.raises(LampError, match="stats_out must have shape"):
        lamp.lamp_subblock_stats(a["subblock_mask_out"], B, HQ, S, 1, 0, torch.zeros(9, dtype=torch.int64))
    with pytest.raises(LampError, match="k8 must have shape"):
        lamp.lamp_quantize_qk(a["q"], a["k"], torch.zeros(B, HQ, S, D, dtype=torch.uint8),
                              torch.zeros(B, HKV, S - 2, D, dtype=torch.uint8),
                              torch.zeros(B * HQ), torch.zeros(B * HKV))
    with pytest.raises(LampError, match="exp2 must have shape"):
        lamp.lamp_debug_convert(torch.zeros(10), exp2=torch.zeros(9))
    with pytest.raises(LampError, match="y must have shape"):
        lamp.lamp_debug_exp2poly(torch.zeros(10), torch.zeros(9))
    with pytest.raises(LampError, match="must be on a GPU"):
        lamp.lamp_debug_exp2poly(torch.zeros(10), torch.zeros(10))
    with pytest.raises(LampError, match="acc8_out must have shape"):
        lamp.lamp_debug_attn_dump_exp2poly(a["q"], a["k"], a["v"], a["out"], 1, 0, 2.0 ** -8, 0.5,
                                           a["subblock_mask_out"], torch.zeros(B, HQ, S, S - 1),
                                           torch.zeros(B, HQ, S, S, dtype=torch.int16))


def test_kept_amax_rejections():
    Sq, Skv = 4, 100
    q = torch.zeros(B, HQ, Sq, D, dtype=torch.bfloat16)
    k = torch.zeros(B, HKV, Skv, D, dtype=torch.bfloat16)
    out = torch.zeros(B, HQ, Sq, D, dtype=torch.float32)
    state = torch.zeros(B, HKV, dtype=torch.int32)

    def rejects(match, fn, *args):
        with pytest.raises(LampError, match=match) as e:
            fn(*args)
        assert e.value.code == LAMP_ERR_INVALID

    rejects("k_amax_state must have dtype", lamp.lamp_attn_decode_with_amax, q, k, k, out,
            torch.zeros(B, HKV, dtype=torch.int64))
    rejects("k_amax_state must have shape", lamp.lamp_attn_decode_with_amax, q, k, k, out,
            torch.zeros(B, HKV + 1, dtype=torch.int32))
    rejects("k_amax_state must not be None", lamp.lamp_attn_decode_with_amax, q, k, k, out, None)
    rejects("v must have shape", lamp.lamp_attn_decode_with_amax, q, k, k[:, :, :50].contiguous(), out, state)
    rejects("must be on a GPU", lamp.lamp_attn_decode_with_amax, q, k, k, out, state)
    rejects("k_new must have dtype", lamp.lamp_kv_amax_update, k.float(), state)
    rejects("k_amax_state must have shape", lamp.lamp_kv_amax_update, k, torch.zeros(B, dtype=torch.int32))
    rejects("k_new must be contiguous", lamp.lamp_kv_amax_update, k.transpose(2, 3).contiguous().transpose(2, 3),
            state)
    rejects("must be on a GPU", lamp.lamp_kv_amax_update, k, state)
