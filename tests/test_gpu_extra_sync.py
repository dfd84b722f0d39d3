"""LDS-race check (needs an MI355X): the test build liblamp_sync.so, in which
every copy into LDS is waited for where it is issued (so each lands up to
two phases earlier than in liblamp.so) and decode's tile stores are fenced
by an extra barrier, must give the outputs and masks of liblamp.so bit for
bit.  A copy that overwrote a slot some wave still reads, or any result that
depended on when a copy lands, would differ.  Cases cover the ping-pong
schedule (paired and unpaired, D = 64 and 128), the D = 256 one-loop
schedule, a sliding window, the plain bf16 and 8-bit-logit modes, the
vector form of the per-entry test, and split-KV decode."""
import ctypes
import os

import numpy as np
import pytest
import torch

from inputs import make_inputs
from parity import say, to_device

pytestmark = pytest.mark.gpu


def _libs():
    import mixed_precision_attention_lamp_amd._lib as L
    sync = os.path.join(os.path.dirname(L.LIB_PATH), "liblamp_sync.so")
    return L.load(), L.load_library(sync)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


FWD = [
    # entry point, B, Hq, Hkv, S, D, causal, window, delta, tau, structure, seed
    ("fwd", 1, 8, 2, 1500, 128, 1, 0, 2 ** -8, 2 ** -1, "channels", 501),      # ping-pong, paired
    ("fwd", 2, 32, 8, 2048, 128, 1, 0, 2 ** -8, 2 ** -1, "channels", 502),     # ping-pong, unpaired
    ("fwd", 1, 4, 4, 1000, 64, 1, 300, 2 ** -4, 2 ** -2, "channels", 503),     # D = 64, window
    ("fwd", 1, 4, 2, 1300, 256, 1, 0, 2 ** -8, 2 ** -1, "channels", 504),      # D = 256 one-loop
    ("fwd", 1, 2, 2, 900, 256, 1, 256, 2 ** -8, 2 ** -1, "sinks", 505),        # D = 256, window
    ("fwd", 1, 8, 2, 1000, 128, 1, 0, 2 ** -8, 2 ** -3, "channels+drift", 506),  # vector per-entry test
    ("bf16", 1, 8, 2, 1000, 128, 1, 0, 0.0, 0.0, "channels", 507),
    ("bf16", 1, 4, 2, 700, 256, 1, 0, 0.0, 0.0, "channels", 508),
    ("logit8", 1, 8, 2, 1000, 128, 1, 0, 2 ** -8, 2 ** -1, "channels", 509),
]


@pytest.mark.parametrize("case", FWD, ids=lambda c: f"{c[0]}-B{c[1]}-Hq{c[2]}-S{c[4]}-D{c[5]}-w{c[7]}")
def test_forward_equal_under_extra_sync(case):
    name, B, Hq, Hkv, S, D, causal, window, delta, tau, st, seed = case
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, st)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    nT = (S + 63) // 64
    res = []
    for lib in _libs():
        out = torch.full((B, Hq, S, D), float("nan"), dtype=torch.float32, device="cuda")
        mask = torch.full((B, Hq, nT, nT), 0x55, dtype=torch.uint8, device="cuda")
        if name == "bf16":
            rc = lib.lamp_attn_fwd_bf16(_p(qd), _p(kd), _p(vd), _p(out), B, Hq, Hkv, S, D, causal, window,
                                        _p(mask))
        else:
            fn = lib.lamp_attn_fwd if name == "fwd" else lib.lamp_attn_fwd_logit8
            rc = fn(_p(qd), _p(kd), _p(vd), _p(out), B, Hq, Hkv, S, D, causal, window, delta, tau, _p(mask))
        assert rc == 0, lib.lamp_last_error()
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), mask.cpu().numpy()))
    same = np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
    say(f"[extra-sync] {case}: outputs and masks equal {same}")
    assert np.isfinite(res[0][0]).all() and same


DECODE = [
    # B, Hq, Hkv, Sq, Skv, D, window, tiles per split, seed
    (2, 8, 2, 16, 3000, 128, 0, 8, 511),
    (1, 4, 4, 1, 777, 64, 0, 3, 512),
    (1, 16, 2, 5, 1300, 128, 400, 4, 513),
]


@pytest.mark.parametrize("case", DECODE)
def test_decode_equal_under_extra_sync(case):
    B, Hq, Hkv, Sq, Skv, D, window, tps, seed = case
    q, k, v = make_inputs(B, Hq, Hkv, Skv, D, seed, "channels", Sq=Sq)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    nT = (Skv + 63) // 64
    res = []
    for lib in _libs():
        out = torch.full((B, Hq, Sq, D), float("nan"), dtype=torch.float32, device="cuda")
        mask = torch.full((B, Hq, nT), 0x55, dtype=torch.uint8, device="cuda")
        rc = lib.lamp_attn_decode(_p(qd), _p(kd), _p(vd), _p(out), B, Hq, Hkv, Sq, Skv, D, 1, window,
                                  2 ** -8, 2 ** -1, tps, _p(mask))
        assert rc == 0, lib.lamp_last_error()
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), mask.cpu().numpy()))
    same = np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
    say(f"[extra-sync] decode {case}: outputs and masks equal {same}")
    assert np.isfinite(res[0][0]).all() and same
