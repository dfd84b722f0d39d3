"""The parity protocols themselves, on the CPU: each accepts the oracle it
checks against and rejects a planted mistake (the other reading of the
8-bit logits, fed in as if a device had computed it).  No GPU."""
import numpy as np

from inputs import make_inputs
from oracle import lamp as L
from parity import assert_parity, assert_parity_logit8, compare, compare_logit8

CASE = (1, 2, 1, 150, 64, 1, 0, 2.0 ** -8, 2.0 ** -1, "channels", 41)


def _inputs():
    B, Hq, Hkv, S, D, causal, window, delta, tau, st, seed = CASE
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, st)
    return q, k, v, causal, window, delta, tau


def test_logit8_protocol_accepts_the_oracle():
    q, k, v, causal, window, delta, tau = _inputs()
    dev = L.lamp_forward(q, k, v, causal, window, delta, tau, logit8=True)
    rep = compare_logit8(q, k, v, causal, window, delta, tau, gpu=dev, label="self")
    assert_parity_logit8(rep)
    assert rep["max_abs"] == 0.0 and rep["excused"] == 0


def test_logit8_protocol_rejects_the_default_reading():
    q, k, v, causal, window, delta, tau = _inputs()
    dev = L.lamp_forward(q, k, v, causal, window, delta, tau)
    rep = compare_logit8(q, k, v, causal, window, delta, tau, gpu=dev, label="planted")
    bad = bool(rep["unexcused"]) or bool(rep["rows_unexplained"]) or rep["mean_abs"] > 5e-4
    assert bad, rep


def test_default_protocol_accepts_the_oracle_and_rejects_logit8():
    q, k, v, causal, window, delta, tau = _inputs()
    dev = L.lamp_forward(q, k, v, causal, window, delta, tau)
    assert_parity(compare(q, k, v, causal, window, delta, tau, gpu=dev, label="self"))
    dev8 = L.lamp_forward(q, k, v, causal, window, delta, tau, logit8=True)
    rep = compare(q, k, v, causal, window, delta, tau, gpu=dev8, label="planted")
    assert bool(rep["unexcused"]) or bool(rep["rows_unexplained"]) or rep["mean_abs"] > 5e-4, rep


def test_decode_protocol_accepts_the_oracle_and_rejects_other_splits():
    from parity import assert_parity_decode, compare_decode
    from inputs import make_inputs as mk
    q, k, v = mk(1, 4, 2, 700, 64, 43, "channels", Sq=9)
    dev = L.decode_forward(q, k, v, 1, 0, 2.0 ** -8, 2.0 ** -2, tiles_per_split=3)
    assert_parity_decode(compare_decode(q, k, v, 1, 0, 2.0 ** -8, 2.0 ** -2, 3, gpu=dev, label="self"))
    # a device that split differently (one split) computes a different result
    dev1 = L.decode_forward(q, k, v, 1, 0, 2.0 ** -8, 2.0 ** -2, tiles_per_split=11)
    rep = compare_decode(q, k, v, 1, 0, 2.0 ** -8, 2.0 ** -2, 3, gpu=dev1, label="planted")
    assert bool(rep["unexcused"]) or bool(rep["rows_unexplained"]) or rep["mean_abs"] > 5e-4, rep


def _flip_case():
    """A unit and tile whose flag some window allows to flip, and one whose
    flag no window allows to flip (seed 43 holds one such fragile flag)."""
    from parity import fragile_mask_bits
    q, k, v = make_inputs(1, 2, 1, 200, 64, 43, "channels")
    causal, window, delta, tau = 1, 0, 2.0 ** -8, 2.0 ** -1
    ctx = L.prepare(q, k, v, causal, window, delta, tau)
    fragile = solid = None
    for (b, h, r) in L.all_units(*q.shape[:3]):
        trace = []
        L.run_unit(ctx, b, h, r, trace=trace)
        for rec in trace[:-1]:
            bits = fragile_mask_bits(ctx, b, h, r, rec)
            if bits and fragile is None:
                fragile = (b, h, r, rec["t"], bits & -bits)
            if solid is None and bits != 0xF:
                free = ~bits & 0xF
                solid = (b, h, r, rec["t"], free & -free)
    return (q, k, v, causal, window, delta, tau), fragile, solid


def _device_with_flip(args, b, h, r, t, bit):
    q, k, v, causal, window, delta, tau = args
    out, mask = L.lamp_forward(q, k, v, causal, window, delta, tau)
    ov = mask.copy()
    ov[b, h, r, t] ^= bit
    out2, _ = L.lamp_forward(q, k, v, causal, window, delta, tau, units=[(b, h, r)], flag_override=ov)
    rows = slice(r * 64, r * 64 + 64)
    out[b, h, rows] = out2[b, h, rows]
    return out, ov


def test_protocol_bounds_an_excused_flag_without_replay():
    args, fragile, solid = _flip_case()
    assert fragile is not None and solid is not None
    dev = _device_with_flip(args, *fragile)
    rep = compare(*args, gpu=dev, label="excused flip")
    assert_parity(rep)
    assert len(rep["excused"]) == 1
    dev = _device_with_flip(args, *solid)
    rep = compare(*args, gpu=dev, label="unexcused flip")
    assert len(rep["unexcused"]) == 1
