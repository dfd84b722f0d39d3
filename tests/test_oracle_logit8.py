"""Pins of the oracle's literal 8-bit-logit variant (``logit8``).  No GPU.

The variant takes the 8-bit accumulation of key-query products that the
abstract of "LampAttention: Look-Ahead Mixed-Precision FlashAttention for
Dedicated Accelerators" describes literally: the log2-domain logit is an
e4m3 value.
Pinned here by

* a two-key input whose logits and weights are worked out by hand, where
  the rounded logit changes an 8-bit weight (and the same input run in the
  default reading, where it does not round);
* the same input at a tau whose threshold lies between a logit and its e4m3
  rounding, so only the variant's second stage fires;
* the scalar exact-rational brute force (oracle.brute, separate code).
"""
import numpy as np
import pytest
import torch

from inputs import make_inputs
from oracle import lamp as L
from oracle.brute import brute_lamp
from oracle.formats import bf16_bits_to_f64, e4m3_decode, e4m3_encode


def _bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _two_keys():
    """D = 64, S = 2, causal.  Both queries are 64 e_0; the keys are e_0 and
    e_0 / 2; the values e_0 and e_1.

    Scales: Q amax 64 -> inverse scale 448/64 = 7, Q codes 448; K amax 1 ->
    inverse scale 448, K codes 448 and 224.  The logits of query 1 are
    log2(e)/8 times the true products 64 and 32: 11.5416 and 5.7708
    (to within the fp32 roundings of the scales, far from any e4m3 midpoint).
    """
    D = 64
    q = np.zeros((1, 1, 2, D))
    q[0, 0, :, 0] = 64.0
    k = np.zeros((1, 1, 2, D))
    k[0, 0, 0, 0] = 1.0
    k[0, 0, 1, 0] = 0.5
    v = np.zeros((1, 1, 2, D))
    v[0, 0, 0, 0] = 1.0
    v[0, 0, 1, 1] = 1.0
    return _bits(q), _bits(k), _bits(v)


def test_two_key_closed_form():
    """Query 1, second stage off.  Default reading: x = 5.7708 - 11.5416 =
    -5.7708, 2^x = 0.018360, which rounds to 9 * 2^-9 (spacing 2^-9 below
    2^-5); the output is (1 e_0 + 9/512 e_1) / (1 + 9/512).  Variant: the
    logits round to 12 (spacing 1 in [8, 16)) and 6 (spacing 1/2 in [4, 8)),
    x = -6, 2^x = 2^-6 exactly; the output is (64 e_0 + e_1) / 65."""
    q, k, v = _two_keys()
    out, mask = L.lamp_forward(q, k, v, causal=True, window=0, delta=2.0 ** -8, tau=np.inf)
    assert int(mask[0, 0, 0, 0]) == 0x80
    assert out[0, 0, 0, 0] == 1.0 and out[0, 0, 0, 1] == 0.0
    assert out[0, 0, 1, 0] == np.float32(512 / 521) and out[0, 0, 1, 1] == np.float32(9 / 521)
    out8, mask8 = L.lamp_forward(q, k, v, causal=True, window=0, delta=2.0 ** -8, tau=np.inf,
                                 logit8=True)
    assert int(mask8[0, 0, 0, 0]) == 0x80
    assert out8[0, 0, 0, 0] == 1.0 and out8[0, 0, 0, 1] == 0.0
    assert out8[0, 0, 1, 0] == np.float32(64 / 65) and out8[0, 0, 1, 1] == np.float32(1 / 65)
    assert np.all(out8[0, 0, :, 2:] == 0.0)


def test_second_stage_reads_the_eight_bit_logit():
    """T2 = 11.8 lies between the fp32 logit 11.5416 of key 0 and its e4m3
    rounding 12: only the variant flags sub-block 0 (keys 0-15)."""
    q, k, v = _two_keys()
    tau = 11.8 / (16 * L.LOG2E)
    _, mask = L.lamp_forward(q, k, v, causal=True, window=0, delta=2.0 ** -8, tau=tau)
    _, mask8 = L.lamp_forward(q, k, v, causal=True, window=0, delta=2.0 ** -8, tau=tau, logit8=True)
    assert int(mask[0, 0, 0, 0]) == 0x80
    assert int(mask8[0, 0, 0, 0]) == 0x81


def test_logits_on_the_e4m3_grid():
    """Every visible logit of the variant is an e4m3 value, and the running
    max is one of them."""
    q, k, v = make_inputs(1, 2, 1, 150, 64, 21, "channels")
    ctx = L.prepare(q, k, v, True, 0, 2.0 ** -8, 2.0 ** -1, logit8=True)
    for r in range(L.n_tiles(150)):
        trace = []
        L.run_unit(ctx, 0, 1, r, trace=trace)
        for rec in trace[:-1]:
            s = rec["s2"][rec["vis"]]
            assert np.array_equal(e4m3_decode(e4m3_encode(s)), s)
            live = np.isfinite(rec["m_new"])
            assert np.all(np.isin(rec["m_new"][live], np.concatenate(
                [tr["s2"][tr["vis"]] for tr in trace[:-1]])))


BRUTE8 = [
    # B, Hq, Hkv, S, D, causal, window, delta, tau, structure, seed, q gain
    (1, 2, 1, 70, 64, 1, 0, 2 ** -8, 2 ** -2, "sinks", 31, 1.0),
    (1, 2, 2, 80, 64, 0, 0, 2 ** -4, 2 ** -3, "channels", 32, 3.0),
    (1, 1, 1, 67, 64, 1, 20, 0.0, 2 ** -1, "channels", 33, 3.0),
]


@pytest.mark.slow
@pytest.mark.parametrize("case", BRUTE8)
def test_brute_force_equals_oracle_logit8(case):
    B, Hq, Hkv, S, D, causal, window, delta, tau, structure, seed, gain = case
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, structure)
    q = _bits(bf16_bits_to_f64(q) * gain)
    bo, bm = brute_lamp(q.tolist(), k.tolist(), v.tolist(), causal, window, delta, tau, logit8=True)
    out, mask = L.lamp_forward(q, k, v, causal, window, delta, tau, logit8=True)
    nT = mask.shape[-1]
    for b in range(B):
        for h in range(Hq):
            for r in range(nT):
                for t in range(nT):
                    assert int(mask[b, h, r, t]) == bm.get((b, h, r, t), 0), (b, h, r, t)
    assert np.abs(out - np.array(bo)).max() <= 4e-7 * max(1.0, np.abs(out).max())
    # the variant must differ from the default reading on these inputs
    out0, _ = L.lamp_forward(q, k, v, causal, window, delta, tau)
    assert np.abs(out0 - out).max() > 1e-4
