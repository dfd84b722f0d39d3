"""Pins of the oracle's split-KV decode.  No GPU.

Decode runs a few query rows (the last positions of the sequence) against
all cached keys, with the KV tiles cut into splits that are processed
independently and merged.  Pinned by

* the scalar exact-rational brute force (oracle.brute.brute_decode,
  separate code) with several splits, GQA, windows and one query row;
* one split against the prefill oracle: the same queries at the end of a
  prefill whose other query rows are zero give the same outputs and flags
  (the prefill oracle is pinned on its own);
* the all-16-bit endpoint against textbook attention, written out here,
  within the bf16 rounding of the weights, for several split sizes;
* closed forms: a single visible key returns its value row.
"""
import math

import numpy as np
import pytest

from inputs import make_inputs
from oracle import lamp as L
from oracle.brute import brute_decode
from oracle.formats import bf16_bits_to_f64

DEC_BRUTE = [
    # B, Hq, Hkv, Sq, Skv, D, causal, window, delta, tau, tiles_per_split, structure, seed
    (1, 2, 1, 3, 200, 64, 1, 0, 2 ** -8, 2 ** -2, 1, "sinks", 61),
    (1, 4, 2, 1, 150, 64, 1, 0, 2 ** -4, 2 ** -3, 2, "channels", 62),
    (1, 2, 2, 5, 140, 64, 1, 70, 0.0, 2 ** -1, 1, "channels", 63),
    (1, 1, 1, 16, 130, 64, 0, 0, 2 ** -8, 2 ** -2, 3, "sinks", 64),
]


@pytest.mark.slow
@pytest.mark.parametrize("case", DEC_BRUTE)
def test_brute_force_equals_decode_oracle(case):
    B, Hq, Hkv, Sq, Skv, D, causal, window, delta, tau, tps, st, seed = case
    q, k, v = make_inputs(B, Hq, Hkv, Skv, D, seed, st, Sq=Sq)
    bo, bm = brute_decode(q.tolist(), k.tolist(), v.tolist(), causal, window, delta, tau, tps)
    out, mask = L.decode_forward(q, k, v, causal, window, delta, tau, tiles_per_split=tps)
    for b in range(B):
        for h in range(Hq):
            for t in range(mask.shape[-1]):
                assert int(mask[b, h, t]) == bm.get((b, h, t), 0), (b, h, t)
    ref = np.array(bo)
    assert np.abs(out - ref).max() <= 4e-7 * max(1.0, np.abs(ref).max())


def test_decode_flags_something_and_splits_matter():
    # the first brute-force case exercises the recompute, and its splits
    # change the result (each split has its own running max)
    B, Hq, Hkv, Sq, Skv, D, causal, window, delta, tau, tps, st, seed = DEC_BRUTE[0]
    q, k, v = make_inputs(B, Hq, Hkv, Skv, D, seed, st, Sq=Sq)
    o1, m1 = L.decode_forward(q, k, v, causal, window, delta, tau, tiles_per_split=1)
    o4, _ = L.decode_forward(q, k, v, causal, window, delta, tau, tiles_per_split=4)
    assert ((m1 & 0x0F) != 0).any()
    assert np.abs(o1 - o4).max() > 0


@pytest.mark.parametrize("shape", [(1, 2, 1, 16, 300, 128, 1, 0, "channels", 65),
                                   (1, 4, 2, 7, 190, 64, 1, 50, "sinks", 66),
                                   (1, 2, 2, 1, 64, 64, 1, 0, "channels", 67)])
def test_one_split_equals_prefill_with_zero_rows(shape):
    """Prefill over Skv rows whose first Skv - Sq query rows are zero: its Q
    scale is that of the Sq decode rows, and the zero rows (logit 0, below
    T2 > 0) flag nothing, so its last row block gives the decode result."""
    B, Hq, Hkv, Sq, Skv, D, causal, window, st, seed = shape
    assert (Skv - Sq) >= ((Skv - 1) // 64) * 64           # decode rows in one row block
    q, k, v = make_inputs(B, Hq, Hkv, Skv, D, seed, st, Sq=Sq)
    qp = np.zeros((B, Hq, Skv, D), dtype=np.uint16)      # bf16 +0
    qp[:, :, Skv - Sq:] = q
    delta, tau = 2.0 ** -8, 2.0 ** -4
    out, mask = L.decode_forward(q, k, v, causal, window, delta, tau)
    r = (Skv - 1) // 64
    units = [(b, h, r) for b in range(B) for h in range(Hq)]
    outp, maskp = L.lamp_forward(qp, k, v, causal, window, delta, tau, units=units)
    assert np.array_equal(out, outp[:, :, Skv - Sq:])
    # tiles only the zero rows see (a window) are visited by the prefill alone
    mp = maskp[:, :, r, :]
    seen = (mask & 0x80) != 0
    assert np.array_equal(mask[seen], mp[seen]) and not (mp[~seen] & 0x0F).any()
    assert ((mask & 0x0F) != 0).any()


def _textbook(q_bits, k_bits, v_bits, causal, window):
    """softmax(q k^T / sqrt(D)) v over the visible keys, in fp64."""
    q, k, v = (bf16_bits_to_f64(x) for x in (q_bits, k_bits, v_bits))
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    out = np.zeros(q.shape)
    for b in range(B):
        for h in range(Hq):
            kk, vv = k[b, h // (Hq // Hkv)], v[b, h // (Hq // Hkv)]
            for i in range(Sq):
                p = Skv - Sq + i
                j = np.arange(Skv)
                vis = np.ones(Skv, dtype=bool)
                if causal:
                    vis &= j <= p
                if window > 0:
                    vis &= p - j < window
                s = kk[vis] @ q[b, h, i] / math.sqrt(D)
                w = np.exp(s - s.max())
                out[b, h, i] = w @ vv[vis] / w.sum()
    return out


@pytest.mark.parametrize("tps", [1, 2, 5, None])
def test_all_sixteen_bit_decode_is_attention(tps):
    q, k, v = make_inputs(1, 4, 2, 300, 64, 68, "channels", Sq=9)
    out, mask = L.decode_forward(q, k, v, 1, 0, 0.0, 0.0, tiles_per_split=tps)
    # every sub-block holding a cached key is recomputed (keys 256..299 fill
    # sub-blocks 0-2 of the last tile)
    assert np.all(mask[..., :-1] == 0x8F) and np.all(mask[..., -1] == 0x87)
    ex = _textbook(q, k, v, 1, 0)
    u = 2.0 ** -8
    assert np.abs(out - ex).max() <= 4 * u / (1 - u) * np.abs(bf16_bits_to_f64(v)).max()
    assert np.abs(out - ex).max() > 0


def test_single_visible_key_returns_its_value():
    # Sq = Skv = 1: the one query sees only key 0, whatever the split
    q, k, v = make_inputs(1, 2, 1, 1, 64, 69, "plain", Sq=1)
    out, mask = L.decode_forward(q, k, v, 1, 0, 2.0 ** -8, 2.0 ** -1, tiles_per_split=1)
    vv = bf16_bits_to_f64(v)
    assert np.array_equal(out[0, 0, 0], vv[0, 0, 0].astype(np.float32))
    assert np.array_equal(out[0, 1, 0], vv[0, 0, 0].astype(np.float32))
    assert mask.shape == (1, 2, 1) and np.all(mask & 0x80)
