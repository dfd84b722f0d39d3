"""Pins of the LampAttention oracle to facts other than itself.  No GPU.

What pins what:
* hand-worked example (tests/golden/worked_s17.json): scales, quantisation,
  logits, 8-bit and 16-bit exponentials, both test stages, the recompute;
* scalar exact-rational brute force (oracle.brute, separate code) on tiny
  inputs: every step, all masking modes, GQA, ragged tails;
* endpoints the pages bracket the method with ("8-bit" and "32-bit" columns
  of tables 1-6): second stage off == tiled 8-bit attention; every sub-block
  in 16-bit == bf16 attention up to bf16 rounding of the weights; exact fp64
  attention within the error of that rounding;
* invariants: normalised weights sum to 1 and reproduce the output; special
  cases with closed forms; monotonicity of the flags in delta and tau;
  quantisation invariants.
"""
import json
import os

import numpy as np
import pytest
import torch

from inputs import make_config_inputs, make_inputs
from oracle import lamp as L
from oracle.brute import brute_lamp
from oracle.formats import bf16_bits_to_f64
from oracle.refs import bf16_attention, eight_bit_attention, exact_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _maxv(v_bits):
    return float(np.abs(bf16_bits_to_f64(v_bits)).max())


# --------------------------------------------------------------------------
# worked example
# --------------------------------------------------------------------------
def _worked_inputs(fx):
    sh = fx["shape"]
    S, D = sh["S"], sh["D"]
    q = np.zeros((1, 1, S, D))
    k = np.zeros((1, 1, S, D))
    for r, ent in fx["inputs"]["q_rows"].items():
        for d, val in ent.items():
            q[0, 0, int(r), int(d)] = val
    for r, ent in fx["inputs"]["k_rows"].items():
        for d, val in ent.items():
            k[0, 0, int(r), int(d)] = val
    v = np.zeros((1, 1, S, D))
    for j in range(S):
        v[0, 0, j, j] = 1.0
    return _bits(q), _bits(k), _bits(v), sh


@pytest.mark.parametrize("case", ["A", "B", "C", "D", "E"])
def test_worked_example(case):
    fx = json.load(open(os.path.join(GOLDEN, "worked_s17.json")))
    q, k, v, sh = _worked_inputs(fx)
    cs = [c for c in fx["cases"] if c["name"] == case][0]
    tau = np.inf if cs["tau"] == "inf" else cs["tau"]
    out, mask = L.lamp_forward(q, k, v, causal=sh["causal"], window=sh["window"],
                               delta=cs["delta"], tau=tau)
    assert mask.shape == (1, 1, 1, 1) and int(mask[0, 0, 0, 0]) == cs["mask"]
    for r, ent in cs["out"].items():
        for d, want in ent.items():
            got = float(out[0, 0, int(r), int(d)])
            assert got == pytest.approx(want, rel=2e-7, abs=1e-12), (case, r, d)


def test_worked_example_scales():
    fx = json.load(open(os.path.join(GOLDEN, "worked_s17.json")))
    q, k, _, _ = _worked_inputs(fx)
    qv, qc, sq, iq = L.quantize(q)
    kv, kc, sk, ik = L.quantize(k)
    assert (sq[0, 0], iq[0, 0], sk[0, 0], ik[0, 0]) == (2.0 ** -6, 64.0, 2.0 ** -5, 32.0)
    assert qv[0, 0, 0, 0] == 112 and qv[0, 0, 1, 0] == 448
    assert kv[0, 0, 0, 0] == 448 and kv[0, 0, 16, 0] == -112
    c8, c16 = L.logit_constants(64, sq[0, 0], sk[0, 0])
    assert c8 == 12102203 / 2.0 ** 37 and c16 == 12102203 / 2.0 ** 26


# --------------------------------------------------------------------------
# brute force
# --------------------------------------------------------------------------
BRUTE_CASES = [
    # B, Hq, Hkv, S, D, causal, window, delta, tau, structure, seed
    (1, 2, 1, 70, 64, 1, 0, 2 ** -8, 2 ** -2, "sinks", 7),
    (1, 2, 2, 80, 64, 0, 0, 2 ** -4, 2 ** -3, "channels", 8),
    (2, 2, 1, 67, 64, 1, 20, 0.0, 2 ** -1, "channels", 9),
    (1, 1, 1, 33, 64, 1, 0, 0.0, 0.0, "plain", 10),
]


@pytest.mark.slow
@pytest.mark.parametrize("case", BRUTE_CASES)
def test_brute_force_equals_oracle(case):
    B, Hq, Hkv, S, D, causal, window, delta, tau, structure, seed = case
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, structure)
    if structure == "channels":
        # scale up so that tau = 2^-3..2^-1 actually flags something
        q = _bits(bf16_bits_to_f64(q) * 3.0)
    bo, bm = brute_lamp(q.tolist(), k.tolist(), v.tolist(), causal, window, delta, tau)
    out, mask = L.lamp_forward(q, k, v, causal, window, delta, tau)
    nT = mask.shape[-1]
    for b in range(B):
        for h in range(Hq):
            for r in range(nT):
                for t in range(nT):
                    assert int(mask[b, h, r, t]) == bm.get((b, h, r, t), 0), (b, h, r, t)
    np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-6)
    assert np.abs(out - np.array(bo)).max() <= 4e-7 * max(1.0, np.abs(out).max())


def test_brute_force_flags_something():
    # the brute-force cases above must exercise the recompute path
    q, k, v = make_inputs(1, 2, 1, 70, 64, 7, "sinks")
    _, mask = L.lamp_forward(q, k, v, True, 0, 2 ** -8, 2 ** -2)
    assert ((mask & 0x0F) != 0).any()


# --------------------------------------------------------------------------
# endpoints
# --------------------------------------------------------------------------
ENDPOINT_SHAPES = [
    (1, 1, 1, 256, 64, 1, 0, "sinks", 1),
    (1, 4, 2, 200, 128, 1, 0, "channels", 11),
    (1, 2, 1, 190, 64, 1, 50, "channels", 12),
    (1, 2, 2, 130, 64, 0, 0, "channels", 13),
]


@pytest.mark.parametrize("shape", ENDPOINT_SHAPES)
def test_second_stage_off_is_eight_bit_attention(shape):
    B, Hq, Hkv, S, D, causal, window, structure, seed = shape
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, structure)
    out, mask = L.lamp_forward(q, k, v, causal, window, 2 ** -8, np.inf)
    visited = mask != 0
    assert np.all(mask[visited] == 0x80)
    ref = eight_bit_attention(q, k, v, causal, window)
    # oracle output is rounded to fp32 once; REF8 keeps fp64
    assert np.abs(out - ref).max() <= 2.0 ** -23 * np.abs(ref).max() + 1e-12


@pytest.mark.parametrize("shape", ENDPOINT_SHAPES)
def test_all_sixteen_bit_is_bf16_attention(shape):
    B, Hq, Hkv, S, D, causal, window, structure, seed = shape
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, structure)
    out, mask = L.lamp_forward(q, k, v, causal, window, 0.0, 0.0)
    st = L.subblock_stats(mask, S, causal, window)
    assert st["flagged_subblocks"] == st["visited_subblocks"]
    ref = bf16_attention(q, k, v, causal, window)
    # weights carry one bf16 rounding (unit roundoff 2^-8) on each side
    u = 2.0 ** -8
    bound = 4 * u / (1 - u) * _maxv(v)
    assert np.abs(out - ref).max() <= bound
    ex = exact_attention(q, k, v, causal, window)
    assert np.abs(out - ex).max() <= bound


@pytest.mark.parametrize("shape", ENDPOINT_SHAPES)
def test_plain_bf16_is_bf16_attention(shape):
    # the tiled 16-bit baseline against the untiled definitions: bf16 attention
    # with the global row max, and exact attention, each within the bf16
    # rounding of the weights
    B, Hq, Hkv, S, D, causal, window, structure, seed = shape
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, structure)
    out, mask = L.plain_forward(q, k, v, causal, window)
    visited = mask != 0
    assert np.all(mask[visited] == 0x8F)
    st = L.subblock_stats(mask, S, causal, window)
    assert st["flagged_subblocks"] == st["visited_subblocks"] > 0
    u = 2.0 ** -8
    bound = 4 * u / (1 - u) * _maxv(v)
    assert np.abs(out - bf16_attention(q, k, v, causal, window)).max() <= bound
    assert np.abs(out - exact_attention(q, k, v, causal, window)).max() <= bound


def test_plain_bf16_special_cases():
    # one key: the output is v0; equal keys: every weight is exactly 1 and the
    # output is the mean of the visible values; zero queries: cumulative mean
    q, k, v = make_inputs(1, 2, 1, 1, 64, 3, "plain")
    out, _ = L.plain_forward(q, k, v, True, 0)
    assert np.array_equal(out[0, :, 0], np.repeat(bf16_bits_to_f64(v)[0, :, 0], 2, axis=0))
    S, D = 100, 64
    q, k1, v = make_inputs(1, 1, 1, S, D, 5, "plain")
    k = np.repeat(k1[:, :, :1], S, axis=2)
    out, _ = L.plain_forward(q, k, v, False, 0)
    vv = bf16_bits_to_f64(v)[0, 0]
    np.testing.assert_allclose(out[0, 0], np.repeat(vv.mean(axis=0)[None], S, axis=0), atol=1e-6)
    qz = np.zeros_like(q)
    out, _ = L.plain_forward(qz, k1, v, True, 30)
    for i in (0, 29, 30, 99):
        np.testing.assert_allclose(out[0, 0, i], vv[max(0, i - 29):i + 1].mean(axis=0), atol=1e-6)


def test_lamp_recovers_from_eight_bit_error():
    # the pages' claim: sending a minority of sub-blocks to 16-bit recovers
    # most of the 8-bit error (tables 1-6); on the sink workload
    q, k, v, cfg = make_config_inputs("tiny")
    ex = exact_attention(q, k, v, True, 0)
    lamp, mask = L.lamp_forward(q, k, v, True, 0, 2 ** -8, 2 ** -1)
    r8 = eight_bit_attention(q, k, v, True, 0)
    st = L.subblock_stats(mask, cfg["S"], True, 0)
    assert 0 < st["r_sb"] < 0.5
    assert np.abs(lamp - ex).max() < 0.5 * np.abs(r8 - ex).max()


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shape", ENDPOINT_SHAPES[:3])
def test_normalised_weights_sum_to_one(shape):
    B, Hq, Hkv, S, D, causal, window, structure, seed = shape
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, structure)
    ctx = L.prepare(q, k, v, causal, window, 2 ** -8, 2 ** -2)
    vv = bf16_bits_to_f64(v)
    for (b, hq, r) in [(0, 0, 0), (0, Hq - 1, L.n_tiles(S) - 1), (0, 0, L.n_tiles(S) // 2)]:
        trace = []
        out, _ = L.run_unit(ctx, b, hq, r, trace=trace)
        fin = trace[-1]
        rows = out.shape[0]
        W = np.zeros((rows, S))
        for rec in trace[:-1]:
            scale = np.exp2(rec["m_new"] - fin["m"]) / fin["ell"]
            W[:, rec["cols"]] = rec["p"] * scale[:, None]
        np.testing.assert_allclose(W.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(W @ vv[b, hq // (Hq // Hkv)], out, rtol=0, atol=1e-6)
        # every visible entry is counted, every masked one is not
        rws = np.arange(r * 64, r * 64 + rows)
        vis = L.visible(rws, np.arange(S), causal, window)
        assert np.all(W[~vis] == 0)


def test_single_key_returns_v0():
    q, k, v = make_inputs(1, 2, 1, 1, 64, 3, "plain")
    for dl, ta in ((2 ** -8, 2 ** -1), (0.0, 0.0), (2 ** -8, np.inf)):
        out, mask = L.lamp_forward(q, k, v, True, 0, dl, ta)
        assert np.array_equal(out[0, :, 0], np.repeat(bf16_bits_to_f64(v)[0, :, 0], 2, axis=0))


def test_zero_queries_average_visible_values():
    B, Hq, S, D = 1, 2, 150, 64
    _, k, v = make_inputs(B, Hq, 1, S, D, 4, "channels")
    q = np.zeros((B, Hq, S, D), dtype=np.uint16)
    out, mask = L.lamp_forward(q, k, v, True, 0, 2 ** -8, 2 ** -1)
    assert np.all((mask[mask != 0] & 0x0F) == 0)          # |s| = 0 < T2
    vv = bf16_bits_to_f64(v)[0, 0]
    mean = np.cumsum(vv, axis=0) / np.arange(1, S + 1)[:, None]
    np.testing.assert_allclose(out[0, 0], mean, rtol=0, atol=1e-6)
    # window: the mean over the last W keys
    out_w, _ = L.lamp_forward(q, k, v, True, 30, 2 ** -8, 2 ** -1)
    for i in (0, 29, 30, 100, 149):
        np.testing.assert_allclose(out_w[0, 1, i], vv[max(0, i - 29):i + 1].mean(axis=0), atol=1e-6)


def test_equal_keys_give_uniform_mean():
    S, D = 100, 64
    q, k1, v = make_inputs(1, 1, 1, S, D, 5, "plain")
    k = np.repeat(k1[:, :, :1], S, axis=2)
    out, _ = L.lamp_forward(q, k, v, False, 0, 2 ** -8, 2 ** -1)
    vv = bf16_bits_to_f64(v)[0, 0]
    np.testing.assert_allclose(out[0, 0], np.repeat(vv.mean(axis=0)[None], S, axis=0), atol=1e-6)


def test_one_dominant_key_flags_only_its_subblock():
    S, D = 128, 64
    q = np.zeros((1, 1, S, D))
    q[..., 0] = 1.0
    k = np.random.default_rng(6).standard_normal((1, 1, S, D)) * 0.01
    k[0, 0, 37, 0] = 320.0           # logit 320/8 = 40 for every query
    _, _, v = make_inputs(1, 1, 1, S, D, 6, "plain")
    qb, kb = _bits(q), _bits(k)
    out, mask = L.lamp_forward(qb, kb, v, False, 0, 2 ** -8, 2 ** -1)
    # key 37 is sub-block 2 of tile 0; the other entries have p8 = 0 < delta
    assert np.all(mask[0, 0, :, 0] == 0x80 | (1 << 2))
    assert np.all(mask[0, 0, :, 1] == 0x80)
    np.testing.assert_allclose(out[0, 0], np.repeat(bf16_bits_to_f64(v)[0, 0, 37][None], S, axis=0),
                               atol=1e-12)
    # with the first stage disabled every sub-block holds sensitive entries?
    # no: the other logits are ~0.01 * |q| / 8, far below T2, so still one
    _, mask0 = L.lamp_forward(qb, kb, v, False, 0, 0.0, 2 ** -1)
    assert np.array_equal(mask0, mask)


@pytest.mark.parametrize("shape", ENDPOINT_SHAPES[:3])
def test_flags_monotone_in_tau_and_delta(shape):
    B, Hq, Hkv, S, D, causal, window, structure, seed = shape
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, structure)
    q = _bits(bf16_bits_to_f64(q) * 2.0)
    masks = {}
    for dl in (0.0, 2 ** -8, 2 ** -4):
        for t in range(6):
            _, m = L.lamp_forward(q, k, v, causal, window, dl, 2.0 ** -t)
            masks[dl, t] = m & 0x0F
    for dl in (0.0, 2 ** -8, 2 ** -4):
        for t in range(5):
            # smaller tau flags a superset
            assert np.all((masks[dl, t] & ~masks[dl, t + 1]) == 0)
    for t in range(6):
        assert np.all((masks[2 ** -4, t] & ~masks[2 ** -8, t]) == 0)
        assert np.all((masks[2 ** -8, t] & ~masks[0.0, t]) == 0)
    assert masks[0.0, 5].any()


def test_quantisation_invariants():
    q, k, v = make_inputs(2, 3, 3, 77, 64, 14, "channels")
    vals, codes, scale, inv = L.quantize(q)
    amax = np.abs(vals).max(axis=(2, 3))
    assert np.all(amax == 448.0)
    # scaling the input by a power of two leaves the codes unchanged
    q2 = _bits(bf16_bits_to_f64(q) * 2.0 ** -5)
    _, codes2, scale2, _ = L.quantize(q2)
    assert np.array_equal(codes, codes2)
    assert np.array_equal(scale2, scale * 2.0 ** -5)
    # an all-zero head has scale 1 and zero codes
    z = q.copy()
    z[1, 2] = 0
    _, cz, sz, iz = L.quantize(z)
    assert sz[1, 2] == 1.0 and iz[1, 2] == 1.0 and np.all(cz[1, 2] == 0)


def test_stats_closed_forms():
    S = 300
    nT = L.n_tiles(S)
    mask = np.zeros((1, 2, nT, nT), dtype=np.uint8)
    for r in range(nT):
        for t in range(r + 1):
            mask[:, :, r, t] = 0x80
    st = L.subblock_stats(mask, S, True, 0)
    assert st["visited_tiles"] == 2 * nT * (nT + 1) // 2
    assert st["visible_entries"] == 2 * S * (S + 1) // 2
    assert st["hist"] == [st["visited_tiles"], 0, 0, 0, 0]
    assert st["r_sb"] == 0.0
    mask[:, :, :, :] = np.where(mask != 0, 0x8F, 0)
    st = L.subblock_stats(mask, S, True, 0)
    assert st["r_e"] == 1.0 and st["r_sb"] == 1.0
