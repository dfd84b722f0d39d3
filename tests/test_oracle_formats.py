"""Pins of the oracle's software formats against independent implementations.

The e4m3fn and bf16 roundings are checked against torch's CPU casts (separate
code), hand values, and exact rational arithmetic; fma32 against exact
rationals.  No GPU.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.formats import (bf16_bits_to_f64, e4m3_decode, e4m3_encode, exp2_f32, fl32,
                            fma32, round_bf16, round_e4m3)


def _torch_e4m3(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.float().double().numpy(), t.view(torch.uint8).numpy()


def _all_finite_e4m3():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    return codes, e4m3_decode(codes)


def test_e4m3_hand_values():
    cases = {1.5 * 2 ** -9: 2 ** -8, 2 ** -10: 0.0, 0.53125: 0.5, 0.59375: 0.625,
             464.0: 448.0, 465.0: 448.0, 1e6: 448.0, -1e-9: 0.0, 2 ** -9: 2 ** -9,
             0.75 * 2 ** -9: 2 ** -9, 2.5 * 2 ** -9: 2 ** -8, 3.5 * 2 ** -9: 4 * 2 ** -9}
    for x, want in cases.items():
        assert round_e4m3(x) == want, x
    assert np.signbit(round_e4m3(-1e-9))
    assert e4m3_encode(round_e4m3(-1e-9)) == 0x80


def test_e4m3_codes_roundtrip():
    codes, vals = _all_finite_e4m3()
    assert np.array_equal(e4m3_encode(vals), codes)
    assert np.array_equal(round_e4m3(vals), vals)
    pos = np.sort(vals[vals > 0])
    assert pos[0] == 2.0 ** -9 and pos[-1] == 448.0 and pos.size == 126


def test_e4m3_matches_torch_near_every_midpoint():
    _, vals = _all_finite_e4m3()
    grid = np.unique(vals)
    mids = (grid[:-1] + grid[1:]) / 2.0
    mids = mids[np.abs(mids) < 464]
    pts = [grid, mids]
    m32 = mids.astype(np.float32)
    for k in range(1, 4):
        up, dn = m32.copy(), m32.copy()
        for _ in range(k):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(-np.inf))
        pts += [up.astype(np.float64), dn.astype(np.float64)]
    x = np.concatenate(pts)
    x = x[np.abs(x) < 464].astype(np.float32)
    tv, tb = _torch_e4m3(x)
    assert np.array_equal(round_e4m3(x.astype(np.float64)), tv)
    assert np.array_equal(e4m3_encode(round_e4m3(x.astype(np.float64))), tb)


def test_e4m3_matches_torch_random():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(-463.9, 463.9, 200_000),
        rng.standard_normal(200_000) * np.exp2(rng.integers(-14, 8, 200_000)),
    ]).astype(np.float32)
    x = x[np.abs(x) < 464]          # torch's cast is not saturating beyond the last midpoint
    tv, tb = _torch_e4m3(x)
    ours = round_e4m3(x.astype(np.float64))
    assert np.array_equal(ours, tv)
    assert np.array_equal(e4m3_encode(ours), tb)


def test_bf16_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, 300_000, dtype=np.uint64).astype(np.uint32)
    exps = (bits >> 23) & 0xFF
    bits = bits[(exps > 0) & (exps < 0xFE)]
    ties = (bits & 0xFFFF0000) | 0x8000          # exact halfway cases
    x = np.concatenate([bits, ties]).view(np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16).float().double().numpy()
    assert np.array_equal(round_bf16(x.astype(np.float64)), t)
    assert round_bf16(1.0 + 2 ** -8) == 1.0            # tie to even (down)
    assert round_bf16(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6  # tie to even (up)


def test_bf16_bits_to_f64():
    assert bf16_bits_to_f64(np.uint16(0x3F80)) == 1.0
    assert bf16_bits_to_f64(np.uint16(0xC0A0)) == -5.0
    assert bf16_bits_to_f64(np.uint16(0x0001)) == 2.0 ** -133


def test_fma32_exact():
    rng = np.random.default_rng(2)
    a = fl32(rng.standard_normal(3000) * 1e3)
    b = fl32(rng.standard_normal(3000))
    c = fl32(rng.standard_normal(3000) * 1e3)
    got = fma32(a, b, c)
    for i in range(a.size):
        ex = Fraction(a[i]) * Fraction(b[i]) + Fraction(c[i])
        r = float(np.float32(float(ex)))
        # exact rounding check: no fp32 is closer to ex than the result
        lo = float(np.nextafter(np.float32(got[i]), np.float32(-np.inf)))
        hi = float(np.nextafter(np.float32(got[i]), np.float32(np.inf)))
        d = abs(Fraction(got[i]) - ex)
        assert d <= abs(Fraction(lo) - ex) and d <= abs(Fraction(hi) - ex), (i, r)


def test_fma32_double_rounding_case():
    # a = b = 1 + 2^-12: a*b = 1 + 2^-11 + 2^-24, exactly the fp32 midpoint
    # between lo = 1 + 2^-11 (even) and hi = lo + 2^-23.  Adding +-2^-80 in
    # fp64 rounds back onto the midpoint; a second rounding to fp32 would then
    # always give lo, but the exact sum lies above (below) the midpoint.
    a = b = 1.0 + 2.0 ** -12
    assert a * b == 1.0 + 2.0 ** -11 + 2.0 ** -24
    lo, hi = 1.0 + 2.0 ** -11, 1.0 + 2.0 ** -11 + 2.0 ** -23
    assert fma32(a, b, 2.0 ** -80) == hi
    assert fma32(a, b, -(2.0 ** -80)) == lo
    assert fma32(a, b, 0.0) == lo          # exact tie: even mantissa


def test_exp2_f32_integers_and_monotone():
    assert exp2_f32(np.arange(-140, 120)).tolist() == [float(np.float32(2.0 ** k)) for k in range(-140, 120)]
    x = np.sort(fl32(np.random.default_rng(3).uniform(-30, 5, 5000)))
    e = exp2_f32(x)
    assert np.all(np.diff(e) >= 0)


@pytest.mark.parametrize("v", [0.0, 1.0, -2.5, 3.0e-5])
def test_fl32_identity_on_fp32(v):
    assert fl32(np.float32(v)) == np.float32(v)
