"""Pins of the oracle's polynomial exp2 (``formats.exp2_poly_f32``) and of the
variant that takes the 8-bit exponentials from it (``exp_poly``).  No GPU.

The abstract of "LampAttention: Look-Ahead Mixed-Precision FlashAttention for
Dedicated Accelerators" has the exponentials taken in 8-bit formats without
saying how they are evaluated.  The variant defines the exponential by its
fp32 steps (clamp, split x = n + f, a degree-5 Horner polynomial of fused
multiply-adds, scale by 2^n), so that every implementation of those steps
gives the same bits.  Pinned here by

* closed forms: integer arguments give exact powers of two; the clamp;
* the mathematics: the result is within 2^-22 of 2^x (relative) over the
  whole argument range, and a dropped, negated or swapped coefficient breaks
  that bound (planted in a copy of the oracle's coefficients);
* the scalar exact-rational brute force (oracle.brute, separate code and a
  separately written coefficient table), bit for bit;
* its e4m3 rounding: the same 8-bit weight as the correctly rounded exp2
  except within the bound of an e4m3 rounding midpoint;
* the forward pass: the brute force with the variant equals the oracle's.
"""
import numpy as np
import pytest

from inputs import make_inputs
from oracle import brute
from oracle import formats as F
from oracle import lamp as L


def _f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _args(n_random, seed):
    """fp32 arguments over [-32, 2^-10]: random, the integers, the half
    integers (ties of the rounding of n) and their fp32 neighbours."""
    rng = np.random.default_rng(seed)
    ints = np.arange(-32, 1, dtype=np.float64)
    halves = ints[:-1] + 0.5
    pts = [ints, halves, rng.uniform(-32, 2.0 ** -10, n_random), rng.uniform(-1, 2.0 ** -10, n_random // 4)]
    h32 = halves.astype(np.float32)
    up, dn = h32.copy(), h32.copy()
    for _ in range(3):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        pts += [up.astype(np.float64), dn.astype(np.float64)]
    return _f32(np.concatenate(pts))


def test_integer_arguments_and_clamp():
    n = np.arange(-30, 1, dtype=np.float64)
    assert np.array_equal(F.exp2_poly_f32(n), np.exp2(n))
    low = np.array([-30.5, -31.0, -100.0, -1e30, -np.inf])
    assert np.all(F.exp2_poly_f32(low) == 2.0 ** -30)
    # rint ties to even: -0.5 -> n = 0, f = -0.5; -1.5 -> n = -2, f = 0.5
    a, b = F.exp2_poly_f32(np.array([-0.5, -1.5]))
    assert abs(a / 2 ** -0.5 - 1) < 2 ** -22 and abs(b / 2 ** -1.5 - 1) < 2 ** -22


def _max_rel_error(coeffs=None, n=400_000, seed=3):
    x = _args(n, seed)
    x = x[x >= -30]
    if coeffs is None:
        y = F.exp2_poly_f32(x)
    else:
        saved = F.EXP2_POLY_C
        try:
            F.EXP2_POLY_C = tuple(coeffs)
            y = F.exp2_poly_f32(x)
        finally:
            F.EXP2_POLY_C = saved
    return float(np.max(np.abs(y / np.exp2(x) - 1.0)))


def test_relative_error_bound():
    err = _max_rel_error()
    assert err <= 2.0 ** -22, err


def test_planted_mistakes_break_the_bound():
    c = list(F.EXP2_POLY_C)
    mutants = []
    for k in range(5):
        d = c.copy()
        d[k] = 0.0                      # a dropped term
        mutants.append(d)
        d = c.copy()
        d[k] = -c[k]                    # a wrong sign
        mutants.append(d)
    for k in range(4):
        d = c.copy()
        d[k], d[k + 1] = c[k + 1], c[k]  # two coefficients transposed
        mutants.append(d)
    mutants.append([c[0] * (1 + 2.0 ** -16)] + c[1:])   # a perturbed leading coefficient
    for d in mutants:
        assert _max_rel_error(d, n=20_000) > 2.0 ** -22, d


def test_brute_force_bit_for_bit():
    x = _args(3000, 4)
    want = np.array([float(brute.exp2_poly(float(v))) for v in x])
    got = F.exp2_poly_f32(x)
    assert np.array_equal(got, want), x[np.nonzero(got != want)[0][:5]]


def test_e4m3_weights_agree_with_the_correctly_rounded_exp2():
    """The 8-bit weight of the polynomial equals that of the correctly rounded
    exp2 unless 2^x lies within 2^-22 (relative) of an e4m3 midpoint."""
    x = _args(1_000_000, 5)
    x = x[x <= 0]
    p = F.round_e4m3(F.exp2_poly_f32(x))
    e = np.exp2(x)
    q = F.round_e4m3(F.exp2_f32(x))
    codes = np.array([c for c in range(127)], dtype=np.uint8)
    grid = np.unique(F.e4m3_decode(codes))
    mids = (grid[:-1] + grid[1:]) / 2
    j = np.clip(np.searchsorted(mids, e), 1, mids.size - 1)
    near = np.minimum(np.abs(e - mids[j - 1]), np.abs(e - mids[j])) <= 2.0 ** -22 * e
    assert np.all((p == q) | near)
    assert int((p != q).sum()) <= int(near.sum())


def test_variant_close_to_the_default_reading():
    """On activation-like inputs the variant's 8-bit weights equal the
    default reading's in all but a handful of entries."""
    q, k, v = make_inputs(1, 2, 1, 200, 64, 61, "channels")
    ctx0 = L.prepare(q, k, v, True, 0, 2.0 ** -8, 2.0 ** -1)
    ctx1 = L.prepare(q, k, v, True, 0, 2.0 ** -8, 2.0 ** -1, exp_poly=True)
    n, diff = 0, 0
    for (b, h, r) in L.all_units(1, 2, 200):
        t0, t1 = [], []
        L.run_unit(ctx0, b, h, r, trace=t0)
        L.run_unit(ctx1, b, h, r, trace=t1)
        for a, c in zip(t0[:-1], t1[:-1]):
            n += int(a["vis"].sum())
            diff += int((a["vis"] & (a["p8"] != c["p8"])).sum())
    assert diff <= max(2, n // 10000), (diff, n)


@pytest.mark.slow
def test_brute_force_equals_oracle_exp_poly():
    q, k, v = make_inputs(1, 2, 1, 70, 64, 62, "sinks")
    bo, bm = brute.brute_lamp(q.tolist(), k.tolist(), v.tolist(), 1, 0, 2.0 ** -8, 2.0 ** -2, exp_poly=True)
    out, mask = L.lamp_forward(q, k, v, True, 0, 2.0 ** -8, 2.0 ** -2, exp_poly=True)
    nT = mask.shape[-1]
    for h in range(2):
        for r in range(nT):
            for t in range(nT):
                assert int(mask[0, h, r, t]) == bm.get((0, h, r, t), 0), (h, r, t)
    assert np.abs(out - np.array(bo)).max() <= 4e-7 * max(1.0, np.abs(out).max())
