"""Software rounding to the formats the method uses (oracle; test infrastructure).

The method of "LampAttention: Look-Ahead Mixed-Precision FlashAttention for
Dedicated Accelerators" (abstract) computes key-query products and
exponentials with 8-bit number formats and redoes sensitive sub-blocks with
16-bit ones.  The pages do not name the formats; the readings used here are

* 8-bit  = OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7),
  3 fraction bits, no infinities, largest finite 448, subnormal spacing 2^-9.
  Round to nearest, ties to even; out-of-range magnitudes saturate to 448.
* 16-bit = bfloat16: the top 16 bits of an IEEE fp32, round to nearest even.
* all intermediate arithmetic that a GPU would do in fp32 is modelled as the
  exact result rounded once to fp32 (``fl32``).

Every function works on NumPy fp64 arrays that carry exact values.
"""
from fractions import Fraction

import numpy as np

E4M3_MAX = 448.0


def fl32(x):
    """Round exact fp64 values to the nearest fp32 (ties to even), returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_e4m3(y):
    """Round to the e4m3fn grid: nearest, ties to even, saturating at +-448.

    Within the binade [2^e, 2^(e+1)) the grid spacing is 2^(e-3); below 2^-6
    (the smallest normal) the spacing stays 2^-9 (subnormals).  Dividing by a
    power of two is exact, so ``rint`` (half to even) on the scaled value is
    the round-to-nearest-even of the format.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, k = np.frexp(a)                     # a = f * 2^k, f in [0.5, 1)
    e = np.maximum(k - 1, -6)              # binade exponent, floored at 2^-6
    q = np.ldexp(1.0, e - 3)               # grid spacing in that binade
    r = np.rint(a / q) * q
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, y)


def e4m3_encode(y):
    """Byte codes of values already on the e4m3fn grid (sign bit kept for -0)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, k = np.frexp(a)
    e = k - 1
    sub = a < 2.0 ** -6
    mant_sub = np.rint(a * 2.0 ** 9)                       # 0..7 (8 == 2^-6 is normal)
    exp_field = np.where(sub, 0, e + 7)
    mant_norm = np.rint((np.ldexp(a, -e) - 1.0) * 8.0)
    code = np.where(sub, mant_sub, exp_field * 8 + mant_norm).astype(np.int64)
    code = np.where(np.signbit(y), code | 0x80, code)
    return code.astype(np.uint8)


def e4m3_decode(codes):
    """Values of e4m3fn byte codes (0x7F / 0xFF are NaN)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 0x7
    v = np.where(ef == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, ef - 7))
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return s * v


def bf16_bits_to_f64(bits):
    """Exact values of bfloat16 bit patterns (uint16)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(x):
    """Round fp32 values to bfloat16, nearest even; returns exact fp64 values.

    The input is first rounded to fp32 (a no-op for values that already are);
    the 16 low bits of the fp32 pattern are then rounded away.
    """
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    return bf16_bits_to_f64(r.astype(np.uint16))


def _f32_neighbours(d):
    """The two fp32 values bracketing fp64 ``d`` (equal if d is an fp32)."""
    r = d.astype(np.float32)
    rd = r.astype(np.float64)
    up = np.nextafter(r, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(r, np.float32(-np.inf)).astype(np.float64)
    lo = np.where(rd <= d, rd, dn)
    hi = np.where(rd >= d, rd, up)
    return lo, hi


def fma32(a, b, c):
    """fp32 fused multiply-add: the exact a*b + c rounded once to fp32.

    a, b, c must be fp32 values (held in fp64).  a*b is exact in fp64
    (24 + 24 significant bits); the addition can round in fp64, and a second
    rounding to fp32 is then wrong only when the fp64 sum lands exactly on an
    fp32 midpoint.  Those (rare) entries are redone in exact rational
    arithmetic.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    a, b, c = np.broadcast_arrays(a, b, c)
    shape = a.shape
    a, b, c = (np.atleast_1d(z) for z in (a, b, c))
    d = a * b + c
    out = fl32(d)
    finite = np.isfinite(d)
    lo, hi = _f32_neighbours(np.where(finite, d, 0.0))
    tie = finite & (lo != hi) & (d - lo == hi - d)
    if np.any(tie):
        out = out.copy()
        for idx in zip(*np.nonzero(tie)):
            exact = Fraction(float(a[idx])) * Fraction(float(b[idx])) + Fraction(float(c[idx]))
            mid = Fraction(float(d[idx]))
            if exact > mid:
                out[idx] = hi[idx]
            elif exact < mid:
                out[idx] = lo[idx]
            # exact == mid: the fp32 round-to-even of d is already right
    return out.reshape(shape)


# The polynomial exp2 of the bit-reproducible variant (abstract: the
# exponentials are taken in 8-bit formats; the pages do not say how they are
# evaluated).  Read here as a function defined by its steps, each an fp32
# operation rounded to nearest-even, so that any implementation of the same
# steps gives the same bits:
#   x <- max(x, -30)      (2^-30 and everything below it round to 0 in e4m3)
#   n = rint(x)           (ties to even), f = x - n (exact, |f| <= 1/2)
#   p = 1 + f(c1 + f(c2 + f(c3 + f(c4 + f c5))))  by Horner's rule, every step
#       one fused multiply-add rounded once to fp32, innermost first
#   result = p * 2^n      (exact: p in [0.7, 1.5], n >= -30, so it stays normal)
# c1..c5 are a minimax fit of the relative error of 2^f on [-1/2, 1/2] with
# the constant term fixed at 1, each rounded to fp32; the fp32 evaluation
# stays within 2^-22 of 2^x, relative.
EXP2_POLY_XMIN = -30.0
EXP2_POLY_C = tuple(float.fromhex(h) for h in (
    "0x1.62e42ap-1", "0x1.ebf9aep-3", "0x1.c6b64ep-5", "0x1.3cee66p-7", "0x1.5c10d4p-10"))


def exp2_poly_f32(x):
    """The polynomial exp2 above, on fp32 arguments (held in fp64); NaN
    arguments take the clamp's value, as an IEEE maxNum does."""
    x = np.fmax(np.asarray(x, dtype=np.float64), EXP2_POLY_XMIN)
    n = np.rint(x)
    f = x - n
    c1, c2, c3, c4, c5 = EXP2_POLY_C
    p = fma32(c5, f, c4)
    for c in (c3, c2, c1, 1.0):
        p = fma32(p, f, c)
    return np.ldexp(p, n.astype(np.int64))


def exp2_f32(x):
    """fp32 exp2: the fp64 exp2 of an fp32 argument, rounded to fp32.

    This is the correctly rounded fp32 result except when exp2(x) lies within
    about 2^-53 (relative) of an fp32 midpoint.
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", under="ignore"):
        return fl32(np.exp2(x))
