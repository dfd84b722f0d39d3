"""Scalar brute force of the LampAttention forward pass for tiny inputs.

Test infrastructure.  This is a second, independent formulation of the method
of "LampAttention: Look-Ahead Mixed-Precision FlashAttention for Dedicated
Accelerators" (abstract: 8-bit key-query products and exponentials, adaptive
16-bit recompute of sensitive sub-blocks; tables 1-6: sub-blocks of tiles),
under the same readings as ``oracle.lamp`` but sharing none of its code: every
rounding is done here on exact rationals (``fractions.Fraction``), the e4m3
rounding picks the nearest entry of the enumerated code table, and everything
runs in plain Python loops, one entry at a time.  It exists to catch indexing,
broadcasting and rounding mistakes in the vectorised oracle, and is only
usable for a few hundred keys.
"""
import bisect
import math
from fractions import Fraction

LOG2E = 1.4426950408889634


def _floor_log2(a):
    """floor(log2 a) for a positive Fraction, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _round_binary(a, prec, emin):
    """Round a Fraction to a binary format with ``prec`` significant bits and
    smallest normal exponent ``emin`` (nearest, ties to even).  No overflow."""
    if a == 0:
        return Fraction(0)
    sign = -1 if a < 0 else 1
    a = abs(a)
    e = max(_floor_log2(a), emin)
    unit = Fraction(2) ** (e - prec + 1)
    n = a / unit
    q, rem = divmod(n.numerator, n.denominator)
    twice = 2 * rem
    if twice > n.denominator or (twice == n.denominator and q % 2 == 1):
        q += 1
    return sign * q * unit


def to_f32(a):
    """Nearest fp32 value of an exact rational (inf beyond the range)."""
    r = _round_binary(Fraction(a), 24, -126)
    if abs(r) >= Fraction(2) ** 128:
        return math.inf if r > 0 else -math.inf
    return r


def to_bf16(a):
    """Nearest bfloat16 value of an exact rational."""
    return _round_binary(Fraction(a), 8, -126)


def _e4m3_table():
    """Positive finite e4m3fn values, indexed by code 0..126."""
    vals = []
    for code in range(127):
        ef, m = code >> 3, code & 7
        if ef == 0:
            vals.append(Fraction(m, 512))
        else:
            vals.append((1 + Fraction(m, 8)) * Fraction(2) ** (ef - 7))
    return vals


E4M3_TABLE = _e4m3_table()


def to_e4m3(a):
    """Nearest e4m3fn value (ties to the even code), saturating at 448."""
    a = Fraction(a)
    mag = abs(a)
    hi = bisect.bisect_left(E4M3_TABLE, mag)      # first code with value >= mag
    if hi == len(E4M3_TABLE):
        v = E4M3_TABLE[-1]                          # beyond 448: saturate
    elif hi == 0 or E4M3_TABLE[hi] == mag:
        v = E4M3_TABLE[hi]
    else:
        lo = hi - 1
        dl, dh = mag - E4M3_TABLE[lo], E4M3_TABLE[hi] - mag
        if dl < dh or (dl == dh and lo % 2 == 0):
            v = E4M3_TABLE[lo]
        else:
            v = E4M3_TABLE[hi]
    return -v if a < 0 else v


def _exp2_f32(x):
    """fp32 exp2 of an fp32 argument (fp64 pow rounded once more to fp32)."""
    if x == -math.inf:
        return Fraction(0)
    try:
        return to_f32(Fraction(math.pow(2.0, float(x))))
    except OverflowError:
        return math.inf


# The polynomial exp2 of the bit-reproducible variant, step by step on exact
# rationals: clamp at -30, n = rint(x) (ties to even), f = x - n, Horner's
# rule from the degree-5 coefficient down with every multiply-add rounded once
# to fp32, then scaled by 2^n.  The coefficients are the fp32 values
# m * 2^e below (24-bit integer m).
_POLY_C = [Fraction(0xB17215, 2 ** 24), Fraction(0xF5FCD7, 2 ** 26), Fraction(0xE35B27, 2 ** 28),
           Fraction(0x9E7733, 2 ** 30), Fraction(0xAE086A, 2 ** 33)]


def exp2_poly(x):
    """The variant's exp2 of an fp32 value x (a float), as a Fraction."""
    xf = Fraction(-30) if x == -math.inf else max(Fraction(x), Fraction(-30))
    fl = math.floor(xf)
    rest = xf - fl
    n = fl + 1 if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and fl % 2 == 1) else fl
    f = xf - n
    p = _POLY_C[4]
    for c in (_POLY_C[3], _POLY_C[2], _POLY_C[1], _POLY_C[0], Fraction(1)):
        p = to_f32(p * f + c)
    return p * Fraction(2) ** n


def _bf16(bits):
    """Exact value of a bfloat16 bit pattern."""
    bits = int(bits)
    sign = -1 if bits & 0x8000 else 1
    ef = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if ef == 0:
        return sign * Fraction(m, 128) * Fraction(2) ** -126
    return sign * (1 + Fraction(m, 128)) * Fraction(2) ** (ef - 127)


def brute_lamp(q_bits, k_bits, v_bits, causal, window, delta, tau, logit8=False, exp_poly=False):
    """Whole forward pass; returns (out as nested lists of float, mask dict).

    mask[(b, hq, r, t)] = byte for visited tiles only.  ``logit8``: the
    variant whose log2-domain logits are rounded to e4m3 before the running
    max, the exponentials and the second stage read them.  ``exp_poly``: the
    variant whose 8-bit exponentials come from the polynomial exp2.
    """
    B, Hq, S, D = (len(q_bits), len(q_bits[0]), len(q_bits[0][0]), len(q_bits[0][0][0]))
    Hkv = len(k_bits[0])
    G = Hq // Hkv
    q = [[[[_bf16(x) for x in row] for row in h] for h in bb] for bb in q_bits]
    k = [[[[_bf16(x) for x in row] for row in h] for h in bb] for bb in k_bits]
    v = [[[[_bf16(x) for x in row] for row in h] for h in bb] for bb in v_bits]

    def scales(t, b, h):
        a = max(abs(x) for row in t[b][h] for x in row)
        if a == 0:
            return Fraction(1), Fraction(1)
        return to_f32(a / 448), to_f32(Fraction(448) / a)

    def quant(t, b, h):
        _, inv = scales(t, b, h)
        return [[to_e4m3(to_f32(x * inv)) for x in row] for row in t[b][h]]

    L = Fraction(LOG2E / math.sqrt(D))                     # fp64 value, exact
    c16 = to_f32(L)
    T2 = to_f32(Fraction(16 * float(tau) * LOG2E)) if math.isfinite(16 * float(tau) * LOG2E) \
        else (math.inf if tau > 0 else -math.inf)

    def vis(i, j):
        if i >= S or j >= S:
            return False
        if causal and j > i:
            return False
        if window > 0 and i - j >= window:
            return False
        return True

    nT = (S + 63) // 64
    out = [[[[0.0] * D for _ in range(S)] for _ in range(Hq)] for _ in range(B)]
    mask = {}
    for b in range(B):
        for hq in range(Hq):
            hk = hq // G
            q8, k8 = quant(q, b, hq), quant(k, b, hk)
            sq, _ = scales(q, b, hq)
            sk, _ = scales(k, b, hk)
            c8 = to_f32(Fraction(float(sq) * float(sk) * float(L)))   # fp64 product, then fp32
            for r in range(nT):
                rows = [i for i in range(64 * r, 64 * r + 64) if i < S]
                m = {i: -math.inf for i in rows}
                ell = {i: Fraction(0) for i in rows}
                acc_o = {i: [Fraction(0)] * D for i in rows}
                for t in range(nT):
                    keys = list(range(64 * t, 64 * t + 64))
                    if not any(vis(i, j) for i in rows for j in keys):
                        continue
                    acc8, s2 = {}, {}
                    for i in rows:
                        for j in keys:
                            if vis(i, j):
                                a = sum(q8[i][d] * k8[j][d] for d in range(D))
                                acc8[i, j] = to_f32(a)
                                s2[i, j] = to_f32(acc8[i, j] * c8)
                                if logit8:
                                    s2[i, j] = to_e4m3(s2[i, j])
                    m_new = {}
                    for i in rows:
                        cand = [s2[i, j] for j in keys if (i, j) in s2]
                        m_new[i] = max([m[i]] + cand) if cand else m[i]
                    p, flags = {}, [False] * 4
                    for (i, j), a in acc8.items():
                        arg = s2[i, j] - m_new[i] if logit8 else a * c8 - m_new[i]
                        e = exp2_poly(to_f32(arg)) if exp_poly else _exp2_f32(to_f32(arg))
                        p8 = to_e4m3(e)
                        p[i, j] = p8
                        active = (delta <= 0) or (p8 >= Fraction(delta))
                        if active and abs(s2[i, j]) >= T2:
                            flags[(j - 64 * t) // 16] = True
                    for (i, j) in list(p):
                        c = (j - 64 * t) // 16
                        if flags[c]:
                            a16 = to_f32(sum(q[b][hq][i][d] * k[b][hk][j][d] for d in range(D)))
                            p[i, j] = to_bf16(_exp2_f32(to_f32(a16 * c16 - m_new[i])))
                    for i in rows:
                        if m_new[i] == -math.inf:
                            continue
                        alpha = Fraction(0) if m[i] == -math.inf else \
                            Fraction(math.pow(2.0, float(m[i] - m_new[i])))
                        ell[i] = alpha * ell[i]
                        acc_o[i] = [alpha * o for o in acc_o[i]]
                        for j in keys:
                            if (i, j) in p:
                                ell[i] += p[i, j]
                                vj = v[b][hk][j]
                                acc_o[i] = [o + p[i, j] * vj[d] for d, o in enumerate(acc_o[i])]
                        m[i] = m_new[i]
                    mask[b, hq, r, t] = 0x80 | sum(int(f) << c for c, f in enumerate(flags))
                for i in rows:
                    out[b][hq][i] = [float(to_f32(o / ell[i])) for o in acc_o[i]]
    return out, mask


def brute_decode(q_bits, k_bits, v_bits, causal, window, delta, tau, tiles_per_split):
    """Split-KV decode, one entry at a time in exact rationals.

    q_bits [B][Hq][Sq][D] are the queries at positions Skv - Sq .. Skv - 1 of
    k_bits / v_bits [B][Hkv][Skv][D].  The KV tiles are cut into runs of
    ``tiles_per_split``; each run is processed from an empty state and the
    runs are merged exactly.  Returns (out as nested lists of float, mask
    dict {(b, hq, t): byte} for visited tiles).
    """
    B, Hq, Sq, D = (len(q_bits), len(q_bits[0]), len(q_bits[0][0]), len(q_bits[0][0][0]))
    Hkv, Skv = len(k_bits[0]), len(k_bits[0][0])
    G = Hq // Hkv
    q = [[[[_bf16(x) for x in row] for row in h] for h in bb] for bb in q_bits]
    k = [[[[_bf16(x) for x in row] for row in h] for h in bb] for bb in k_bits]
    v = [[[[_bf16(x) for x in row] for row in h] for h in bb] for bb in v_bits]

    def scales(rows):
        a = max(abs(x) for row in rows for x in row)
        if a == 0:
            return Fraction(1), Fraction(1)
        return to_f32(a / 448), to_f32(Fraction(448) / a)

    L = Fraction(LOG2E / math.sqrt(D))
    c16 = to_f32(L)
    T2 = to_f32(Fraction(16 * float(tau) * LOG2E)) if math.isfinite(16 * float(tau) * LOG2E) \
        else (math.inf if tau > 0 else -math.inf)
    off = Skv - Sq

    def seen(i, j):
        """Query row i (position off + i) sees key j."""
        p = off + i
        if j >= Skv or (causal and j > p) or (window > 0 and p - j >= window):
            return False
        return True

    nT = (Skv + 63) // 64
    out = [[None] * Hq for _ in range(B)]
    mask = {}
    for b in range(B):
        for hq in range(Hq):
            hk = hq // G
            sq, iq = scales(q[b][hq])
            sk, ik = scales(k[b][hk])
            q8 = [[to_e4m3(to_f32(x * iq)) for x in row] for row in q[b][hq]]
            k8 = [[to_e4m3(to_f32(x * ik)) for x in row] for row in k[b][hk]]
            c8 = to_f32(Fraction(float(sq) * float(sk) * float(L)))
            runs = []                       # per split: {i: (m, ell, acc)}
            for t0 in range(0, nT, tiles_per_split):
                m = {i: -math.inf for i in range(Sq)}
                ell = {i: Fraction(0) for i in range(Sq)}
                acc = {i: [Fraction(0)] * D for i in range(Sq)}
                for t in range(t0, min(t0 + tiles_per_split, nT)):
                    keys = range(64 * t, 64 * t + 64)
                    pairs = [(i, j) for i in range(Sq) for j in keys if seen(i, j)]
                    if not pairs:
                        continue
                    s2 = {(i, j): to_f32(to_f32(sum(q8[i][d] * k8[j][d] for d in range(D))) * c8)
                          for (i, j) in pairs}
                    m_new = dict(m)
                    for (i, j), x in s2.items():
                        m_new[i] = max(m_new[i], x)
                    p, flags = {}, [False] * 4
                    for (i, j) in pairs:
                        a8 = to_f32(sum(q8[i][d] * k8[j][d] for d in range(D)))
                        p8 = to_e4m3(_exp2_f32(to_f32(a8 * c8 - m_new[i])))
                        p[i, j] = p8
                        if ((delta <= 0) or (p8 >= Fraction(delta))) and abs(s2[i, j]) >= T2:
                            flags[(j - 64 * t) // 16] = True
                    for (i, j) in pairs:
                        if flags[(j - 64 * t) // 16]:
                            a16 = to_f32(sum(q[b][hq][i][d] * k[b][hk][j][d] for d in range(D)))
                            p[i, j] = to_bf16(_exp2_f32(to_f32(a16 * c16 - m_new[i])))
                    for i in range(Sq):
                        if m_new[i] == -math.inf:
                            continue
                        f = Fraction(0) if m[i] == -math.inf else \
                            Fraction(math.pow(2.0, float(m[i] - m_new[i])))
                        ell[i] *= f
                        acc[i] = [f * o for o in acc[i]]
                        for j in keys:
                            if (i, j) in p:
                                ell[i] += p[i, j]
                                acc[i] = [o + p[i, j] * v[b][hk][j][d] for d, o in enumerate(acc[i])]
                        m[i] = m_new[i]
                    mask[b, hq, t] = 0x80 | sum(int(x) << c for c, x in enumerate(flags))
                runs.append((m, ell, acc))
            rows = []
            for i in range(Sq):
                top = max(r[0][i] for r in runs)
                num, den = [Fraction(0)] * D, Fraction(0)
                for m, ell, acc in runs:
                    if m[i] == -math.inf:
                        continue
                    w = Fraction(math.pow(2.0, float(m[i] - top)))
                    den += w * ell[i]
                    num = [n + w * o for n, o in zip(num, acc[i])]
                rows.append([float(to_f32(n / den)) for n in num])
            out[b][hq] = rows
    return out, mask
