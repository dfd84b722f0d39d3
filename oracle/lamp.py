"""LampAttention forward pass, step by step (oracle; test infrastructure).

Source: "LampAttention: Look-Ahead Mixed-Precision FlashAttention for
Dedicated Accelerators".  The abstract fixes the pipeline: a FlashAttention
that sums key-query products and takes exponentials with 8-bit number
formats, then finds the sensitive sub-blocks adaptively and redoes them with
16-bit ones.  The title calls the identification
"look-ahead".  Tables 1-6 count "16-bit sub-blocks per tile" (0 / 1 / 2+), so
the decision unit is a sub-block of a tile.  Every table and figure caption
runs the method with two parameters, delta = 2^-8 and tau = 2^-1; figures 6
and 7 contrast delta = 2^-8 with a "disabled first stage", so delta belongs to
a first stage of the test and tau to a second.

The pages give no formula, format or tile size.  The readings taken here
(each one a plain choice the rest of the pages supports):

* geometry: 64 x 64 tiles of (query rows, keys), each split into four
  64 x 16 sub-blocks; KV tiles of a row block are visited in ascending order;
* 8-bit format e4m3fn for Q, K and the exponentials; per-(batch, head)
  amax/448 scales for Q and K; the 8-bit key-query products are summed
  exactly and rounded once to fp32 (no 8-bit accumulator exists on the GPU,
  and the logit itself is not re-rounded to 8 bits);
* 16-bit format bf16 (the inputs' own format) for the recompute, with its
  exponentials rounded to bf16;
* logits are kept in the log2 domain: s = acc * c with c = log2(e)/sqrt(D)
  times the two scales; the running row max comes from the 8-bit logits only
  (the recompute reuses it, so a 16-bit weight may exceed 1);
* first stage (delta): an entry is active iff its 8-bit exponential p8 >= delta
  (delta <= 0 disables the stage: every visible entry is active);
* second stage (tau): an active entry is sensitive iff its logit magnitude is
  at least T2 = 16 * tau * log2(e) in the log2 domain -- the first-order
  relative error of exp(s) under an 8-bit logit error of relative size 2^-4
  (the e4m3 unit roundoff) is 2^-4 * |s|, compared with tau;
* a sub-block is flagged (recomputed in 16-bit) iff it holds a sensitive entry.

A second, literal reading of the abstract's 8-bit accumulation is kept as a variant
(``logit8``): the log2-domain logit s = fl32(acc * c) is itself rounded to
e4m3 (saturating at 448) before anything uses it.  The running max, the
exponential's argument s8 - m (exact: both are e4m3 values) and the second
stage all read the 8-bit logit; the 16-bit recompute is unchanged.

A third variant (``exp_poly``) makes the 8-bit exponentials bit-reproducible:
they come from ``formats.exp2_poly_f32``, a degree-5 polynomial exp2 defined
by its fp32 steps, instead of the correctly rounded exp2; everything else is
unchanged (the 16-bit recompute keeps the correctly rounded exp2).

Masking: causal (key j visible to query i iff j <= i) and an optional sliding
window W (additionally i - j < W).  GQA: query head hq reads kv head hq // G.
"""
import math

import numpy as np

from .formats import (bf16_bits_to_f64, e4m3_encode, exp2_f32, exp2_poly_f32, fl32, fma32,
                      round_bf16, round_e4m3)

LOG2E = 1.4426950408889634          # fp64 nearest to log2(e)
BR = 64                             # query rows per tile
BC = 64                             # keys per tile
SBW = 16                            # keys per sub-block
NSB = BC // SBW                     # sub-blocks per tile


# --------------------------------------------------------------------------
# Step 1-2: per-head scales and e4m3 quantisation of Q and K
# --------------------------------------------------------------------------
def head_scales(bits):
    """amax scales per (batch, head) of a bf16 tensor [B, H, S, D].

    a = max |x| over the head's slab (exact).  If a == 0 the scale and its
    inverse are 1, otherwise scale = fl32(a / 448) and inv = fl32(448 / a).
    """
    B, H = bits.shape[:2]
    a = np.zeros((B, H))
    for b in range(B):          # one slab at a time keeps the temporaries small
        for h in range(H):
            a[b, h] = np.abs(bf16_bits_to_f64(bits[b, h])).max()
    safe = np.where(a > 0, a, 1.0)
    scale = np.where(a > 0, fl32(safe / 448.0), 1.0)
    inv = np.where(a > 0, fl32(448.0 / safe), 1.0)
    return scale, inv


def quantize(bits):
    """e4m3 quantisation of a bf16 tensor with per-head amax scales.

    x8 = E4M3(fl32(x * inv)).  Returns (values, byte codes, scale, inv).
    """
    x = bf16_bits_to_f64(bits)
    scale, inv = head_scales(bits)
    y = fl32(x * inv[:, :, None, None])
    vals = round_e4m3(y)
    return vals, e4m3_encode(vals), scale, inv


# --------------------------------------------------------------------------
# Step 3: constants of one (batch, query head)
# --------------------------------------------------------------------------
def log2_scale(D):
    """L_D = log2(e) / sqrt(D) in fp64 (the softmax scale in the log2 domain)."""
    return LOG2E / math.sqrt(D)


def logit_constants(D, sq, sk):
    """c8 multiplies the 8-bit accumulator, c16 the 16-bit one (both fp32)."""
    L = log2_scale(D)
    c8 = float(fl32(float(sq) * float(sk) * L))
    c16 = float(fl32(L))
    return c8, c16


def tau_threshold(tau):
    """T2 = fl32(16 * tau * log2 e); +inf disables the second stage, <= 0 passes all."""
    with np.errstate(over="ignore"):
        return float(fl32(16.0 * float(tau) * LOG2E))


# --------------------------------------------------------------------------
# Geometry
# --------------------------------------------------------------------------
def visible(rows, cols, causal, window):
    """vis[i, j] for query indices ``rows`` and key indices ``cols``."""
    i = rows[:, None]
    j = cols[None, :]
    v = np.ones((rows.size, cols.size), dtype=bool)
    if causal:
        v &= j <= i
    if window > 0:
        v &= (i - j) < window
    return v


def n_tiles(S):
    return (S + BC - 1) // BC


# --------------------------------------------------------------------------
# Step 4: the two-stage look-ahead test of one tile
# --------------------------------------------------------------------------
def stage_one(p8, vis, delta):
    """Active entries: visible and (first stage disabled or p8 >= delta)."""
    if delta <= 0:
        return vis.copy()
    return vis & (p8 >= delta)


def stage_two(active, s2, T2):
    """Sensitive entries: active and |s2| >= T2."""
    return active & (np.abs(s2) >= T2)


def subblock_flags(sens):
    """flag[c] = some sensitive entry among keys [16c, 16c + 16) of the tile."""
    n = sens.shape[1]
    return [bool(sens[:, c * SBW:min((c + 1) * SBW, n)].any()) if c * SBW < n else False
            for c in range(NSB)]


def _ulp_step(x, k):
    """Move fp32 values k representable steps (k may be negative)."""
    y = np.asarray(x, dtype=np.float64).astype(np.float32)
    target = np.float32(np.inf) if k > 0 else np.float32(-np.inf)
    for _ in range(abs(k)):
        y = np.nextafter(y, target)
    return y.astype(np.float64)


def fragile_flags(e, s2, vis, delta, T2, k):
    """Per sub-block: could moving each test statistic by k fp32 ulps flip the flag?

    Both stages are monotone in their statistic (the fp32 exponential e and
    |s2|), so the flag computed with every statistic pushed down by k ulps and
    the flag with every statistic pushed up bound all flags reachable by such
    perturbations.
    """
    res = []
    for sgn in (-k, k):
        e_k = _ulp_step(e, sgn)
        s_k = _ulp_step(np.abs(s2), sgn)
        act = stage_one(round_e4m3(e_k), vis, delta)
        res.append(subblock_flags(act & (s_k >= T2)))
    return [lo != hi for lo, hi in zip(*res)]


# --------------------------------------------------------------------------
# The forward pass of one unit (batch b, query head hq, row block r)
# --------------------------------------------------------------------------
def run_unit(ctx, b, hq, r, flag_override=None, trace=None, tiles=None):
    """Process one 64-row query block through its visible KV tiles.

    Returns (out rows fp32 values [n, D], {t: mask byte}).  ``flag_override``
    maps t -> 4-bit flags replacing the computed ones (used to replay a run
    whose flags are given).  ``trace`` (a list) receives per-tile records.
    ``tiles`` restricts the KV tiles visited (default: all, ascending).
    Query row i of the slab sits at sequence position i + q_off (q_off > 0
    when the queries are the last rows of a longer key sequence).
    """
    S, D, G = ctx["S"], ctx["D"], ctx["G"]
    hk = hq // G
    rows = np.arange(r * BR, min(r * BR + BR, ctx["Sq"]))   # query rows of the slab
    pos = rows + ctx["q_off"]                               # their sequence positions
    nr = rows.size
    c8, c16 = logit_constants(D, ctx["sq"][b, hq], ctx["sk"][b, hk])
    T2 = ctx["T2"]
    delta = ctx["delta"]
    q8 = ctx["q8"][b, hq, rows]           # e4m3 values (fp64)
    q16 = ctx["q16"][b, hq, rows]         # bf16 values (fp64)

    m = np.full(nr, -np.inf)              # running row max (8-bit logits, log2 domain)
    ell = np.zeros(nr)                    # running sum of weights (fp64)
    O = np.zeros((nr, D))                 # running weighted sum of V rows (fp64)
    mask = {}
    for t in (tiles if tiles is not None else range(n_tiles(S))):
        cols = np.arange(t * BC, min(t * BC + BC, S))
        vis = visible(pos, cols, ctx["causal"], ctx["window"])
        if not vis.any():
            continue
        k8 = ctx["k8"][b, hk, cols]
        # (a) 8-bit products, summed exactly (all partial sums are multiples of
        #     2^-18 below 2^26, so fp64 holds them exactly), rounded to fp32.
        acc8 = fl32(q8 @ k8.T)
        s32 = f32 = fl32(acc8 * c8)
        if ctx["logit8"]:
            s32 = round_e4m3(f32)            # the 8-bit logit (variant)
        s2 = np.where(vis, s32, -np.inf)
        # (b) running max over the 8-bit logits of this tile
        m_new = np.maximum(m, s2.max(axis=1))
        live = m_new > -np.inf
        safe_m = np.where(live, m_new, 0.0)
        # (c) 8-bit exponentials against the running max
        if ctx["logit8"]:
            x = np.where(vis, fl32(s32 - safe_m[:, None]), -np.inf)
        else:
            x = np.where(vis, fma32(acc8, c8, -safe_m[:, None]), -np.inf)
        with np.errstate(invalid="ignore"):
            e = np.where(vis, exp2_poly_f32(x) if ctx.get("exp_poly") else exp2_f32(x), 0.0)
        p8 = round_e4m3(e)
        # (d) look-ahead test, first and second stage
        active = stage_one(p8, vis, delta)
        sens = stage_two(active, s2, T2)
        flags = subblock_flags(sens)
        if flag_override is not None and t in flag_override:
            flags = [bool((flag_override[t] >> c) & 1) for c in range(NSB)]
        # (e) flagged sub-blocks are recomputed in 16-bit
        p = np.where(vis, p8, 0.0)
        e16 = np.full(p.shape, np.nan)       # fp32 16-bit exponentials (diagnostics)
        for c in range(NSB):
            if not flags[c]:
                continue
            sub = slice(c * SBW, min((c + 1) * SBW, cols.size))
            k16 = ctx["k16"][b, hk, cols[sub]]
            acc16 = fl32(q16 @ k16.T)
            x16 = fma32(acc16, c16, -safe_m[:, None])
            e16[:, sub] = exp2_f32(x16)
            p16 = round_bf16(e16[:, sub])
            p[:, sub] = np.where(vis[:, sub], p16, 0.0)
        # (f) online-softmax rescale and P.V
        alpha = np.where(np.isneginf(m), 0.0, np.exp2(m - safe_m))
        alpha = np.where(live, alpha, 1.0)
        ell = alpha * ell + p.sum(axis=1)
        O = alpha[:, None] * O + p @ ctx["v"][b, hk, cols]
        m = m_new
        # (g) mask byte: bit 7 = tile visited, bit c = sub-block c in 16-bit
        byte = 0x80
        for c in range(NSB):
            byte |= int(flags[c]) << c
        mask[t] = byte
        if trace is not None:
            trace.append(dict(t=t, cols=cols, vis=vis, acc8=acc8, s2=s2, f32=f32, e=e,
                              p8=p8, p=p, e16=e16, flags=flags, m_new=m_new.copy(), T2=T2))
    # Step 5: normalise
    out = fl32(O / ell[:, None])
    if trace is not None:
        trace.append(dict(final=True, m=m, ell=ell, O=O))
    return out, mask


# --------------------------------------------------------------------------
# The 16-bit baseline: plain bf16 FlashAttention, no 8-bit pass
# --------------------------------------------------------------------------
def plain_unit(ctx, b, hq, r, trace=None):
    """One 64-row query block of plain bf16 FlashAttention.

    The "16-bit" baseline of tables 1-6 read as the same tiled kernel with
    every sub-block in 16-bit and no 8-bit pass: logits are the bf16
    products summed exactly and rounded once to fp32, s = fl32(acc * c16);
    the running row max comes from these logits; exponentials
    exp2(fma(acc, c16, -m)) are rounded to bf16; online-softmax rescale and
    P.V as in ``run_unit``.  The mask byte of every visited tile is 0x8F
    (all four sub-blocks in 16-bit).  Returns (out rows, {t: mask byte}).
    """
    S, D, G = ctx["S"], ctx["D"], ctx["G"]
    hk = hq // G
    rows = np.arange(r * BR, min(r * BR + BR, S))
    nr = rows.size
    c16 = float(fl32(log2_scale(D)))
    q16 = ctx["q16"][b, hq, rows]
    m = np.full(nr, -np.inf)
    ell = np.zeros(nr)
    O = np.zeros((nr, D))
    mask = {}
    for t in range(n_tiles(S)):
        cols = np.arange(t * BC, min(t * BC + BC, S))
        vis = visible(rows, cols, ctx["causal"], ctx["window"])
        if not vis.any():
            continue
        acc16 = fl32(q16 @ ctx["k16"][b, hk, cols].T)
        s16 = np.where(vis, fl32(acc16 * c16), -np.inf)
        m_new = np.maximum(m, s16.max(axis=1))
        live = m_new > -np.inf
        safe_m = np.where(live, m_new, 0.0)
        x = np.where(vis, fma32(acc16, c16, -safe_m[:, None]), -np.inf)
        e = np.where(vis, exp2_f32(x), 0.0)
        p = np.where(vis, round_bf16(e), 0.0)
        alpha = np.where(np.isneginf(m), 0.0, np.exp2(m - safe_m))
        alpha = np.where(live, alpha, 1.0)
        ell = alpha * ell + p.sum(axis=1)
        O = alpha[:, None] * O + p @ ctx["v"][b, hk, cols]
        m = m_new
        mask[t] = 0x80 | ((1 << NSB) - 1)
        if trace is not None:
            trace.append(dict(t=t, cols=cols, vis=vis, acc16=acc16, s16=s16, e=e, p=p,
                              m_new=m_new.copy()))
    out = fl32(O / ell[:, None])
    if trace is not None:
        trace.append(dict(final=True, m=m, ell=ell, O=O))
    return out, mask


def plain_forward(q_bits, k_bits, v_bits, causal=True, window=0, units=None):
    """Plain bf16 FlashAttention over ``units`` (default: all); same return
    convention as ``lamp_forward``."""
    ctx = prepare(q_bits, k_bits, v_bits, causal, window, 0.0, 0.0)
    B, Hq, S, D = ctx["B"], ctx["Hq"], ctx["S"], ctx["D"]
    nT = n_tiles(S)
    out = np.full((B, Hq, S, D), np.nan, dtype=np.float32)
    mask = np.zeros((B, Hq, nT, nT), dtype=np.uint8)
    for (b, hq, r) in (units if units is not None else all_units(B, Hq, S)):
        o, mk = plain_unit(ctx, b, hq, r)
        out[b, hq, r * BR:r * BR + o.shape[0]] = o.astype(np.float32)
        for t, byte in mk.items():
            mask[b, hq, r, t] = byte
    return out, mask


# --------------------------------------------------------------------------
# Whole forward pass
# --------------------------------------------------------------------------
class PerHead:
    """Values of a [B, H, S, D] tensor, computed one (batch, head) slab at a
    time on first use and kept.  Indexed like the full array with a leading
    (b, h): ``x[b, h, rows]``.  Nothing but evaluation order differs from
    computing the whole tensor up front: every step here is per head."""

    def __init__(self, slab):
        self._slab = slab
        self._cache = {}

    def __getitem__(self, idx):
        key = (int(idx[0]), int(idx[1]))
        if key not in self._cache:
            self._cache[key] = self._slab(*key)
        return self._cache[key][tuple(idx[2:])]


def prepare(q_bits, k_bits, v_bits, causal, window, delta, tau, logit8=False, exp_poly=False):
    """Scales of Q and K, and per-head access to everything the units read
    (the e4m3 values of Q and K, and the bf16 values of Q, K and V).
    ``logit8`` selects the variant whose log2-domain logits are e4m3 values,
    ``exp_poly`` the one whose 8-bit exponentials use the polynomial exp2.
    Q may hold fewer rows than K and V (decode): they are then the last
    positions of the sequence."""
    B, Hq, Sq, D = q_bits.shape
    Hkv, S = k_bits.shape[1], k_bits.shape[2]
    assert Hq % Hkv == 0 and k_bits.shape == v_bits.shape == (B, Hkv, S, D) and Sq <= S
    sq, iq = head_scales(q_bits)
    sk, ik = head_scales(k_bits)

    def e4m3_slab(bits, inv):
        # the quantisation of step 2 on one head: E4M3(fl32(x * inv))
        return lambda b, h: round_e4m3(fl32(bf16_bits_to_f64(bits[b, h]) * inv[b, h]))

    def bf16_slab(bits):
        return lambda b, h: bf16_bits_to_f64(bits[b, h])

    return dict(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, G=Hq // Hkv, Sq=Sq, q_off=S - Sq,
                causal=bool(causal), window=int(window),
                delta=float(delta), T2=tau_threshold(tau), logit8=bool(logit8), exp_poly=bool(exp_poly),
                q8=PerHead(e4m3_slab(q_bits, iq)), k8=PerHead(e4m3_slab(k_bits, ik)), sq=sq, sk=sk,
                q16=PerHead(bf16_slab(q_bits)), k16=PerHead(bf16_slab(k_bits)),
                v=PerHead(bf16_slab(v_bits)))


def all_units(B, Hq, S):
    nr = n_tiles(S)
    return [(b, h, r) for b in range(B) for h in range(Hq) for r in range(nr)]


def lamp_forward(q_bits, k_bits, v_bits, causal=True, window=0, delta=2.0 ** -8,
                 tau=2.0 ** -1, units=None, flag_override=None, logit8=False, exp_poly=False):
    """The LampAttention forward pass over ``units`` (default: all).

    q_bits [B, Hq, S, D], k_bits / v_bits [B, Hkv, S, D]: bf16 bit patterns.
    Returns (out fp32 [B, Hq, S, D] (rows of units not computed are NaN),
    mask uint8 [B, Hq, nT, nT]).  ``flag_override`` is a mask array of the
    same shape whose low 4 bits replace the computed flags of visited tiles.
    ``logit8``: the variant with e4m3 logits; ``exp_poly``: the variant with
    the polynomial exp2 for the 8-bit exponentials.
    """
    ctx = prepare(q_bits, k_bits, v_bits, causal, window, delta, tau, logit8, exp_poly)
    B, Hq, S, D = ctx["B"], ctx["Hq"], ctx["S"], ctx["D"]
    nT = n_tiles(S)
    out = np.full((B, Hq, S, D), np.nan, dtype=np.float32)
    mask = np.zeros((B, Hq, nT, nT), dtype=np.uint8)
    for (b, hq, r) in (units if units is not None else all_units(B, Hq, S)):
        ov = None
        if flag_override is not None:
            ov = {t: int(flag_override[b, hq, r, t]) & 0xF for t in range(nT)}
        o, mk = run_unit(ctx, b, hq, r, flag_override=ov)
        out[b, hq, r * BR:r * BR + o.shape[0]] = o.astype(np.float32)
        for t, byte in mk.items():
            mask[b, hq, r, t] = byte
    return out, mask


# --------------------------------------------------------------------------
# Decode: a few query rows against a long key sequence, split over KV tiles
# --------------------------------------------------------------------------
def split_tiles(nT, tiles_per_split):
    """The KV-tile ranges of the splits: contiguous, ascending, each
    ``tiles_per_split`` tiles long except possibly the last."""
    return [range(t0, min(t0 + tiles_per_split, nT)) for t0 in range(0, nT, tiles_per_split)]


def merge_splits(parts):
    """Combine per-split (m, ell, O) of the same rows: with M the largest m,
    out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) ell_s (fp64, rounded once
    to fp32).  A split whose running max is -inf (no visible key) weighs 0."""
    M = np.max(np.stack([m for m, _, _ in parts]), axis=0)
    num = np.zeros_like(parts[0][2])
    den = np.zeros_like(parts[0][1])
    for m, ell, O in parts:
        w = np.where(np.isneginf(m), 0.0, np.exp2(np.where(np.isneginf(m), 0.0, m) -
                                                 np.where(np.isneginf(M), 0.0, M)))
        num += w[:, None] * O
        den += w * ell
    with np.errstate(invalid="ignore", divide="ignore"):
        return fl32(num / den[:, None])


def decode_forward(q_bits, k_bits, v_bits, causal=True, window=0, delta=2.0 ** -8, tau=2.0 ** -1,
                   tiles_per_split=None, heads=None, logit8=False):
    """Split-KV decode (reading of the method for a few queries against a
    long key sequence).

    q_bits [B, Hq, Sq, D] holds the queries at the last Sq positions
    (Skv - Sq .. Skv - 1) of k_bits / v_bits [B, Hkv, Skv, D]; Sq <= 64, so
    the Sq rows of a head form one row block (the unit of the look-ahead
    test).  The KV tiles are cut into contiguous splits of
    ``tiles_per_split`` tiles (default: one split).  Each split runs the
    method of ``run_unit`` on its own tiles from an empty state (its own
    running max, sum and output); the splits are then merged exactly
    (``merge_splits``).  Scales are the per-head amax scales of the Sq query
    rows and of all Skv keys.

    Returns (out fp32 [B, Hq, Sq, D] (heads not computed are NaN), mask uint8
    [B, Hq, nT]: 0x80 | flags for visited tiles).
    """
    ctx = prepare(q_bits, k_bits, v_bits, causal, window, delta, tau, logit8)
    B, Hq, Sq, S, D = ctx["B"], ctx["Hq"], ctx["Sq"], ctx["S"], ctx["D"]
    assert Sq <= BR
    nT = n_tiles(S)
    tps = tiles_per_split if tiles_per_split else nT
    out = np.full((B, Hq, Sq, D), np.nan, dtype=np.float32)
    mask = np.zeros((B, Hq, nT), dtype=np.uint8)
    for (b, hq) in (heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]):
        parts = []
        for tr in split_tiles(nT, tps):
            trace = []
            with np.errstate(invalid="ignore", divide="ignore"):
                _, mk = run_unit(ctx, b, hq, 0, trace=trace, tiles=tr)
            fin = trace[-1]
            parts.append((fin["m"], fin["ell"], fin["O"]))
            for t, byte in mk.items():
                mask[b, hq, t] = byte
        out[b, hq] = merge_splits(parts).astype(np.float32)
    return out, mask


# --------------------------------------------------------------------------
# Counters reported with every run (tables 1-6 "16-bit sub-blocks per tile")
# --------------------------------------------------------------------------
def subblock_stats(mask, S, causal, window):
    """Histogram and recompute fractions from a mask, by brute force on vis.

    Returns dict(hist=[n0..n4] over visited tiles, visited_tiles,
    visited_subblocks, flagged_subblocks, visible_entries,
    flagged_entries, r_sb, r_e, pages_buckets=[0, 1, 2+] fractions).
    """
    B, Hq, nT, _ = mask.shape
    hist = np.zeros(5, dtype=np.int64)
    vsb = fsb = ve = fe = 0
    for r in range(nT):
        rows = np.arange(r * BR, min(r * BR + BR, S))
        for t in range(nT):
            cols = np.arange(t * BC, min(t * BC + BC, S))
            vis = visible(rows, cols, causal, window)
            if not vis.any():
                continue
            counts = [int(vis[:, c * SBW:(c + 1) * SBW].sum()) for c in range(NSB)]
            bytes_ = mask[:, :, r, t].astype(np.int64)
            for c in range(NSB):
                if counts[c] == 0:
                    continue
                bit = (bytes_ >> c) & 1
                vsb += B * Hq
                fsb += int(bit.sum())
                ve += counts[c] * B * Hq
                fe += counts[c] * int(bit.sum())
            pc = sum(((bytes_ >> c) & 1) for c in range(NSB))
            for n in range(5):
                hist[n] += int((pc == n).sum())
    vt = int(hist.sum())
    return dict(hist=hist.tolist(), visited_tiles=vt, visited_subblocks=vsb,
                flagged_subblocks=fsb, visible_entries=ve, flagged_entries=fe,
                r_sb=fsb / vsb if vsb else 0.0, r_e=fe / ve if ve else 0.0,
                pages_buckets=[hist[0] / vt, hist[1] / vt, hist[2:].sum() / vt] if vt else [0, 0, 0])
