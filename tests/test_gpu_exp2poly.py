"""The bit-reproducible variant (lamp_attn_fwd_exp2poly) against the oracle's
exp_poly reading, through the C ABI (needs an MI355X).

* the device polynomial exp2 equals the oracle's bit for bit over millions of
  arguments (every integer and half-integer, their fp32 neighbours, random
  values, and a dense run around the first-stage threshold of delta = 2^-8);
* given the device's own 8-bit accumulators, every 8-bit weight that entered
  P.V equals the oracle's e4m3(P(fma(acc, c8, -m))) exactly, with no window;
* the forward pass on small shapes under the parity protocol, and the
  Qwen3-8B-shaped workload at full size on sampled units.
"""
import numpy as np
import pytest
import torch

from inputs import make_config_inputs, make_inputs
from oracle import lamp as L
from oracle.formats import bf16_bits_to_f64, exp2_poly_f32, fl32, fma32, round_e4m3

from parity import assert_parity, compare, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import mixed_precision_attention_lamp_amd as lamp
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lamp.load()
    yield
    torch.cuda.synchronize()


def _arguments():
    rng = np.random.default_rng(70)
    ints = np.arange(-40, 1, dtype=np.float64)
    halves = (ints[:-1] + 0.5).astype(np.float32)
    pts = [ints, halves.astype(np.float64)]
    up, dn = halves.copy(), halves.copy()
    for _ in range(4):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        pts += [up.astype(np.float64), dn.astype(np.float64)]
    # every fp32 value within 2^14 ulps of -8 (the first-stage threshold of
    # delta = 2^-8 lies just below it)
    base = np.float32(-8.0).view(np.int32)
    pts.append(np.arange(base - (1 << 14), base + (1 << 14), dtype=np.int32).view(np.float32).astype(np.float64))
    pts += [rng.uniform(-40, 2.0 ** -10, 1 << 21), rng.uniform(-1, 2.0 ** -10, 1 << 20),
            rng.uniform(-2.0 ** -10, 2.0 ** -10, 1 << 18)]
    return fl32(np.concatenate(pts))


def test_device_exp2poly_bit_exact():
    import mixed_precision_attention_lamp_amd as lamp
    x = _arguments()
    say(f"[exp2poly] {x.size} arguments in [{x.min():.1f}, {x.max():.2e}]")
    xd = torch.from_numpy(x.astype(np.float32)).cuda()
    yd = torch.empty_like(xd)
    lamp.lamp_debug_exp2poly(xd, yd)
    torch.cuda.synchronize()
    got = yd.cpu().numpy().astype(np.float64)
    want = exp2_poly_f32(x)
    bad = np.nonzero(got != want)[0]
    say(f"[exp2poly] device vs oracle: {bad.size} differ; max rel error vs 2^x "
        f"{np.max(np.abs(want / np.exp2(np.maximum(x, -30.0)) - 1)):.3e}")
    assert bad.size == 0, [(x[i], got[i], want[i]) for i in bad[:5]]


DUMP = [
    # B, Hq, Hkv, S, D, causal, window, delta, tau, structure, seed
    (1, 4, 2, 260, 128, 1, 0, 2 ** -8, 2 ** -1, "channels", 71),
    (1, 2, 1, 200, 64, 0, 0, 2 ** -8, 2 ** -3, "sinks", 72),
    (1, 2, 2, 150, 256, 1, 70, 2 ** -4, 2 ** -1, "channels", 73),
    (1, 2, 1, 130, 128, 1, 0, 2 ** -8, np.inf, "channels+drift", 74),
]


@pytest.mark.parametrize("case", DUMP)
def test_dump_weights_bit_exact(case):
    """From the device's own accumulators, the oracle's steps (running max,
    x = fma(acc, c8, -m), e4m3 of the polynomial exp2) give every 8-bit weight
    that the device used, bit for bit."""
    import mixed_precision_attention_lamp_amd as lamp
    B, Hq, Hkv, S, D, causal, window, delta, tau, st, seed = case
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, st)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    nT = L.n_tiles(S)
    out = torch.empty((B, Hq, S, D), dtype=torch.float32, device="cuda")
    mask = torch.empty((B, Hq, nT, nT), dtype=torch.uint8, device="cuda")
    acc = torch.full((B, Hq, S, S), float("nan"), dtype=torch.float32, device="cuda")
    pw = torch.zeros((B, Hq, S, S), dtype=torch.int16, device="cuda")
    lamp.lamp_debug_attn_dump_exp2poly(qd, kd, vd, out, causal, window, delta, tau, mask, acc, pw)
    torch.cuda.synchronize()
    acc_g = acc.cpu().numpy().astype(np.float64)
    p_g = bf16_bits_to_f64(pw.cpu().numpy().view(np.uint16))
    mask_g = mask.cpu().numpy()
    ctx = L.prepare(q, k, v, causal, window, delta, tau, exp_poly=True)
    G = Hq // Hkv
    n_cmp = n_bad = 0
    for (b, h, r) in L.all_units(B, Hq, S):
        rows = np.arange(r * 64, min(r * 64 + 64, S))
        c8, _ = L.logit_constants(D, ctx["sq"][b, h], ctx["sk"][b, h // G])
        m = np.full(rows.size, -np.inf)
        for t in range(nT):
            cols = np.arange(t * 64, min(t * 64 + 64, S))
            vis = L.visible(rows, cols, causal, window)
            if not vis.any():
                continue
            ga = acc_g[b, h][np.ix_(rows, cols)]
            s2 = np.where(vis, fl32(ga * c8), -np.inf)
            m = np.maximum(m, s2.max(axis=1))
            safe = np.where(np.isfinite(m), m, 0.0)
            x = fma32(np.where(vis, ga, 0.0), c8, -safe[:, None])
            p8 = round_e4m3(exp2_poly_f32(x))
            flags = int(mask_g[b, h, r, t])
            eight = vis.copy()
            for c in range(4):
                if (flags >> c) & 1:
                    eight[:, c * 16:(c + 1) * 16] = False
            gp = p_g[b, h][np.ix_(rows, cols)]
            n_cmp += int(eight.sum())
            n_bad += int((eight & (gp != p8)).sum())
    say(f"[exp2poly-dump] {case}: 8-bit weights compared {n_cmp}, differing {n_bad}")
    assert n_cmp > 0
    assert n_bad == 0


SMALL = [
    (1, 4, 2, 260, 128, 1, 0, 2 ** -8, 2 ** -1, "channels", 81),
    (2, 8, 1, 300, 64, 1, 0, 2 ** -8, 2 ** -1, "sinks", 82),
    (1, 4, 4, 190, 128, 1, 64, 2 ** -4, 2 ** -2, "channels+drift", 83),
    (1, 2, 1, 200, 256, 1, 0, 2 ** -8, 2 ** -1, "channels", 84),
    (1, 3, 1, 129, 64, 0, 0, 0.0, 2 ** -3, "channels", 85),
    (1, 2, 1, 70, 128, 1, 0, 2 ** -8, np.inf, "sinks", 86),
    (1, 1, 1, 1, 64, 1, 0, 2 ** -8, 2 ** -1, "plain", 87),
    (1, 8, 1, 140, 128, 1, 0, 2 ** -8, 2 ** -2, "sinks", 89),          # G = 8
    (2, 2, 2, 257, 64, 1, 100, 2 ** -4, 2 ** -1, "channels+drift", 90),  # D = 64, window, ragged
    (1, 2, 1, 64, 128, 1, 0, 0.0, 0.0, "channels", 91),                 # one tile, all 16-bit
    (1, 2, 2, 190, 256, 0, 0, 2 ** -8, 2 ** -3, "sinks", 92),           # D = 256, non-causal
]


@pytest.mark.parametrize("case", SMALL)
def test_exp2poly_parity_small(case):
    B, Hq, Hkv, S, D, causal, window, delta, tau, st, seed = case
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, st)
    rep = compare(q, k, v, causal, window, delta, tau, label=f"exp2poly {case}", exp_poly=True)
    assert_parity(rep)


def test_exp2poly_deterministic():
    """Two calls on the same inputs give the same bits (outputs and mask)."""
    q, k, v = make_inputs(1, 4, 2, 300, 128, 93, "channels")
    import mixed_precision_attention_lamp_amd as lamp
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o1, m1 = lamp.attention(qd, kd, vd, True, 0, 2 ** -8, 2 ** -1, exp_poly=True)
    o2, m2 = lamp.attention(qd, kd, vd, True, 0, 2 ** -8, 2 ** -1, exp_poly=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(m1, m2)


@pytest.mark.parametrize("name,n", [("qwen3-8b", 8), ("gemma3-12b", 4)])
def test_exp2poly_parity_full_size(name, n):
    """Full-size workloads in one call each, sampled units against the oracle."""
    q, k, v, cfg = make_config_inputs(name)
    B, Hq, S, _ = q.shape
    nT = L.n_tiles(S)
    rng = np.random.default_rng(88)
    units = sorted({(0, 0, nT - 1), (B - 1, Hq - 1, 0)} |
                   {(int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(nT))) for _ in range(n - 2)})
    rep = compare(q, k, v, cfg["causal"], cfg["window"], 2 ** -8, 2 ** -1, units=units,
                  label=f"exp2poly {name}", exp_poly=True)
    assert_parity(rep)
