"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

* device conversions (e4m3 rounding, e4m3 -> bf16, bf16 rounding, exp2)
  against the oracle's software formats;
* the quantisation pass, bit-exact;
* the forward pass on small shapes that span several tiles and a ragged
  tail, every masking mode, GQA groups of 1..8, the endpoints of delta / tau;
* the full Qwen3-8B-shaped workload in the launch configuration the bench
  times, on sampled units;
* exact device-only invariants (determinism, V scaling, batch duplication);
* the device histogram of 16-bit sub-blocks against the oracle's.
"""
import functools

import numpy as np
import pytest
import torch

from inputs import make_config_inputs, make_inputs
from oracle import lamp as L
from oracle.formats import (bf16_bits_to_f64, e4m3_decode, e4m3_encode, exp2_f32, round_bf16,
                            round_e4m3)

from parity import (EPS_ACC8, assert_parity, assert_parity_logit8, assert_parity_plain, compare,
                    compare_logit8, compare_plain, fragile_alternatives, logit8_unit, run_gpu, say,
                    to_device, unit_windows)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import mixed_precision_attention_lamp_amd as lamp
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lamp.load()
    yield
    torch.cuda.synchronize()


# --------------------------------------------------------------------------
# conversions
# --------------------------------------------------------------------------
def _conversion_points():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    grid = np.unique(e4m3_decode(codes))
    mids = (grid[:-1] + grid[1:]) / 2
    pts = [grid, mids]
    m32 = mids.astype(np.float32)
    up, dn = m32.copy(), m32.copy()
    for _ in range(3):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        pts += [up.astype(np.float64), dn.astype(np.float64)]
    rng = np.random.default_rng(20)
    pts += [rng.uniform(0, 1, 1 << 20), rng.uniform(-448, 448, 1 << 18),
            rng.uniform(-2 ** -6, 2 ** -6, 1 << 18)]
    x = np.concatenate(pts).astype(np.float32)
    return x[np.abs(x) <= 448]


def test_device_e4m3_and_bf16_conversions():
    import mixed_precision_attention_lamp_amd as lamp
    x = _conversion_points()
    xd = torch.from_numpy(x).cuda()
    n = x.size
    e8 = torch.empty(n, dtype=torch.uint8, device="cuda")
    e8b = torch.empty(n, dtype=torch.int16, device="cuda")
    b16 = torch.empty(n, dtype=torch.int16, device="cuda")
    ex = torch.empty(n, dtype=torch.float32, device="cuda")
    lamp.lamp_debug_convert(xd, e8, e8b, b16, ex)
    torch.cuda.synchronize()
    want = round_e4m3(x.astype(np.float64))
    got_codes = e8.cpu().numpy()
    bad = np.nonzero(got_codes != e4m3_encode(want))[0]
    say(f"[convert] e4m3 code mismatches {bad.size} of {n}")
    assert bad.size == 0, list(zip(x[bad[:8]], got_codes[bad[:8]], e4m3_encode(want)[bad[:8]]))
    dec = bf16_bits_to_f64(e8b.cpu().numpy().view(np.uint16))
    assert np.array_equal(dec, want)
    gb = bf16_bits_to_f64(b16.cpu().numpy().view(np.uint16))
    assert np.array_equal(gb, round_bf16(x.astype(np.float64)))


def test_device_exp2_error():
    import mixed_precision_attention_lamp_amd as lamp
    x = np.random.default_rng(21).uniform(-40, 0.5, 1 << 20).astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    ex = torch.empty_like(xd)
    lamp.lamp_debug_convert(xd, exp2=ex)
    torch.cuda.synchronize()
    g = ex.cpu().numpy()
    ref = exp2_f32(x.astype(np.float64)).astype(np.float32)
    ulps = np.abs(g.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    say(f"[convert] exp2: max ulp error {ulps.max()}, fraction exact {np.mean(ulps == 0):.4f}")
    assert ulps.max() <= 2


def _fp8_blocks(kind, n, seed):
    """n operand pairs [n, 16, 128] of e4m3 codes: uniformly random finite
    codes, or activation-like rows (N(0, 1) times log-normal channel scales,
    1-3 outlier channels x10 in b, each block scaled to amax 448)."""
    rng = np.random.default_rng(seed)
    if kind == "random":
        finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
        return rng.choice(finite, (n, 16, 128)), rng.choice(finite, (n, 16, 128))
    a = np.empty((n, 16, 128), dtype=np.uint8)
    b = np.empty_like(a)
    for i in range(n):
        sa, sb = rng.lognormal(0, 0.5, 128), rng.lognormal(0, 0.5, 128)
        sb[rng.choice(128, rng.integers(1, 4), replace=False)] *= 10
        x = rng.standard_normal((16, 128)) * sa
        y = rng.standard_normal((16, 128)) * sb
        a[i] = e4m3_encode(round_e4m3(x * (448 / np.abs(x).max())))
        b[i] = e4m3_encode(round_e4m3(y * (448 / np.abs(y).max())))
    return a, b


@pytest.mark.parametrize("kind,n,bound", [("activation-like", 2048, EPS_ACC8), ("random", 1024, 2.0 ** -10.75)])
def test_fp8_accumulation_error(kind, n, bound):
    """The attention kernel's 8-bit Q.K^T instruction against the exact sums of
    its e4m3 products: the error, relative to the largest product of each
    dot product, stays within the window the parity protocol assumes
    (activation-like operands, the workloads' recipe) and within 2^-10.75
    for uniformly random codes (the widest dynamic range)."""
    import mixed_precision_attention_lamp_amd as lamp
    a, b = _fp8_blocks(kind, n, 17 if kind == "random" else 18)
    out = torch.empty((n, 16, 16), dtype=torch.float32, device="cuda")
    lamp.lamp_debug_fp8_dot(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    av, bv = e4m3_decode(a), e4m3_decode(b)
    prod = av[:, :, None, :] * bv[:, None, :, :]          # exact in fp64
    exact = prod.sum(axis=-1)
    maxp = np.abs(prod).max(axis=-1)
    rel = np.where(maxp > 0, np.abs(got - exact) / np.where(maxp > 0, maxp, 1.0), 0.0)
    fl = exact.astype(np.float32).astype(np.float64)
    say(f"[fp8-dot] {kind}: {n * 256} dot products; equal to the exactly rounded sum "
        f"{np.mean(got == fl):.4f}; worst error 2^{np.log2(max(rel.max(), 1e-300)):.2f} of the largest "
        f"product (bound 2^{np.log2(bound):.2f}); mean 2^{np.log2(max(rel.mean(), 1e-300)):.2f}")
    assert np.isfinite(got).all()
    assert rel.max() <= bound


# --------------------------------------------------------------------------
# quantisation
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(1, 1, 1, 256, 64, "sinks", 1), (2, 4, 2, 200, 128, "channels", 30),
                                   (1, 8, 1, 67, 64, "plain", 31), (1, 2, 2, 4096, 128, "channels", 32)])
def test_quantize_bit_exact(shape):
    import mixed_precision_attention_lamp_amd as lamp
    B, Hq, Hkv, S, D, st, seed = shape
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, st)
    q[0, 0, :3] = 0                     # include zero rows
    qd, kd = to_device(q), to_device(k)
    q8 = torch.empty((B, Hq, S, D), dtype=torch.uint8, device="cuda")
    k8 = torch.empty((B, Hkv, S, D), dtype=torch.uint8, device="cuda")
    qs = torch.empty(B * Hq, dtype=torch.float32, device="cuda")
    ks = torch.empty(B * Hkv, dtype=torch.float32, device="cuda")
    lamp.lamp_quantize_qk(qd, kd, q8, k8, qs, ks)
    torch.cuda.synchronize()
    _, qc, sq, _ = L.quantize(q)
    _, kc, sk, _ = L.quantize(k)
    assert np.array_equal(q8.cpu().numpy(), qc)
    assert np.array_equal(k8.cpu().numpy(), kc)
    assert np.array_equal(qs.cpu().numpy().astype(np.float64), sq.reshape(-1))
    assert np.array_equal(ks.cpu().numpy().astype(np.float64), sk.reshape(-1))


# --------------------------------------------------------------------------
# forward pass, small shapes
# --------------------------------------------------------------------------
SMALL = [
    # B, Hq, Hkv, S, D, causal, window, delta, tau, structure, seed
    (1, 1, 1, 256, 64, 1, 0, 2 ** -8, 2 ** -1, "sinks", 1),          # the tiny workload
    (1, 4, 1, 300, 128, 1, 0, 2 ** -8, 2 ** -1, "channels", 40),    # G = 4, ragged tail
    (2, 8, 1, 200, 128, 1, 0, 2 ** -8, 2 ** -3, "channels", 41),    # G = 8
    (1, 4, 2, 190, 64, 1, 0, 2 ** -4, 2 ** -2, "channels", 42),     # G = 2
    (1, 3, 3, 130, 128, 0, 0, 2 ** -8, 2 ** -1, "channels", 43),    # non-causal, G = 1
    (1, 2, 2, 333, 128, 1, 100, 2 ** -8, 2 ** -1, "channels", 44),  # sliding window
    (1, 4, 4, 257, 64, 1, 64, 0.0, 2 ** -2, "channels", 45),        # window, first stage off
    (1, 2, 1, 65, 128, 1, 0, 2 ** -8, 2 ** -1, "sinks", 46),        # one full + one 1-row block
    (1, 1, 1, 1, 64, 1, 0, 2 ** -8, 2 ** -1, "plain", 47),          # S = 1
    (1, 4, 1, 500, 128, 1, 0, 2 ** -8, 2 ** -5, "channels+drift", 48),
    (1, 2, 1, 200, 256, 1, 0, 2 ** -8, 2 ** -1, "channels", 51),    # D = 256, G = 2
    (1, 3, 3, 290, 256, 1, 100, 2 ** -4, 2 ** -2, "channels", 52),  # D = 256, window, G = 1
    (1, 2, 2, 70, 256, 0, 0, 0.0, 0.0, "channels", 53),             # D = 256, all 16-bit
    (1, 4, 4, 129, 256, 1, 0, 0.0, 2 ** -3, "sinks", 54),           # D = 256, first stage off
]


@pytest.mark.parametrize("case", SMALL)
def test_forward_parity_small(case):
    B, Hq, Hkv, S, D, causal, window, delta, tau, st, seed = case
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, st)
    rep = compare(q, k, v, causal, window, delta, tau, label=str(case))
    assert_parity(rep)


@pytest.mark.parametrize("ends", [(2 ** -8, np.inf), (0.0, 0.0), (0.0, np.inf), (2 ** -4, 2 ** -5)])
def test_forward_parity_endpoints(ends):
    delta, tau = ends
    q, k, v = make_inputs(1, 4, 2, 260, 128, 50, "channels")
    rep = compare(q, k, v, 1, 0, delta, tau, label=f"endpoint {ends}")
    assert_parity(rep)
    _, mask = run_gpu(q, k, v, 1, 0, delta, tau)
    st = L.subblock_stats(mask, 260, True, 0)
    if tau == np.inf:
        assert st["flagged_subblocks"] == 0
    if delta <= 0 and tau <= 0:
        assert st["flagged_subblocks"] == st["visited_subblocks"]


# --------------------------------------------------------------------------
# per-entry dumps: 8-bit accumulators and the weights that enter P.V
# --------------------------------------------------------------------------
DUMP = [SMALL[0], SMALL[1], SMALL[5], (1, 3, 3, 130, 64, 0, 0, 0.0, 2 ** -2, "channels", 49),
        (1, 2, 1, 260, 128, 1, 0, 0.0, 0.0, "channels", 50), SMALL[11]]


@pytest.mark.parametrize("case", DUMP)
def test_dump_accumulators_and_weights(case):
    """The FP8 matrix-core accumulators stay within the accumulation bound the
    parity protocol assumes, and every weight that differs from the oracle's
    is one whose exponential lies within its window of a rounding midpoint."""
    import mixed_precision_attention_lamp_amd as lamp
    B, Hq, Hkv, S, D, causal, window, delta, tau, st, seed = case
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, st)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    nT = L.n_tiles(S)
    out = torch.empty((B, Hq, S, D), dtype=torch.float32, device="cuda")
    mask = torch.empty((B, Hq, nT, nT), dtype=torch.uint8, device="cuda")
    acc = torch.full((B, Hq, S, S), float("nan"), dtype=torch.float32, device="cuda")
    pw = torch.zeros((B, Hq, S, S), dtype=torch.int16, device="cuda")
    lamp.lamp_debug_attn_dump(qd, kd, vd, out, causal, window, delta, tau, mask, acc, pw)
    torch.cuda.synchronize()
    acc_g = acc.cpu().numpy().astype(np.float64)
    p_g = bf16_bits_to_f64(pw.cpu().numpy().view(np.uint16))
    ctx = L.prepare(q, k, v, causal, window, delta, tau)
    n_vis = n_acc_exact = n_p_bad = n_p_unexplained = n_fragile = 0
    worst = 0.0
    G = Hq // Hkv
    for (b, h, r) in L.all_units(B, Hq, S):
        trace = []
        L.run_unit(ctx, b, h, r, trace=trace)
        wins = unit_windows(ctx, b, h, r, trace)
        for rec in trace[:-1]:
            rows = np.arange(r * 64, r * 64 + rec["vis"].shape[0])
            vis = rec["vis"]
            ga = acc_g[b, h][np.ix_(rows, rec["cols"])]
            gp = p_g[b, h][np.ix_(rows, rec["cols"])]
            q8 = ctx["q8"][b, h, rows]
            k8 = ctx["k8"][b, h // G, rec["cols"]]
            maxp = np.max(np.abs(q8[:, None, :] * k8[None, :, :]), axis=2)
            exact = q8 @ k8.T
            ratio = np.where(vis & (maxp > 0), np.abs(ga - exact) / np.where(maxp > 0, maxp, 1), 0.0)
            worst = max(worst, float(ratio.max()))
            n_vis += int(vis.sum())
            n_acc_exact += int((vis & (ga == rec["acc8"])).sum())
            alt = fragile_alternatives(ctx, b, h, r, rec, wins[rec["t"]])
            bad = vis & (gp != rec["p"])
            n_fragile += int((vis & (alt > 0)).sum())
            n_p_bad += int(bad.sum())
            n_p_unexplained += int((bad & (alt == 0)).sum())
    say(f"[dump] {case}: visible {n_vis}; 8-bit accumulators equal to the exactly rounded sum "
        f"{n_acc_exact}, worst error 2^{np.log2(max(worst, 1e-300)):.2f} max|q8 k8| "
        f"(bound 2^{np.log2(EPS_ACC8):.1f}); weights differing {n_p_bad}, all within a midpoint "
        f"window: {n_p_unexplained == 0} (entries in a window {n_fragile})")
    assert worst <= EPS_ACC8
    assert n_p_unexplained == 0


# --------------------------------------------------------------------------
# full-size Qwen3-8B-shaped workload, sampled units
# --------------------------------------------------------------------------
def _sample_units(B, Hq, S, n, seed):
    nT = L.n_tiles(S)
    rng = np.random.default_rng(seed)
    units = {(0, 0, nT - 1), (B - 1, Hq - 1, 0), (0, Hq - 1, nT // 2), (B - 1, 0, nT - 1)}
    while len(units) < n:
        units.add((int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(nT))))
    return sorted(units)


FULL = [
    # workload, delta, tau, sampled units: every (delta, tau) point the
    # workloads are timed at (the Qwen3-32B tau sweep, both Gemma deltas)
    ("qwen3-8b", 2 ** -8, 2 ** -1, 12),
    ("qwen3-32b", 2 ** -8, 2 ** 0, 6),
    ("qwen3-32b", 2 ** -8, 2 ** -1, 6),
    ("qwen3-32b", 2 ** -8, 2 ** -3, 6),
    ("qwen3-32b", 2 ** -8, 2 ** -5, 6),
    ("gemma3-12b", 2 ** -8, 2 ** -1, 8),
    ("gemma3-12b", 2 ** -4, 2 ** -1, 8),
    ("gemma3-12b-w1024", 2 ** -8, 2 ** -1, 8),
    ("gemma3-12b-w1024", 2 ** -4, 2 ** -1, 8),
    ("qwen3-30b-a3b", 2 ** -8, 2 ** -1, 6),
]


@functools.lru_cache(maxsize=1)
def _workload(name):
    return make_config_inputs(name)


@pytest.mark.parametrize("full", FULL, ids=[f"{f[0]}-d2^{int(np.log2(f[1]))}-t2^{int(np.log2(f[2]))}" for f in FULL])
def test_forward_parity_full_size(full):
    """Each full-size workload in the launch configuration the bench times
    (one call over every head and row block); the oracle checks sampled
    (batch, head, 64-row block) units, always including the first and last
    row blocks."""
    name, delta, tau, n = full
    q, k, v, cfg = _workload(name)
    units = _sample_units(cfg["B"], cfg["Hq"], cfg["S"], n, 7)
    rep = compare(q, k, v, cfg["causal"], cfg["window"], delta, tau, units=units,
                  label=f"{name} sampled")
    assert_parity(rep)


# --------------------------------------------------------------------------
# the plain bf16 baseline
# --------------------------------------------------------------------------
PLAIN = [
    # B, Hq, Hkv, S, D, causal, window, structure, seed
    (1, 1, 1, 256, 64, 1, 0, "sinks", 81),
    (1, 4, 1, 300, 128, 1, 0, "channels", 82),     # G = 4, ragged tail
    (2, 8, 2, 200, 128, 1, 0, "channels", 83),
    (1, 3, 3, 130, 64, 0, 0, "channels", 84),      # non-causal
    (1, 2, 2, 333, 128, 1, 100, "channels", 85),   # sliding window
    (1, 1, 1, 1, 128, 1, 0, "plain", 86),          # S = 1
    (1, 4, 2, 300, 256, 1, 0, "channels", 87),     # D = 256: one-loop schedule, ragged tail
    (1, 2, 2, 333, 256, 1, 100, "channels", 88),   # D = 256 with a sliding window
    (1, 2, 1, 130, 256, 0, 0, "channels", 89),     # D = 256, non-causal
]


@pytest.mark.parametrize("case", PLAIN)
def test_plain_bf16_parity_small(case):
    B, Hq, Hkv, S, D, causal, window, st, seed = case
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, st)
    assert_parity_plain(compare_plain(q, k, v, causal, window, label=str(case)))


def test_plain_bf16_parity_full_size():
    q, k, v, cfg = make_config_inputs("qwen3-8b")
    units = _sample_units(cfg["B"], cfg["Hq"], cfg["S"], 10, 9)
    assert_parity_plain(compare_plain(q, k, v, cfg["causal"], cfg["window"], units=units,
                                      label="qwen3-8b sampled"))


def test_plain_bf16_parity_full_size_d256():
    """The plain bf16 baseline at D = 256 (one-loop schedule, K16 tiles in
    the K8 slots) on the Gemma-3-12B-shaped workload, sampled units."""
    q, k, v, cfg = _workload("gemma3-12b")
    units = _sample_units(cfg["B"], cfg["Hq"], cfg["S"], 6, 11)
    assert_parity_plain(compare_plain(q, k, v, cfg["causal"], cfg["window"], units=units,
                                      label="gemma3-12b sampled"))


# --------------------------------------------------------------------------
# the 8-bit-logit variant
# --------------------------------------------------------------------------
LOGIT8 = [
    # B, Hq, Hkv, S, D, causal, window, delta, tau, structure, seed
    (1, 1, 1, 256, 64, 1, 0, 2 ** -8, 2 ** -1, "sinks", 91),
    (1, 4, 1, 300, 128, 1, 0, 2 ** -8, 2 ** -1, "channels", 92),    # G = 4, ragged tail
    (2, 8, 2, 200, 128, 1, 0, 2 ** -8, 2 ** -3, "channels", 93),    # G = 4, B = 2
    (1, 3, 3, 130, 128, 0, 0, 2 ** -8, 2 ** -1, "channels", 94),    # non-causal
    (1, 2, 2, 333, 128, 1, 100, 2 ** -8, 2 ** -1, "channels", 95),  # sliding window
    (1, 4, 4, 257, 64, 1, 64, 0.0, 2 ** -2, "channels", 96),        # first stage off
    (1, 2, 1, 260, 128, 1, 0, 2 ** -8, np.inf, "channels", 97),     # second stage off
    (1, 4, 1, 500, 128, 1, 0, 2 ** -8, 2 ** -5, "channels+drift", 98),
    (1, 2, 1, 200, 256, 1, 0, 2 ** -8, 2 ** -1, "channels", 99),    # D = 256
    (1, 3, 3, 290, 256, 1, 100, 2 ** -4, 2 ** -2, "channels", 100), # D = 256, window
    (1, 1, 1, 1, 64, 1, 0, 2 ** -8, 2 ** -1, "plain", 101),         # S = 1
]


@pytest.mark.parametrize("case", LOGIT8)
def test_logit8_parity_small(case):
    B, Hq, Hkv, S, D, causal, window, delta, tau, st, seed = case
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, st)
    assert_parity_logit8(compare_logit8(q, k, v, causal, window, delta, tau, label=str(case)))


@pytest.mark.parametrize("case", [LOGIT8[1], LOGIT8[5], LOGIT8[8]])
def test_logit8_dump(case):
    """Every 8-bit logit the device uses is an e4m3 value within the
    admissible range of the oracle's fp32 logit, every flag that differs is
    excused, and every weight that differs from the oracle's is one that the
    protocol's windows allow to round the other way (or one of an excused
    sub-block, taken in the other precision)."""
    import mixed_precision_attention_lamp_amd as lamp
    B, Hq, Hkv, S, D, causal, window, delta, tau, st, seed = case
    q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, st)
    nT = L.n_tiles(S)
    out = torch.empty((B, Hq, S, D), dtype=torch.float32, device="cuda")
    mask = torch.empty((B, Hq, nT, nT), dtype=torch.uint8, device="cuda")
    s8 = torch.full((B, Hq, S, S), float("nan"), dtype=torch.float32, device="cuda")
    pw = torch.zeros((B, Hq, S, S), dtype=torch.int16, device="cuda")
    lamp.lamp_debug_attn_dump_logit8(to_device(q), to_device(k), to_device(v), out, causal, window,
                                     delta, tau, mask, s8, pw)
    torch.cuda.synchronize()
    s8_g = s8.cpu().numpy().astype(np.float64)
    p_g = bf16_bits_to_f64(pw.cpu().numpy().view(np.uint16))
    mask_g = mask.cpu().numpy()
    ctx = L.prepare(q, k, v, causal, window, delta, tau, logit8=True)
    n_vis = n_flip = n_p_bad = n_p_unexplained = n_outside = n_off_grid = 0
    n_flag_bad = 0
    for (b, h, r) in L.all_units(B, Hq, S):
        w = logit8_unit(ctx, b, h, r)
        flipped = {}
        for rec in w["trace"][:-1]:
            want = 0x80 | sum(int(f) << c for c, f in enumerate(rec["flags"]))
            x = int(mask_g[b, h, r, rec["t"]]) ^ want
            if x:
                n_flag_bad += int((x & 0x80) != 0 or (x & ~w["fragile"][rec["t"]] & 0x0F) != 0)
                flipped[rec["t"]] = x & 0x0F
        if flipped:
            w = logit8_unit(ctx, b, h, r, flag_bits=flipped)
        keep = ~w["max_fragile"]
        for rec in w["trace"][:-1]:
            t, vis = rec["t"], rec["vis"]
            rows = np.arange(r * 64, r * 64 + vis.shape[0])
            gs = s8_g[b, h][np.ix_(rows, rec["cols"])]
            gp = p_g[b, h][np.ix_(rows, rec["cols"])]
            n_vis += int(vis.sum())
            n_off_grid += int((e4m3_decode(e4m3_encode(gs[vis])) != gs[vis]).sum())
            n_outside += int((vis & ((gs < w["lo8"][t]) | (gs > w["hi8"][t]))).sum())
            n_flip += int((vis & (gs != rec["s2"])).sum())
            bad = vis & keep[:, None] & (gp != rec["p"])
            n_p_bad += int(bad.sum())
            n_p_unexplained += int((bad & (w["alt"][t] == 0)).sum())
    say(f"[dump-logit8] {case}: visible {n_vis}; 8-bit logits off the e4m3 grid {n_off_grid}, "
        f"outside their window {n_outside}, rounded the other way {n_flip}; weights differing "
        f"{n_p_bad} (rows with a fixed max), unexplained {n_p_unexplained}")
    assert n_off_grid == 0 and n_outside == 0 and n_p_unexplained == 0 and n_flag_bad == 0


def test_logit8_parity_full_size():
    """The Qwen3-8B-shaped workload in one call, sampled units."""
    q, k, v, cfg = make_config_inputs("qwen3-8b")
    units = _sample_units(cfg["B"], cfg["Hq"], cfg["S"], 8, 11)
    assert_parity_logit8(compare_logit8(q, k, v, cfg["causal"], cfg["window"], 2 ** -8, 2 ** -1,
                                        units=units, label="qwen3-8b sampled"))


# --------------------------------------------------------------------------
# exact device-only invariants
# --------------------------------------------------------------------------
def test_deterministic_and_exact_invariants():
    q, k, v = make_inputs(2, 4, 2, 320, 128, 60, "channels")
    o1, m1 = run_gpu(q, k, v, 1, 0, 2 ** -8, 2 ** -2)
    o2, m2 = run_gpu(q, k, v, 1, 0, 2 ** -8, 2 ** -2)
    assert np.array_equal(o1, o2) and np.array_equal(m1, m2)
    # scaling V by 2 scales the output exactly and leaves the mask alone
    v2 = (torch.from_numpy(bf16_bits_to_f64(v) * 2).float().to(torch.bfloat16)
          .view(torch.int16).numpy().view(np.uint16))
    o3, m3 = run_gpu(q, k, v2, 1, 0, 2 ** -8, 2 ** -2)
    assert np.array_equal(o3, 2 * o1) and np.array_equal(m3, m1)
    # a duplicated batch gives identical halves
    qq, kk, vv = (np.concatenate([x[:1], x[:1]]) for x in (q, k, v))
    o4, m4 = run_gpu(qq, kk, vv, 1, 0, 2 ** -8, 2 ** -2)
    assert np.array_equal(o4[0], o4[1]) and np.array_equal(m4[0], m4[1])
    assert np.array_equal(o4[0], o1[0])


def test_device_stats_match_oracle_counts():
    import mixed_precision_attention_lamp_amd as lamp
    for (S, causal, window) in ((300, 1, 0), (333, 1, 100), (130, 0, 0)):
        q, k, v = make_inputs(1, 4, 2, S, 64, 70 + S, "channels")
        qd, kd, vd = to_device(q), to_device(k), to_device(v)
        _, mask = lamp.attention(qd, kd, vd, causal, window, 2 ** -8, 2 ** -3)
        dev = lamp.subblock_stats(mask, S, causal, window)
        host = L.subblock_stats(mask.cpu().numpy(), S, causal, window)
        for key in ("hist", "visited_tiles", "visited_subblocks", "flagged_subblocks",
                    "visible_entries", "flagged_entries"):
            assert dev[key] == host[key], (key, dev[key], host[key])
