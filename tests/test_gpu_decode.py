"""Split-KV decode on the GPU against the oracle's decode, through the C ABI
(needs an MI355X).

Cases span Sq = 1..16 query rows, GQA groups of 1..8 (four- and eight-wave
workgroups), D = 64 / 128 / 256, ragged key counts, windows that leave whole
splits empty, every test mode, split sizes from one tile to all tiles, the
library's own split choice, and the full-size decode workload on sampled
heads.
"""
import numpy as np
import pytest
import torch

from inputs import make_config_inputs, make_inputs
from oracle import lamp as L
from parity import assert_parity_decode, compare_decode, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import mixed_precision_attention_lamp_amd as lamp
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lamp.load()
    yield
    torch.cuda.synchronize()


DECODE = [
    # B, Hq, Hkv, Sq, Skv, D, causal, window, delta, tau, tiles/split, structure, seed
    (2, 8, 2, 16, 1000, 128, 1, 0, 2 ** -8, 2 ** -1, 4, "channels", 201),    # G = 4, ragged
    (1, 4, 4, 1, 777, 128, 1, 0, 2 ** -8, 2 ** -2, 3, "channels", 202),      # Sq = 1, G = 1
    (1, 16, 2, 5, 640, 128, 1, 0, 2 ** -8, 2 ** -1, 2, "sinks", 203),        # G = 8
    (1, 8, 2, 16, 1500, 64, 1, 0, 2 ** -4, 2 ** -3, 5, "channels", 204),     # D = 64
    (1, 4, 2, 8, 900, 256, 1, 0, 2 ** -8, 2 ** -1, 3, "channels", 205),      # D = 256
    (1, 4, 2, 16, 1200, 128, 1, 300, 2 ** -8, 2 ** -1, 2, "channels", 206),  # window: empty splits
    (1, 4, 1, 16, 500, 128, 0, 0, 2 ** -8, 2 ** -1, 1, "channels", 207),     # non-causal, 1-tile splits
    (1, 4, 1, 16, 700, 128, 1, 0, 0.0, 2 ** -2, 3, "channels", 208),         # first stage off
    (1, 4, 1, 16, 700, 128, 1, 0, 2 ** -8, np.inf, 3, "channels", 209),      # second stage off
    (1, 2, 1, 3, 3, 64, 1, 0, 2 ** -8, 2 ** -1, 1, "plain", 210),            # Skv = 3
    (1, 4, 2, 16, 2000, 128, 1, 0, 0.0, 0.0, 4, "channels", 211),            # every sub-block 16-bit
    (1, 12, 2, 16, 800, 128, 1, 0, 2 ** -8, 2 ** -1, 2, "channels", 212),    # G = 6
    (1, 8, 2, 16, 1100, 64, 1, 0, 2 ** -8, 2 ** -3, 100, "channels+drift", 213),  # one split
    # rows past Sq and window / Skv edge tiles with the first stage off
    (1, 4, 2, 7, 1300, 128, 1, 200, 0.0, 2 ** -3, 3, "channels", 214),
    # the same with both stages, on drifting keys (per-entry test on edge tiles)
    (1, 8, 2, 5, 1250, 128, 1, 150, 2 ** -8, 2 ** -4, 2, "channels+drift", 215),
    # one split of 79 tiles: mask bytes of more than 64 tiles per split
    (1, 4, 2, 16, 5000, 128, 1, 0, 2 ** -8, 2 ** -1, 79, "channels", 216),
    # a window that starts inside the second 64-tile chunk of a split
    (1, 4, 4, 3, 9000, 64, 1, 4700, 2 ** -8, 2 ** -1, 141, "channels", 217),
]


@pytest.mark.parametrize("case", DECODE)
def test_decode_parity(case):
    B, Hq, Hkv, Sq, Skv, D, causal, window, delta, tau, tps, st, seed = case
    q, k, v = make_inputs(B, Hq, Hkv, Skv, D, seed, st, Sq=Sq)
    assert_parity_decode(compare_decode(q, k, v, causal, window, delta, tau, min(tps, L.n_tiles(Skv)),
                                        label=str(case)))


def test_decode_library_split_choice():
    """tiles_per_split = 0 uses lamp_decode_tiles_per_split's choice."""
    import mixed_precision_attention_lamp_amd as lamp
    B, Hq, Hkv, Sq, Skv, D = 2, 8, 2, 16, 3000, 128
    tps = lamp.lamp_decode_tiles_per_split(B, Hq, Hkv, Sq, Skv, D)
    say(f"[decode] library split for B={B} Hkv={Hkv} Skv={Skv}: {tps} tiles per split")
    assert 1 <= tps <= L.n_tiles(Skv)
    q, k, v = make_inputs(B, Hq, Hkv, Skv, D, 220, "channels", Sq=Sq)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o0, m0 = lamp.attention_decode(qd, kd, vd, True, 0, 2 ** -8, 2 ** -1, tiles_per_split=0)
    o1, m1 = lamp.attention_decode(qd, kd, vd, True, 0, 2 ** -8, 2 ** -1, tiles_per_split=tps)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(m0, m1)
    assert_parity_decode(compare_decode(q, k, v, 1, 0, 2 ** -8, 2 ** -1, tps,
                                        gpu=(o0.cpu().numpy(), m0.cpu().numpy()), label="library split"))


def test_decode_rejects_unsupported():
    import mixed_precision_attention_lamp_amd as lamp
    q, k, v = make_inputs(1, 2, 1, 64, 128, 221, "plain", Sq=17)
    with pytest.raises(lamp.LampError):
        lamp.attention_decode(to_device(q), to_device(k), to_device(v))
    q, k, v = make_inputs(1, 16, 1, 64, 128, 222, "plain", Sq=4)
    with pytest.raises(lamp.LampError):        # G = 16
        lamp.attention_decode(to_device(q), to_device(k), to_device(v))


def test_decode_full_size():
    """The full-size decode workload in the launch configuration the bench
    times (library split), sampled heads."""
    import mixed_precision_attention_lamp_amd as lamp
    q, k, v, cfg = make_config_inputs("qwen3-8b-decode")
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    tps = lamp.lamp_decode_tiles_per_split(B, Hq, Hkv, Sq, Skv, D)
    rng = np.random.default_rng(5)
    heads = sorted({(0, 0), (B - 1, Hq - 1)} | {(int(rng.integers(B)), int(rng.integers(Hq)))
                                               for _ in range(6)})
    out, mask = lamp.attention_decode(to_device(q), to_device(k), to_device(v), True, 0, 2 ** -8, 2 ** -1)
    torch.cuda.synchronize()
    assert_parity_decode(compare_decode(q, k, v, 1, 0, 2 ** -8, 2 ** -1, tps, heads=heads,
                                        gpu=(out.cpu().numpy(), mask.cpu().numpy()),
                                        label=f"qwen3-8b-decode sampled, {tps} tiles per split"))


KEPT = [
    # B, Hq, Hkv, Sq, Skv, D, causal, window, pieces of the cache, structure, seed
    (2, 8, 2, 16, 3000, 128, 1, 0, (1000, 1984, 16), "channels", 231),
    (1, 4, 1, 1, 777, 64, 1, 0, (777,), "channels", 232),
    (1, 8, 4, 5, 1300, 256, 1, 400, (1, 650, 649), "sinks", 233),
]


@pytest.mark.parametrize("case", KEPT)
def test_decode_with_kept_amax(case):
    """Kept K maxima, folded in from the cache in pieces, equal the oracle's
    per-head amax; decode with them equals lamp_attn_decode bit for bit, and
    folding in the newest keys again changes nothing."""
    import mixed_precision_attention_lamp_amd as lamp
    B, Hq, Hkv, Sq, Skv, D, causal, window, pieces, st, seed = case
    assert sum(pieces) == Skv
    q, k, v = make_inputs(B, Hq, Hkv, Skv, D, seed, st, Sq=Sq)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    state = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    start = 0
    for n in pieces:
        lamp.lamp_kv_amax_update(kd[:, :, start:start + n].contiguous(), state)
        start += n
    torch.cuda.synchronize()
    # the oracle's per-head scales come from the same maxima
    scale, _ = L.head_scales(k)
    kept = state.cpu().numpy().astype(np.uint32)
    amax = (kept.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(np.where(amax > 0, (amax / 448.0).astype(np.float32), np.float32(1.0)),
                          np.asarray(scale, dtype=np.float32).reshape(B, Hkv))
    nT = L.n_tiles(Skv)
    res = []
    for fn in ("full", "kept"):
        out = torch.full((B, Hq, Sq, D), float("nan"), dtype=torch.float32, device="cuda")
        mask = torch.full((B, Hq, nT), 0x55, dtype=torch.uint8, device="cuda")
        if fn == "full":
            lamp.lamp_attn_decode(qd, kd, vd, out, causal, window, 2 ** -8, 2 ** -1, 0, mask)
        else:
            lamp.lamp_attn_decode_with_amax(qd, kd, vd, out, state, causal, window, 2 ** -8, 2 ** -1, 0, mask)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), mask.cpu().numpy()))
    lamp.lamp_kv_amax_update(kd[:, :, Skv - Sq:].contiguous(), state)
    torch.cuda.synchronize()
    again = np.array_equal(state.cpu().numpy().astype(np.uint32), kept)
    say(f"[decode-kept] {case}: scales equal the oracle's; outputs equal {np.array_equal(res[0][0], res[1][0])}, "
        f"masks equal {np.array_equal(res[0][1], res[1][1])}, state unchanged by the newest keys {again}")
    assert np.isfinite(res[0][0]).all()
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1]) and again
