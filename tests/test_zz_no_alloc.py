"""lamp_attn_fwd_noalloc, the entry point for callers that cannot allocate
device memory, through the C ABI (needs an MI355X): two calls in a row, the
second on a smaller input, each equal bit for bit to lamp_attn_fwd on the
same input (the same kernels, with the workspace in the library's fixed
scratch array), and a request beyond the array rejected before any launch."""
import numpy as np
import pytest
import torch

from inputs import make_inputs
from parity import say, to_device

pytestmark = pytest.mark.gpu


def _both(q, k, v, causal, window, delta, tau):
    import mixed_precision_attention_lamp_amd as lamp
    B, Hq, S, D = q.shape
    nT = (S + 63) // 64
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    outs = []
    for fn in (lamp.lamp_attn_fwd, lamp.lamp_attn_fwd_noalloc):
        out = torch.full((B, Hq, S, D), float("nan"), dtype=torch.float32, device="cuda")
        mask = torch.full((B, Hq, nT, nT), 0x55, dtype=torch.uint8, device="cuda")
        fn(qd, kd, vd, out, causal, window, delta, tau, mask)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), mask.cpu().numpy()))
    return outs


def test_noalloc_matches_lamp_attn_fwd_twice_then_smaller():
    # the first call fills the scratch array with a larger problem's K8 and
    # V^T; the second, smaller one must not read any of it
    for (B, Hq, Hkv, S, D, causal, window, st, seed) in ((1, 8, 2, 1500, 128, 1, 0, "channels", 301),
                                                          (1, 2, 1, 333, 64, 1, 100, "channels", 302)):
        q, k, v = make_inputs(B, Hq, Hkv, S, D, seed, st)
        (o1, m1), (o2, m2) = _both(q, k, v, causal, window, 2.0 ** -8, 2.0 ** -1)
        say(f"[noalloc] B={B} Hq={Hq} Hkv={Hkv} S={S} D={D}: outputs equal {np.array_equal(o1, o2)}, "
            f"masks equal {np.array_equal(m1, m2)}")
        assert np.isfinite(o1).all()
        assert np.array_equal(o1, o2) and np.array_equal(m1, m2)


def test_noalloc_rejects_a_workspace_beyond_the_scratch_array():
    import mixed_precision_attention_lamp_amd as lamp
    from mixed_precision_attention_lamp_amd._lib import LAMP_ERR_UNSUPPORTED
    # K8 and V^T need 3 * B * Hkv * S * D = 3 * 1 * 8 * 32768 * 128 bytes = 96 MiB > 64 MiB
    B, Hq, Hkv, S, D = 1, 8, 8, 32768, 128
    q = torch.zeros((B, Hq, S, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, S, D), dtype=torch.bfloat16, device="cuda")
    out = torch.full((B, Hq, S, D), 3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(lamp.LampError) as e:
        lamp.lamp_attn_fwd_noalloc(q, k, k, out, 1, 0, 2.0 ** -8, 0.5)
    assert e.value.code == LAMP_ERR_UNSUPPORTED
    say(f"[noalloc] {e.value}")
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
