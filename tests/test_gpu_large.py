"""Tensors of more than 2^31 elements through the C ABI (needs an MI355X).

The Qwen3-8B-shaped prefill (Hq = 32, Hkv = 8, S = 4096, D = 128) at B = 130:
Q holds 2^31 + 2^25 bf16 elements and the output 2^33 + 2^27 bytes.  The
input is a B = 2 draw repeated 65 times along the batch, so every batch of
the large call must equal, bit for bit, the batch of the B = 2 call it
repeats (output and mask), and the B = 2 call is checked against the oracle
on sampled units.  Any offset computed in 32 bits shows up as a mismatch in
the late batches."""
import numpy as np
import pytest
import torch

from inputs import make_inputs
from parity import assert_parity, compare, say, to_device

pytestmark = pytest.mark.gpu


def test_prefill_beyond_2_31_elements():
    import mixed_precision_attention_lamp_amd as lamp
    B0, Hq, Hkv, S, D, rep = 2, 32, 8, 4096, 128, 65
    delta, tau = 2.0 ** -8, 2.0 ** -1
    q, k, v = make_inputs(B0, Hq, Hkv, S, D, 411, "channels")
    nT = (S + 63) // 64
    # the B = 2 call against the oracle: first and last row blocks and a few others
    units = [(0, 0, 0), (1, Hq - 1, nT - 1), (0, 17, 31), (1, 5, 12)]
    assert_parity(compare(q, k, v, 1, 0, delta, tau, units=units, label="B=2 sampled"))

    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    out2 = torch.empty((B0, Hq, S, D), dtype=torch.float32, device="cuda")
    mask2 = torch.empty((B0, Hq, nT, nT), dtype=torch.uint8, device="cuda")
    lamp.lamp_attn_fwd(qd, kd, vd, out2, 1, 0, delta, tau, mask2)

    B = B0 * rep
    assert B * Hq * S * D > 2 ** 31
    qL = qd.repeat(rep, 1, 1, 1)
    kL, vL = kd.repeat(rep, 1, 1, 1), vd.repeat(rep, 1, 1, 1)
    del qd, kd, vd
    outL = torch.full((B, Hq, S, D), float("nan"), dtype=torch.float32, device="cuda")
    maskL = torch.full((B, Hq, nT, nT), 0x55, dtype=torch.uint8, device="cuda")
    lamp.lamp_attn_fwd(qL, kL, vL, outL, 1, 0, delta, tau, maskL)
    torch.cuda.synchronize()
    same_out = [bool(torch.equal(outL[b], out2[b % B0])) for b in range(B)]
    same_mask = [bool(torch.equal(maskL[b], mask2[b % B0])) for b in range(B)]
    say(f"[large] B={B} Hq={Hq} S={S} D={D} ({B * Hq * S * D} elements): batches equal to the B=2 call: "
        f"output {sum(same_out)}/{B}, mask {sum(same_mask)}/{B}")
    assert all(same_out) and all(same_mask)
