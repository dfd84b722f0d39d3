"""The C ABI's resource rules on the device (needs an MI355X): the
workspace limit turns an oversized request into LAMP_ERR_NOMEM with nothing
launched, and calls on two streams (one workspace each) may overlap in time
without changing a bit of either result."""
import os

import numpy as np
import pytest
import torch

from inputs import make_inputs
from parity import run_gpu, say, to_device

pytestmark = pytest.mark.gpu


def test_workspace_limit_gives_nomem_and_leaves_outputs_alone():
    import mixed_precision_attention_lamp_amd as lamp
    from mixed_precision_attention_lamp_amd._lib import LAMP_ERR_NOMEM
    q, k, v = make_inputs(1, 2, 1, 300, 64, 61, "channels")
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    out = torch.full((1, 2, 300, 64), 7.0, dtype=torch.float32, device="cuda")
    old = os.environ.get("LAMP_WORKSPACE_LIMIT_BYTES")
    os.environ["LAMP_WORKSPACE_LIMIT_BYTES"] = "4096"
    try:
        with pytest.raises(lamp.LampError) as e:
            lamp.lamp_attn_fwd(qd, kd, vd, out, 1, 0, 2.0 ** -8, 0.5)
        assert e.value.code == LAMP_ERR_NOMEM
        say(f"[boundary] {e.value}")
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())
    finally:
        if old is None:
            del os.environ["LAMP_WORKSPACE_LIMIT_BYTES"]
        else:
            os.environ["LAMP_WORKSPACE_LIMIT_BYTES"] = old
    lamp.lamp_attn_fwd(qd, kd, vd, out, 1, 0, 2.0 ** -8, 0.5)
    torch.cuda.synchronize()
    ref, _ = run_gpu(q, k, v, 1, 0, 2.0 ** -8, 0.5)
    assert np.array_equal(out.cpu().numpy(), ref)


def test_two_streams_overlap_without_interference():
    import mixed_precision_attention_lamp_amd as lamp
    cases = [make_inputs(1, 8, 2, 1500, 128, 62, "channels"), make_inputs(2, 4, 4, 900, 64, 63, "channels")]
    refs = [run_gpu(q, k, v, 1, 0, 2.0 ** -8, 0.5) for (q, k, v) in cases]
    dev = [tuple(to_device(x) for x in c) for c in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    torch.cuda.synchronize()
    for rep in range(3):
        outs = []
        # enqueue both calls before waiting for either
        for (qd, kd, vd), s in zip(dev, streams):
            with torch.cuda.stream(s):
                outs.append(lamp.attention(qd, kd, vd, True, 0, 2.0 ** -8, 0.5))
        torch.cuda.synchronize()
        for (o, m), (ro, rm) in zip(outs, refs):
            assert np.array_equal(o.cpu().numpy(), ro) and np.array_equal(m.cpu().numpy(), rm)
    lamp.lamp_set_stream(None)
