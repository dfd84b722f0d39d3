"""Seeded synthetic attention inputs with the shapes of the evaluated models.

The pages evaluate on real Qwen3 / Gemma 3 activations (tables 1-6), which are
not available here; these draws stand in for them with the models' attention
shapes.  Recipe (numpy PCG64, ``default_rng(seed)``), draw order fixed:

1. Q [B,Hq,S,D], K [B,Hkv,S,D], V [B,Hkv,S,D] ~ N(0, 1) in fp32.
2. structure "sinks": K rows 0..3 of every kv head are multiplied by 8.
   structure "channels" (and "channels+drift"): per (tensor, batch, head,
   channel) scale ~ LogNormal(0, 0.5) on Q, K and V (drawn in that order);
   then per (batch, kv head) max(1, round(0.01 D)) distinct K channels are
   multiplied by 10 (outlier channels).
3. "channels+drift" only: per (batch, kv head) a random unit vector u; every
   query of the heads reading that kv head gets its u-component replaced by
   1, and key j < 16 gets 6 sqrt(D) (1 - j/16) u added, which lifts the logit
   of key j by about 6 (1 - j/16) (keys biased toward the first positions).
4. Cast to bf16 with torch's round-to-nearest-even; returned as uint16 bits.

Decode inputs (Sq < S query rows, the last Sq positions of the sequence)
draw Q as [B,Hq,Sq,D] in step 1; everything else is unchanged.
"""
import numpy as np
import torch

# name -> (B, Hq, Hkv, S, D, causal, window, structure, seed, description)
CONFIGS = {
    "tiny": dict(B=1, Hq=1, Hkv=1, S=256, D=64, causal=1, window=0,
                 structure="sinks", seed=1,
                 desc="tiny causal attention, 4 sink keys x8"),
    "qwen3-8b": dict(B=1, Hq=32, Hkv=8, S=4096, D=128, causal=1, window=0,
                     structure="channels", seed=2,
                     desc="Qwen3-8B-shaped GQA prefill, S=4096"),
    "qwen3-32b": dict(B=2, Hq=64, Hkv=8, S=8192, D=128, causal=1, window=0,
                      structure="channels", seed=3,
                      desc="Qwen3-32B-shaped GQA prefill, B=2, S=8192"),
    "gemma3-12b": dict(B=1, Hq=16, Hkv=8, S=8192, D=256, causal=1, window=0,
                       structure="channels", seed=4,
                       desc="Gemma-3-12B-shaped attention, D=256, S=8192"),
    "gemma3-12b-w1024": dict(B=1, Hq=16, Hkv=8, S=8192, D=256, causal=1, window=1024,
                             structure="channels", seed=4,
                             desc="Gemma-3-12B-shaped sliding-window (1024) attention"),
    "qwen3-30b-a3b": dict(B=1, Hq=32, Hkv=4, S=32768, D=128, causal=1, window=0,
                          structure="channels+drift", seed=5,
                          desc="Qwen3-30B-A3B-shaped long-context GQA prefill, S=32768"),
    # decode: Sq query rows (the last Sq positions) against S cached keys
    "qwen3-8b-decode": dict(B=8, Hq=32, Hkv=8, S=16384, Sq=16, D=128, causal=1, window=0,
                            structure="channels", seed=6,
                            desc="Qwen3-8B-shaped decode, 16 queries against 16384 cached keys, B=8"),
    "qwen3-8b-decode-1": dict(B=8, Hq=32, Hkv=8, S=16384, Sq=1, D=128, causal=1, window=0,
                              structure="channels", seed=6,
                              desc="Qwen3-8B-shaped decode, one query against 16384 cached keys, B=8"),
}


def _to_bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def make_inputs(B, Hq, Hkv, S, D, seed, structure="plain", Sq=None, **_):
    """Draw (q_bits, k_bits, v_bits) as uint16 bf16 bit patterns; Q has Sq
    rows (default S)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, S if Sq is None else Sq, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    if structure == "sinks":
        k[:, :, :4, :] *= 8.0
    elif structure in ("channels", "channels+drift"):
        for x, H in ((q, Hq), (k, Hkv), (v, Hkv)):
            x *= rng.lognormal(0.0, 0.5, size=(B, H, 1, D)).astype(np.float32)
        n_out = max(1, int(round(0.01 * D)))
        for b in range(B):
            for h in range(Hkv):
                ch = rng.choice(D, size=n_out, replace=False)
                k[b, h][:, ch] *= 10.0
        if structure == "channels+drift":
            G = Hq // Hkv
            for b in range(B):
                for h in range(Hkv):
                    u = rng.standard_normal(D)
                    u /= np.linalg.norm(u)
                    u32 = u.astype(np.float32)
                    for hq in range(h * G, (h + 1) * G):
                        qa = q[b, hq]
                        qa -= np.outer(qa @ u32, u32)
                        qa += u32
                    n = min(16, S)
                    lift = (6.0 * np.sqrt(D) * (1.0 - np.arange(n) / 16.0)).astype(np.float32)
                    k[b, h, :n] += lift[:, None] * u32[None, :]
    elif structure != "plain":
        raise ValueError(f"unknown structure {structure!r}")
    return _to_bf16_bits(q), _to_bf16_bits(k), _to_bf16_bits(v)


def make_config_inputs(name):
    """Inputs of a named workload; returns (q_bits, k_bits, v_bits, cfg)."""
    cfg = CONFIGS[name]
    q, k, v = make_inputs(**cfg)
    return q, k, v, cfg
