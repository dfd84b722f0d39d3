"""Endpoint references that pin the LampAttention oracle (test infrastructure).

The abstract of "LampAttention: Look-Ahead Mixed-Precision FlashAttention for
Dedicated Accelerators" brackets the method by two baselines that the tables
also report: "8-bit" (nothing recomputed) and "32-bit" (tables 1-6 column
headers).  These functions are the plain definitions of those endpoints and of
exact attention:

* ``exact_attention``: softmax(Q K^T / sqrt(D)) V in fp64 on the bf16 inputs.
* ``bf16_attention``: ordinary attention with bf16 operands, fp32 logits, a
  global row max and bf16-rounded exponentials.  With every sub-block sent to
  16-bit (delta <= 0, tau <= 0) the method must equal it up to the bf16
  rounding of the weights (its running max comes from the 8-bit logits).
* ``eight_bit_attention``: the tiled FlashAttention with 8-bit logits and
  8-bit exponentials and no recompute -- the second stage disabled.  It is
  organised per head over the full logit matrix (all rows at once, one KV tile
  at a time), not per 64-row unit as ``lamp.run_unit``.
"""
import numpy as np

from .formats import bf16_bits_to_f64, exp2_f32, fl32, fma32, round_bf16, round_e4m3
from .lamp import BC, log2_scale, quantize, visible


def _vis_full(S, causal, window):
    idx = np.arange(S)
    return visible(idx, idx, causal, window)


def exact_attention(q_bits, k_bits, v_bits, causal=True, window=0):
    """fp64 softmax(Q K^T / sqrt(D)) V, masked (masked logits excluded)."""
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    v = bf16_bits_to_f64(v_bits)
    B, Hq, S, D = q.shape
    G = Hq // k.shape[1]
    vis = _vis_full(S, causal, window)
    out = np.zeros((B, Hq, S, D))
    for b in range(B):
        for h in range(Hq):
            s = q[b, h] @ k[b, h // G].T / np.sqrt(D)
            s = np.where(vis, s, -np.inf)
            w = np.exp(s - s.max(axis=1, keepdims=True))
            out[b, h] = (w @ v[b, h // G]) / w.sum(axis=1, keepdims=True)
    return out


def bf16_attention(q_bits, k_bits, v_bits, causal=True, window=0):
    """Plain bf16 attention: p = BF16(exp2(fl32(acc16 * c16 - m))) with the global row max."""
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    v = bf16_bits_to_f64(v_bits)
    B, Hq, S, D = q.shape
    G = Hq // k.shape[1]
    c16 = float(fl32(log2_scale(D)))
    vis = _vis_full(S, causal, window)
    out = np.zeros((B, Hq, S, D))
    for b in range(B):
        for h in range(Hq):
            acc = fl32(q[b, h] @ k[b, h // G].T)
            s = np.where(vis, fl32(acc * c16), -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.where(vis, round_bf16(exp2_f32(fma32(acc, c16, -m))), 0.0)
            out[b, h] = (p @ v[b, h // G]) / p.sum(axis=1, keepdims=True)
    return out


def eight_bit_attention(q_bits, k_bits, v_bits, causal=True, window=0):
    """Tiled 8-bit FlashAttention (no recompute), all rows of a head at once."""
    q8, _, sq, _ = quantize(q_bits)
    k8, _, sk, _ = quantize(k_bits)
    v = bf16_bits_to_f64(v_bits)
    B, Hq, S, D = q8.shape
    G = Hq // k8.shape[1]
    L = log2_scale(D)
    vis = _vis_full(S, causal, window)
    out = np.zeros((B, Hq, S, D))
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            c8 = float(fl32(float(sq[b, h]) * float(sk[b, hk]) * L))
            acc = fl32(q8[b, h] @ k8[b, hk].T)
            m = np.full(S, -np.inf)
            ell = np.zeros(S)
            o = np.zeros((S, D))
            for t0 in range(0, S, BC):
                cols = slice(t0, min(t0 + BC, S))
                vb = vis[:, cols]
                # a row without a visible key in this tile keeps m, l and o
                s2 = np.where(vb, fl32(acc[:, cols] * c8), -np.inf)
                m_new = np.maximum(m, s2.max(axis=1))
                ok = m_new > -np.inf
                mm = np.where(ok, m_new, 0.0)
                p = np.where(vb, round_e4m3(exp2_f32(fma32(acc[:, cols], c8, -mm[:, None]))), 0.0)
                a = np.where(ok & (m > -np.inf), np.exp2(m - mm), np.where(ok, 0.0, 1.0))
                ell = a * ell + p.sum(axis=1)
                o = a[:, None] * o + p @ v[b, hk, cols]
                m = m_new
            out[b, h] = o / ell[:, None]
    return out
