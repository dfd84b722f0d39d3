"""MI355X (gfx950) LampAttention forward pass: HIP kernels behind a C ABI.

The method is the look-ahead mixed-precision FlashAttention of "LampAttention:
Look-Ahead Mixed-Precision FlashAttention for Dedicated Accelerators": 8-bit
logits and exponentials per tile, a two-stage (delta, tau) test that flags
sensitive 64x16 sub-blocks, a 16-bit recompute of those only, then online
softmax and P.V.  All of it runs in the kernels of ``liblamp.so``; this
package only marshals torch tensors into the C entry points (see _lib.py) and
allocates outputs.
"""
from ._lib import (LAMP_STATS_LEN, LampError, declared_symbols, lamp_attn_decode,  # noqa: F401
                   lamp_attn_decode_with_amax, lamp_kv_amax_update,
                   lamp_attn_fwd, lamp_attn_fwd_bf16, lamp_attn_fwd_exp2poly, lamp_attn_fwd_logit8,
                   lamp_attn_fwd_noalloc, lamp_debug_attn_dump, lamp_debug_attn_dump_exp2poly, lamp_debug_exp2poly,
                   lamp_decode_tiles_per_split, lamp_debug_fp8_dot,
                   lamp_debug_attn_dump_logit8, lamp_debug_convert, lamp_last_error,
                   lamp_quantize_qk, lamp_read_timing, lamp_release_workspace, lamp_set_stream,
                   lamp_set_timing, lamp_subblock_stats, lamp_version, load)

TILE = 64


def n_tiles(S):
    return (S + TILE - 1) // TILE


def attention(q, k, v, causal=True, window=0, delta=2.0 ** -8, tau=2.0 ** -1, with_mask=True,
              logit8=False, exp_poly=False):
    """Allocate the outputs and run lamp_attn_fwd (lamp_attn_fwd_logit8 when
    logit8, lamp_attn_fwd_exp2poly when exp_poly); returns (out, mask or None)."""
    if logit8 and exp_poly:
        raise ValueError("logit8 and exp_poly are separate variants")
    import torch
    B, Hq, S, D = q.shape
    out = torch.empty((B, Hq, S, D), dtype=torch.float32, device=q.device)
    mask = None
    if with_mask:
        nT = n_tiles(S)
        mask = torch.empty((B, Hq, nT, nT), dtype=torch.uint8, device=q.device)
    fwd = lamp_attn_fwd_logit8 if logit8 else (lamp_attn_fwd_exp2poly if exp_poly else lamp_attn_fwd)
    fwd(q, k, v, out, int(causal), int(window), delta, tau, mask)
    return out, mask


def attention_bf16(q, k, v, causal=True, window=0, with_mask=True):
    """Allocate the outputs and run the plain bf16 baseline (lamp_attn_fwd_bf16)."""
    import torch
    B, Hq, S, D = q.shape
    out = torch.empty((B, Hq, S, D), dtype=torch.float32, device=q.device)
    mask = None
    if with_mask:
        nT = n_tiles(S)
        mask = torch.empty((B, Hq, nT, nT), dtype=torch.uint8, device=q.device)
    lamp_attn_fwd_bf16(q, k, v, out, int(causal), int(window), mask)
    return out, mask


def attention_decode(q, k, v, causal=True, window=0, delta=2.0 ** -8, tau=2.0 ** -1,
                     tiles_per_split=0, with_mask=True):
    """Allocate the outputs and run lamp_attn_decode; returns (out, mask or None)."""
    import torch
    B, Hq, Sq, D = q.shape
    out = torch.empty((B, Hq, Sq, D), dtype=torch.float32, device=q.device)
    mask = None
    if with_mask:
        mask = torch.empty((B, Hq, n_tiles(k.shape[2])), dtype=torch.uint8, device=q.device)
    lamp_attn_decode(q, k, v, out, int(causal), int(window), delta, tau, tiles_per_split, mask)
    return out, mask


def subblock_stats(mask, S, causal, window):
    """Device-reduced histogram of 16-bit sub-blocks per tile (10 int64, as a dict)."""
    import torch
    B, Hq = mask.shape[:2]
    st = torch.empty(LAMP_STATS_LEN, dtype=torch.int64, device=mask.device)
    lamp_subblock_stats(mask, B, Hq, S, int(causal), int(window), st)
    v = st.cpu().tolist()
    vt = v[5]
    return dict(hist=v[0:5], visited_tiles=vt, visited_subblocks=v[6], flagged_subblocks=v[7],
                visible_entries=v[8], flagged_entries=v[9],
                r_sb=v[7] / v[6] if v[6] else 0.0, r_e=v[9] / v[8] if v[8] else 0.0,
                pages_buckets=[v[0] / vt, v[1] / vt, sum(v[2:5]) / vt] if vt else [0.0, 0.0, 0.0])
