"""Bench of the LampAttention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload qwen3-8b]
                    [--delta D] [--tau T] [--no-cpu-baseline]
    python bench.py --copy-calibrate      # plain 1 GiB device copy (counter calibration)
    python bench.py --grid [--workload W] # speed/recompute curve over (delta, tau)
    python bench.py --workload qwen3-8b-decode   # split-KV decode (lamp_attn_decode)
    python bench.py --workload qwen3-8b-decode --kept-amax   # decode with kept K maxima

A step is one lamp_attn_fwd call (quantisation pass, V transpose and the fused
attention kernel) over one batch of seeded synthetic input already resident
in HBM.  Prints one JSON line with the throughput, the roofline of the
dominant kernel (the fused attention kernel, timed with HIP events on the
stream it is launched on), the recompute statistics and the CPU oracle timed
on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s + % blended FP8/bf16 roofline; 16-bit sub-block fraction"
PEAK_FP8 = 5.0e15          # MI355X dense FP8 matrix FLOP/s
PEAK_BF16 = 2.5e15         # MI355X dense bf16 matrix FLOP/s
PEAK_HBM = 8.0e12          # MI355X HBM3E bytes/s
COPY_BYTES = 1 << 30       # size of the calibration copy

# HBM traffic of the attention kernel per workload, from two rocprofv3 --pmc
# runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by the same
# counter's reading for a plain copy of COPY_BYTES (profiles/
# attn_qwen3_8b_hbm_traffic.md, attn_gemma3_12b_counters.md).  Valid only for
# the kernel source whose hash is recorded; any change to it makes the figure
# null.  (Taken on sources that compile to the same instructions as this
# one: later edits changed comments, or only other kernels.)
TRAFFIC = [
    {"kernel_hash": "4dc6632fac05b9a8", "workload": "qwen3-8b", "delta": 2.0 ** -8, "tau": 2.0 ** -1,
     "bytes_per_launch": 130208276.1},
    {"kernel_hash": "4dc6632fac05b9a8", "workload": "gemma3-12b", "delta": 2.0 ** -8, "tau": 2.0 ** -1,
     "bytes_per_launch": 585246394.0},
]


# Vector-issue ceiling of the attention kernel per workload, from the
# instruction counters (profiles/attn_qwen3_8b_sq_counters.md,
# attn_gemma3_12b_counters.md): vector cycles per SIMD per launch (full-rate
# instructions 4 cycles, v_exp_f32 and v_cvt_pk_fp8_f32 8, matrix products 4
# of issue), i.e. the launch time if the vector units were never idle.  Valid
# only for the recorded kernel source.
VALU_CEILING = [
    {"kernel_hash": "4dc6632fac05b9a8", "workload": "qwen3-8b", "delta": 2.0 ** -8, "tau": 2.0 ** -1,
     "cycles_per_simd": 208688.3, "clock_hz": 2.4e9, "source": "profiles/attn_qwen3_8b_sq_counters.md"},
    {"kernel_hash": "4dc6632fac05b9a8", "workload": "gemma3-12b", "delta": 2.0 ** -8, "tau": 2.0 ** -1,
     "cycles_per_simd": 586847.4, "clock_hz": 2.4e9, "source": "profiles/attn_gemma3_12b_counters.md"},
]


def _record(records, args, kernel_hash):
    """The record of `records` measured on this kernel source and workload point."""
    for r in records:
        if (r["kernel_hash"] == kernel_hash and r["workload"] == args.workload
                and r["delta"] == args.delta and r["tau"] == args.tau):
            return r
    return None


# The same for the decode kernel on the qwen3-8b-decode workload
# (profiles/decode_qwen3_8b_hbm_traffic.md), library split.
TRAFFIC_DECODE = {"kernel_hash": "0fa370a478cfbdf6", "workload": "qwen3-8b-decode", "delta": 2.0 ** -8,
                  "tau": 2.0 ** -1, "bytes_per_launch": 555052289.2}


def decode_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixed_precision_attention_lamp_amd", "csrc")
    for name in ("decode.hip", "tiles.hpp", "common.hpp"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixed_precision_attention_lamp_amd", "csrc")
    for name in ("attn.hip", "tiles.hpp", "common.hpp"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def copy_calibrate():
    """A plain device-to-device copy of COPY_BYTES, five times (for counter
    calibration: the copy reads and writes exactly COPY_BYTES each time)."""
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 5}), flush=True)


def visible_pairs_per_head(S, causal, window):
    """Exact count of visible (query, key) pairs of one head."""
    i = np.arange(S, dtype=np.int64)
    hi = i if causal else np.full(S, S - 1)
    lo = np.maximum(0, i - window + 1) if window > 0 else np.zeros(S, dtype=np.int64)
    return int(np.maximum(0, hi - lo + 1).sum())


def unit_pairs(r, S, causal, window):
    i = np.arange(r * 64, min(r * 64 + 64, S), dtype=np.int64)
    hi = i if causal else np.full(i.size, S - 1)
    lo = np.maximum(0, i - window + 1) if window > 0 else np.zeros(i.size, dtype=np.int64)
    return int(np.maximum(0, hi - lo + 1).sum())


_CTX = None


def _oracle_unit(unit):
    """Worker: one (b, hq, r) unit through the oracle (CPU baseline only).
    The oracle context is inherited from the parent through fork."""
    from oracle import lamp as L
    L.run_unit(_CTX, *unit)
    return unit


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_expectation(unit):
    """Worker: the parity protocol's oracle-side expectation of one unit
    (output rows, mask bytes, excusable flags, flip bound)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import parity
    return unit, parity.unit_expectation(_CTX, *unit)


def parity_units(B, Hq, nT, n=32, seed=77):
    """Units the bench's parity check compares: the first and last row block
    of four heads, then random units."""
    rng = np.random.default_rng(seed)
    units = set()
    for h in np.linspace(0, Hq - 1, 4).astype(int):
        b = int(rng.integers(B))
        units.update({(b, int(h), 0), (b, int(h), nT - 1)})
    while len(units) < min(n, B * Hq * nT):
        units.add((int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(nT))))
    return sorted(units)


def single_core_tiny():
    """Seconds of one core for the whole tiny workload through the oracle."""
    from inputs import make_config_inputs
    from oracle import lamp as L
    q, k, v, cfg = make_config_inputs("tiny")
    t0 = time.perf_counter()
    L.lamp_forward(q, k, v, cfg["causal"], cfg["window"], 2.0 ** -8, 2.0 ** -1)
    return time.perf_counter() - t0


def cpu_baseline(q, k, v, cfg, delta, tau, budget_s, cores, with_parity=True, exp_poly=False):
    """Time the oracle on sampled units of the same workload (reported
    baseline), then (untimed) compute the parity protocol's expectation of
    the units the bench compares with the device output afterwards."""
    global _CTX
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    from oracle import lamp as L
    threadpool_limits(1)
    tiny_s = single_core_tiny()
    _CTX = L.prepare(q, k, v, cfg["causal"], cfg["window"], delta, tau, exp_poly=exp_poly)
    B, Hq, S, D = q.shape
    nT = L.n_tiles(S)
    rng = np.random.default_rng(123)
    # first a calibration unit, then as many random units as fit the budget
    units = [(int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(nT)))
             for _ in range(4096)]
    t0 = time.perf_counter()
    _oracle_unit(units[0])
    one = max(time.perf_counter() - t0, 1e-3)
    n = max(cores, min(len(units), int(budget_s * cores / one)))
    sample = units[:n]
    expectations = {}
    t0 = time.perf_counter()
    if cores > 1:
        with mp.get_context("fork").Pool(cores) as pool:
            for _ in pool.imap_unordered(_oracle_unit, sample, chunksize=1):
                pass
            wall = time.perf_counter() - t0
            if with_parity:
                for u, e in pool.imap_unordered(_oracle_expectation, parity_units(B, Hq, nT), chunksize=1):
                    expectations[u] = e
    else:
        for u in sample:
            _oracle_unit(u)
        wall = time.perf_counter() - t0
        if with_parity:
            for u in parity_units(B, Hq, nT):
                expectations[u] = _oracle_expectation(u)[1]
    flops = sum(4.0 * D * unit_pairs(r, S, cfg["causal"], cfg["window"]) for (_, _, r) in sample)
    return dict(value=flops / wall / 1e12, unit="TFLOP/s", cores=cores, kind="oracle",
                sample=f"{len(sample)} random (batch, head, 64-row block) units of the same "
                       f"workload ({flops / 1e9:.2f} GFLOP nominal), {wall:.1f} s wall",
                cpu_model=cpu_model(), cpus_visible=os.cpu_count(),
                single_core_tiny_workload_s=tiny_s, wall_s=wall), expectations


def parity_block(expectations, out, mask):
    """The oracle leg's check of the device output of the last timed step
    against the expectations computed before the GPU was touched (the
    protocol of tests/parity.py; host arrays only)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import parity
    judged, n_sub = [], 0
    S = out.shape[2]
    for (b, h, r), e in sorted(expectations.items()):
        rows = slice(r * 64, min(r * 64 + 64, S))
        judged.append(parity.judge_unit(e, out[b, h, rows], mask[b, h, r], (b, h, r)))
        n_sub += 4 * len(e["mask"])
    rep = parity.summarize(judged, n_sub)
    ok = (rep["finite"] and not rep["unexcused"] and not rep["rows_unexplained"]
          and rep["mean_abs"] <= parity.MEAN_ABS and rep["max_abs"] <= parity.MAX_ABS_CAP
          and rep["rows_above"] <= parity.MAX_ROWS_ABOVE * rep["rows_compared"])
    n_mis = len(rep["excused"]) + len(rep["unexcused"])
    return {"units": len(expectations), "rows": rep["rows_compared"], "max_abs": rep["max_abs"],
            "mean_abs": rep["mean_abs"], "rows_above_4e-3": rep["rows_above"],
            "rows_above_frac": rep["rows_above"] / max(rep["rows_compared"], 1),
            "rows_unexplained": len(rep["rows_unexplained"]), "mask_subblocks": n_sub,
            "mask_mismatches": n_mis, "excused": len(rep["excused"]),
            "within_one_ulp": rep["excused_within_one_ulp"], "unexcused": len(rep["unexcused"]),
            "pass": bool(ok)}


# --------------------------------------------------------------------------
# decode workloads (lamp_attn_decode)
# --------------------------------------------------------------------------
def decode_pairs_per_head(Sq, Skv, causal, window):
    """Visible (query, key) pairs of one head; query i sits at Skv - Sq + i."""
    p = np.arange(Skv - Sq, Skv, dtype=np.int64)
    hi = p if causal else np.full(Sq, Skv - 1)
    lo = np.maximum(0, p - window + 1) if window > 0 else np.zeros(Sq, dtype=np.int64)
    return int(np.maximum(0, hi - lo + 1).sum())


def decode_subblock_entries(Sq, Skv, causal, window):
    """[nT, 4] visible entries per (tile, sub-block) of one head."""
    nT = (Skv + 63) // 64
    p = np.arange(Skv - Sq, Skv, dtype=np.int64)[:, None]
    j = np.arange(nT * 64, dtype=np.int64)[None, :]
    vis = j < Skv
    if causal:
        vis = vis & (j <= p)
    if window > 0:
        vis = vis & (p - j < window)
    return vis.sum(axis=0).reshape(nT, 4, 16).sum(axis=2)


def measure_decode(lamp, torch, tensors, shape, causal, window, delta, tau, tps, steps, warmup, settle_ms=0.0,
                   kept=None):
    """Time `steps` lamp_attn_decode calls after `warmup`; returns the step
    time, the decode kernel time and the amax and scale pass time (HIP
    events on the library's stream; the merge of the splits is in the step
    only), FLOP counts and the recompute counts.  With kept = (state, k_new)
    a step folds the newest keys k_new into the kept K maxima and decodes with
    them (lamp_kv_amax_update + lamp_attn_decode_with_amax)."""
    qd, kd, vd, out, mask = tensors
    B, Hq, Hkv, Sq, Skv, D = shape

    def step():
        if kept is None:
            lamp.lamp_attn_decode(qd, kd, vd, out, causal, window, delta, tau, tps, mask)
        else:
            lamp.lamp_kv_amax_update(kept[1], kept[0])
            lamp.lamp_attn_decode_with_amax(qd, kd, vd, out, kept[0], causal, window, delta, tau, tps, mask)

    settle(torch, step, settle_ms)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    lamp.lamp_set_timing(1)
    lamp.lamp_read_timing()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    prep_ms, attn_ms, ncalls = lamp.lamp_read_timing()
    lamp.lamp_set_timing(0)
    m = mask.cpu().numpy()
    ent = decode_subblock_entries(Sq, Skv, causal, window)            # [nT, 4]
    bits = np.stack([(m >> c) & 1 for c in range(4)], axis=-1)         # [B, Hq, nT, 4]
    visited = (m & 0x80) != 0
    pairs = decode_pairs_per_head(Sq, Skv, causal, window) * B * Hq
    flagged = int((bits * ent[None, None]).sum())
    vsb = int(((ent[None, None] > 0) & visited[..., None]).sum())
    fsb = int((bits * (ent[None, None] > 0)).sum())
    return dict(ms_per_step=total_ms / steps, attn_ms=attn_ms / max(ncalls, 1),
                prep_ms=prep_ms / max(ncalls, 1), pairs=pairs, f_nom=4.0 * D * pairs,
                f_qk8=2.0 * D * pairs, f_pv=2.0 * D * pairs, f_qk16=2.0 * D * flagged,
                stats=dict(r_sb=fsb / vsb if vsb else 0.0, r_e=flagged / pairs if pairs else 0.0,
                           visited_subblocks=vsb, flagged_subblocks=fsb))


def _oracle_decode_head(head):
    """Worker: one (b, hq) decode head through the oracle (CPU baseline only)."""
    from oracle import lamp as L
    b, hq, tps = head
    for tr in L.split_tiles(L.n_tiles(_CTX["S"]), tps):
        with np.errstate(invalid="ignore", divide="ignore"):
            L.run_unit(_CTX, b, hq, 0, tiles=tr)
    return head


def cpu_baseline_decode(q, k, v, cfg, delta, tau, tps, budget_s, cores):
    """Time the oracle on sampled heads of the decode workload (reported baseline)."""
    global _CTX
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    from oracle import lamp as L
    threadpool_limits(1)
    _CTX = L.prepare(q, k, v, cfg["causal"], cfg["window"], delta, tau)
    B, Hq, Sq, D = q.shape
    Skv = k.shape[2]
    rng = np.random.default_rng(321)
    heads = [(int(rng.integers(B)), int(rng.integers(Hq)), tps) for _ in range(4096)]
    t0 = time.perf_counter()
    _oracle_decode_head(heads[0])
    one = max(time.perf_counter() - t0, 1e-3)
    n = max(1, min(len(heads), int(budget_s * cores / one)))
    sample = heads[:n]
    t0 = time.perf_counter()
    if cores > 1 and n > 1:
        with mp.get_context("fork").Pool(min(cores, n)) as pool:
            for _ in pool.imap_unordered(_oracle_decode_head, sample, chunksize=1):
                pass
    else:
        for h in sample:
            _oracle_decode_head(h)
    wall = time.perf_counter() - t0
    flops = 4.0 * D * decode_pairs_per_head(Sq, Skv, cfg["causal"], cfg["window"]) * len(sample)
    return dict(value=flops / wall / 1e12, unit="TFLOP/s", cores=min(cores, n), kind="oracle",
                sample=f"{len(sample)} random (batch, query head) decode heads of the same workload, "
                       f"{tps} tiles per split ({flops / 1e9:.2f} GFLOP nominal), {wall:.1f} s wall")


def run_decode(args, cfg, q, k, v):
    """The decode bench line: lamp_attn_decode on a decode workload."""
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    causal, window = cfg["causal"], cfg["window"]
    # the library's split choice depends on the device; the CPU baseline
    # needs it before the GPU is touched, so it asks in a child process
    import subprocess
    tps = int(subprocess.run(
        [sys.executable, "-c", "import mixed_precision_attention_lamp_amd as l; "
         f"print(l.lamp_decode_tiles_per_split({B}, {Hq}, {Hkv}, {Sq}, {Skv}, {D}))"],
        capture_output=True, text=True, check=True, cwd=ROOT).stdout.strip())
    cb = None
    if not args.no_cpu_baseline:
        cores = max(1, min(len(os.sched_getaffinity(0)), 16))
        # the first head also quantises its K and V slabs, so it overstates the
        # per-head time about fourfold: a quarter of the budget gives the
        # prefill line's 20-30 s of CPU work
        cb = cpu_baseline_decode(q, k, v, cfg, args.delta, args.tau, tps, args.cpu_budget / 4, cores)
    import torch
    import mixed_precision_attention_lamp_amd as lamp
    dev = torch.device("cuda:0")

    def dev_t(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    qd, kd, vd = dev_t(q), dev_t(k), dev_t(v)
    nT = lamp.n_tiles(Skv)
    out = torch.empty((B, Hq, Sq, D), dtype=torch.float32, device=dev)
    mask = torch.empty((B, Hq, nT), dtype=torch.uint8, device=dev)
    kept = None
    if args.kept_amax:
        # the cache's kept K maxima, built once; each step folds in the Sq
        # newest keys (the positions the queries sit at) and decodes
        state = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
        lamp.lamp_kv_amax_update(kd, state)
        kept = (state, kd[:, :, Skv - Sq:].contiguous())
    m = measure_decode(lamp, torch, (qd, kd, vd, out, mask), (B, Hq, Hkv, Sq, Skv, D), causal, window,
                       args.delta, args.tau, tps, args.steps, args.warmup, settle_ms=args.settle_ms, kept=kept)
    n_split = (nT + tps - 1) // tps
    # algorithmic bytes of the decode kernel: K and V read once (bf16), Q
    # read, the split results and the mask bytes written
    part = 4.0 * B * Hq * n_split * Sq * (D + 2)
    kv_bytes = 2.0 * 2.0 * B * Hkv * Skv * D
    alg_bytes = kv_bytes + 2.0 * B * Hq * Sq * D + part + 1.0 * B * Hq * nT
    achieved = alg_bytes / (m["attn_ms"] * 1e-3)
    traffic = None
    if (TRAFFIC_DECODE["kernel_hash"] == decode_source_hash() and TRAFFIC_DECODE["workload"] == args.workload
            and TRAFFIC_DECODE["delta"] == args.delta and TRAFFIC_DECODE["tau"] == args.tau):
        traffic = TRAFFIC_DECODE["bytes_per_launch"]
    res = {
        "metric": METRIC,
        "value": m["f_nom"] / (m["ms_per_step"] * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3+bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {cfg['desc']}", "B": B, "Hq": Hq, "Hkv": Hkv,
                   "Sq": Sq, "Skv": Skv, "D": D, "causal": causal, "window": window,
                   "delta": args.delta, "tau": args.tau, "tiles_per_split": tps, "splits": n_split,
                   "k_scales": "kept maxima, the Sq newest keys folded in per step" if args.kept_amax
                   else "amax pass over the cache per step"},
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM, "traffic": traffic},
        "kernel_ms": {"decode": m["attn_ms"], "amax_and_scales": m["prep_ms"]},
        "step_hbm_frac": (kv_bytes + 2.0 * B * Hkv * Skv * D) / (m["ms_per_step"] * 1e-3) / PEAK_HBM,
        "recompute": {"r_sb": m["stats"]["r_sb"], "r_e": m["stats"]["r_e"]},
        "cpu_baseline": cb,
    }
    print(json.dumps(res), flush=True)


# The (delta, tau) grid of the pages' tables and figures, plus the two
# endpoints of the method: tau = +inf (no 16-bit recompute: the pure 8-bit
# Q.K^T path) and delta = tau = 0 (every visible sub-block recomputed in 16 bit).
GRID_DELTAS = (0.0, 2.0 ** -8, 2.0 ** -4)
GRID_TAUS = tuple(2.0 ** -i for i in range(6))
GRID_ENDPOINTS = ((2.0 ** -8, float("inf"), "8-bit Q.K^T only"), (0.0, 0.0, "all sub-blocks 16-bit"))
PLAIN_NOTE = "plain bf16 FlashAttention (no 8-bit pass)"
LOGIT8_NOTE = "8-bit logits (e4m3-rounded log2-domain logit)"
LOGIT8_POINTS = ((2.0 ** -8, 2.0 ** -1), (2.0 ** -8, float("inf")), (2.0 ** -4, 2.0 ** -1))
EXP2POLY_NOTE = "8-bit exponentials by the bit-reproducible polynomial exp2"
EXP2POLY_POINTS = ((2.0 ** -8, 2.0 ** -1), (2.0 ** -8, float("inf")), (2.0 ** -4, 2.0 ** -1))


def settle(torch, step, settle_ms):
    """Run the step until `settle_ms` of wall time have passed, before the
    warm-up steps: the GPU's clocks take on the order of a hundred launches
    of this kernel to reach their sustained level, and the timed steps are
    meant to see that level.  Returns the number of steps run."""
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(20):
            step()
        n += 20
        torch.cuda.synchronize()
    return n


def measure(lamp, torch, tensors, shape, causal, window, delta, tau, steps, warmup, plain=False,
            logit8=False, settle_ms=0.0, exp_poly=False):
    """Time `steps` calls of lamp_attn_fwd (lamp_attn_fwd_bf16 when plain,
    lamp_attn_fwd_logit8 when logit8, lamp_attn_fwd_exp2poly when exp_poly)
    after `warmup` untimed ones; returns the
    step time, the attention kernel
    time (HIP events on its stream), the algorithmic FLOP counts and the
    sub-block statistics of the last call."""
    qd, kd, vd, out, mask = tensors
    B, Hq, Hkv, S, D = shape

    def step():
        if plain:
            lamp.lamp_attn_fwd_bf16(qd, kd, vd, out, causal, window, mask)
        elif logit8:
            lamp.lamp_attn_fwd_logit8(qd, kd, vd, out, causal, window, delta, tau, mask)
        elif exp_poly:
            lamp.lamp_attn_fwd_exp2poly(qd, kd, vd, out, causal, window, delta, tau, mask)
        else:
            lamp.lamp_attn_fwd(qd, kd, vd, out, causal, window, delta, tau, mask)

    settle_steps = settle(torch, step, settle_ms)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    lamp.lamp_set_timing(1)
    lamp.lamp_read_timing()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    prep_ms, attn_ms, ncalls = lamp.lamp_read_timing()
    lamp.lamp_set_timing(0)
    stats = lamp.subblock_stats(mask, S, causal, window)
    pairs = visible_pairs_per_head(S, causal, window) * B * Hq
    assert pairs == stats["visible_entries"], (pairs, stats["visible_entries"])
    f_qk8 = 0.0 if plain else 2.0 * D * pairs
    f_pv = 2.0 * D * pairs
    f_qk16 = 2.0 * D * stats["flagged_entries"]
    return dict(ms_per_step=total_ms / steps, attn_ms=attn_ms / max(ncalls, 1),
                prep_ms=prep_ms / max(ncalls, 1), pairs=pairs, f_nom=4.0 * D * pairs,
                f_qk8=f_qk8, f_pv=f_pv, f_qk16=f_qk16, stats=stats, settle_steps=settle_steps)


def graph_step_ms(lamp, torch, tensors, causal, window, delta, tau, steps):
    """The same step captured once in a HIP graph (lamp_attn_fwd_noalloc: no
    allocation, no memset) and replayed `steps` times; returns ms per replay,
    or None when the workspace exceeds the entry point's fixed scratch array."""
    qd, kd, vd, out, mask = tensors
    try:
        lamp.lamp_attn_fwd_noalloc(qd, kd, vd, out, causal, window, delta, tau, mask)
    except lamp.LampError:
        return None
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side, capture_error_mode="relaxed"):
            lamp.lamp_attn_fwd_noalloc(qd, kd, vd, out, causal, window, delta, tau, mask)
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(20):
        g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    del g
    return start.elapsed_time(end) / steps


def roofline_of(m):
    """Blended matrix-core roofline of the attention kernel for one measurement."""
    f_alg = m["f_qk8"] + m["f_pv"] + m["f_qk16"]
    t_mfma = m["f_qk8"] / PEAK_FP8 + (m["f_pv"] + m["f_qk16"]) / PEAK_BF16
    peak = f_alg / t_mfma
    achieved = f_alg / (m["attn_ms"] * 1e-3)
    return achieved, peak


def run_grid(args, lamp, torch, tensors, shape, causal, window, cfg):
    """One JSON line per (delta, tau) of the grid and per endpoint."""
    runs = [(d, t, "") for d in GRID_DELTAS for t in GRID_TAUS] + list(GRID_ENDPOINTS)
    runs.append((0.0, 0.0, PLAIN_NOTE))
    runs += [(d, t, LOGIT8_NOTE) for d, t in LOGIT8_POINTS]
    runs += [(d, t, EXP2POLY_NOTE) for d, t in EXP2POLY_POINTS]
    for delta, tau, note in runs:
        m = measure(lamp, torch, tensors, shape, causal, window, delta, tau, args.steps, args.warmup,
                    settle_ms=args.settle_ms / 3,
                    plain=note == PLAIN_NOTE, logit8=note == LOGIT8_NOTE, exp_poly=note == EXP2POLY_NOTE)
        achieved, peak = roofline_of(m)
        print(json.dumps({
            "grid": args.workload, "delta": delta, "tau": tau if tau != float("inf") else "inf",
            "note": note, "ms_per_step": m["ms_per_step"], "attention_ms": m["attn_ms"],
            "nominal_tflops": m["f_nom"] / (m["ms_per_step"] * 1e-3) / 1e12,
            "roofline_frac": achieved / peak, "r_sb": m["stats"]["r_sb"], "r_e": m["stats"]["r_e"],
            "workload": cfg["desc"]}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="qwen3-8b")
    ap.add_argument("--delta", type=float, default=2.0 ** -8)
    ap.add_argument("--tau", type=float, default=2.0 ** -1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="run the step this long before the warm-up steps (clock settling)")
    ap.add_argument("--copy-calibrate", action="store_true")
    ap.add_argument("--kept-amax", action="store_true",
                    help="decode workloads: K scales from kept maxima (lamp_attn_decode_with_amax)")
    ap.add_argument("--exp2poly", action="store_true",
                    help="prefill workloads: the variant with the bit-reproducible polynomial exp2 "
                         "(lamp_attn_fwd_exp2poly), against the oracle's reading of it")
    ap.add_argument("--grid", action="store_true",
                    help="time the (delta, tau) grid and the two endpoints instead of one point")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the kernels run on one GPU only (asked for --gpus {args.gpus}); "
              "the path is single-GPU by design", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibrate:
        copy_calibrate()
        return

    from inputs import make_config_inputs

    q, k, v, cfg = make_config_inputs(args.workload)
    if "Sq" in cfg:
        if args.exp2poly:
            print("bench.py: --exp2poly applies to the prefill workloads only", file=sys.stderr)
            sys.exit(2)
        run_decode(args, cfg, q, k, v)
        return
    if args.exp2poly and args.grid:
        print("bench.py: --grid already times the polynomial-exp2 points; drop --exp2poly", file=sys.stderr)
        sys.exit(2)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    causal, window = cfg["causal"], cfg["window"]

    # The CPU baseline runs first, in worker processes forked before this
    # process touches the GPU.
    cb, expectations = None, {}
    if not args.no_cpu_baseline and not args.grid:
        # the machine's CPU share is 16 threads per GPU, whatever the host shows
        cores = max(1, min(len(os.sched_getaffinity(0)), 16))
        cb, expectations = cpu_baseline(q, k, v, cfg, args.delta, args.tau, args.cpu_budget, cores,
                                        exp_poly=args.exp2poly)
        cb.pop("wall_s", None)

    import torch
    import mixed_precision_attention_lamp_amd as lamp
    dev = torch.device("cuda:0")

    def dev_t(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    qd, kd, vd = dev_t(q), dev_t(k), dev_t(v)
    nT = lamp.n_tiles(S)
    out = torch.empty((B, Hq, S, D), dtype=torch.float32, device=dev)
    mask = torch.empty((B, Hq, nT, nT), dtype=torch.uint8, device=dev)

    tensors = (qd, kd, vd, out, mask)
    shape = (B, Hq, Hkv, S, D)
    if args.grid:
        run_grid(args, lamp, torch, tensors, shape, causal, window, cfg)
        return
    m = measure(lamp, torch, tensors, shape, causal, window, args.delta, args.tau, args.steps,
                args.warmup, settle_ms=args.settle_ms, exp_poly=args.exp2poly)
    parity = parity_block(expectations, out.cpu().numpy(), mask.cpu().numpy()) if expectations else None
    ms_per_step, attn_ms_avg, prep_ms_avg = m["ms_per_step"], m["attn_ms"], m["prep_ms"]
    stats, f_nom = m["stats"], m["f_nom"]
    achieved, blended_peak = roofline_of(m)
    nq, nk = B * Hq * S * D, B * Hkv * S * D
    quant_bytes = 3.0 * (nq + nk)
    # algorithmic bytes of the launches before the attention kernel: Q and K
    # read for their maxima, K read again and its e4m3 codes written, V read
    # and written transposed
    prep_bytes = 2.0 * (nq + nk) + 3.0 * nk + 4.0 * nk
    t_mfma = m["f_qk8"] / PEAK_FP8 + (m["f_pv"] + m["f_qk16"]) / PEAK_BF16
    t_roof = t_mfma + quant_bytes / PEAK_HBM
    # the stricter form: the attention kernel bounded by the larger of its
    # matrix-core time and its minimum HBM traffic (Q8, Q16 and the fp32
    # output; K8, K16 and V: 7 Nq + 5 Nk bytes), plus the quantisation pass
    t_roof_strict = max(t_mfma, (7.0 * nq + 5.0 * nk) / PEAK_HBM) + quant_bytes / PEAK_HBM
    valu_ceiling = None
    # the records were taken on the default kernel, not on the variant
    vrec = None if args.exp2poly else _record(VALU_CEILING, args, kernel_source_hash())
    if vrec is not None:
        t_valu = vrec["cycles_per_simd"] / vrec["clock_hz"]
        valu_ceiling = {"bound": "valu", "ceiling_ms": t_valu * 1e3, "frac": t_valu / (attn_ms_avg * 1e-3),
                        "source": "instruction counters, " + vrec["source"]}
    trec = None if args.exp2poly else _record(TRAFFIC, args, kernel_source_hash())
    traffic = trec["bytes_per_launch"] if trec is not None else None
    res = {
        "metric": METRIC,
        "value": f_nom / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3+bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {cfg['desc']}", "B": B, "Hq": Hq, "Hkv": Hkv,
                   "S": S, "D": D, "causal": causal, "window": window,
                   "delta": args.delta, "tau": args.tau,
                   "exp2": "bit-reproducible polynomial (lamp_attn_fwd_exp2poly)" if args.exp2poly
                   else "hardware v_exp_f32"},
        "roofline": {"bound": "mfma", "achieved": achieved / 1e12, "peak": blended_peak / 1e12,
                     "unit": "TFLOP/s", "frac": achieved / blended_peak, "traffic": traffic},
        "valu_ceiling": valu_ceiling,
        "blended_roofline_frac": t_roof / (ms_per_step * 1e-3),
        "strict_roofline_frac": t_roof_strict / (ms_per_step * 1e-3),
        "executed_tflops": (f_nom + m["f_qk16"]) / (attn_ms_avg * 1e-3) / 1e12,
        "kernel_ms": {"attention": attn_ms_avg, "quantise_and_transpose": prep_ms_avg},
        "prep_hbm": {"bytes": prep_bytes, "GB/s": prep_bytes / (prep_ms_avg * 1e-3) / 1e9,
                     "frac": prep_bytes / (prep_ms_avg * 1e-3) / PEAK_HBM},
        "settle_steps": m["settle_steps"],
        "recompute": {"r_sb": stats["r_sb"], "r_e": stats["r_e"], "hist_0_to_4": stats["hist"],
                      "tiles_0_1_2plus": stats["pages_buckets"]},
    }
    # the same step as one HIP-graph replay (after the timed region, not part of `value`)
    try:
        if args.exp2poly:
            raise RuntimeError("the graph replays the default entry point")
        res["graph_ms_per_step"] = graph_step_ms(lamp, torch, tensors, causal, window, args.delta, args.tau,
                                                 args.steps)
    except Exception as e:   # an informational figure: never lose the line for it
        print(f"bench.py: graph replay not timed ({e})", file=sys.stderr)
        torch.cuda.synchronize()
        res["graph_ms_per_step"] = None
    res["parity"] = parity
    res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
