#!/usr/bin/env python3
"""Benchmark of the RAT+ dilated operator on one MI355X.

Default run (one JSON line): the long prefill B=1, 16 heads x 128,
T=262144, D=64, W=0, bf16 (one step = one rat_dilated_prefill call:
recurrence over keys and values plus dilated attention) gives `value` in
tokens/s; the hybrid-head decode (batch 128, 32 heads x 128, context
131072, D = 8 x 1, 12 x 16, 12 x 64, W=64, 1024 steps) is reported under
"decode"; the tiny fp32 prefill, the T=16384 prefill and the batch-256
decode under "other_configs".  Each workload carries the roofline of its
kernels and a CPU baseline: the fp64 oracle over a pool of host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps N]
                    [--no-decode] [--no-other-configs] [--no-cpu-baseline]
                    [--config N]

--config N measures one workload alone: 1-3 prefill (tiny fp32, T=16384,
T=262144), 4-5 decode (batched, hybrid heads), 6 chunked prefill, 7-8 top-k
decode and prefill, 9 RAT chunk-local prefill, 10 hybrid-head prefill.
Inputs are seeded synthetic data generated on the GPU and resident in HBM
before timing.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15         # flop/s, dense bf16 MFMA
PEAK_F32_VALU = 157.3e12   # flop/s, fp32 vector

CONFIGS = {
    1: dict(kind="prefill", B=1, H=2, Dh=64, T=1024, D=4, W=0, dtype="f32", mu=2.0),
    2: dict(kind="prefill", B=1, H=16, Dh=128, T=16384, D=16, W=128, dtype="bf16", mu=2.0),
    3: dict(kind="prefill", B=1, H=16, Dh=128, T=262144, D=64, W=0, dtype="bf16", mu=3.0),
    4: dict(kind="decode", B=256, H=16, Dh=128, ctx=32768, D=[16] * 16, W=64, steps=1024, mu=2.0,
            dtype="bf16"),
    5: dict(kind="decode", B=128, H=32, Dh=128, ctx=131072, D=[1] * 8 + [16] * 12 + [64] * 12, W=64,
            steps=1024, mu=2.0, dtype="bf16"),
    # auxiliary workloads of the operator's other forms (not the headline line)
    6: dict(kind="chunked", B=1, H=16, Dh=128, T=16384, D=16, W=128, chunk=4096, dtype="bf16", mu=2.0),
    7: dict(kind="topk_decode", B=128, H=16, Dh=128, ctx=32768, block=64, topk=16, score=0, steps=256,
            dtype="bf16", mu=2.0),
    8: dict(kind="topk_prefill", B=1, H=16, Dh=128, T=4096, block=64, topk=16, score=1, dtype="bf16", mu=2.0),
    9: dict(kind="local", B=1, H=16, Dh=128, T=16384, L=16, dtype="bf16", mu=2.0),
    # prefill of the hybrid-head mix (per-head dilation, ragged compact grid)
    10: dict(kind="prefill", B=1, H=32, Dh=128, T=16384, D=[1] * 8 + [16] * 12 + [64] * 12, W=64, dtype="bf16",
             mu=2.0),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "recurrence_augmented_dilated_amd", "csrc")
KERNEL_SOURCES = {"scan": ["scan.hip", "rat_internal.h"], "attention": ["prefill_attn.hip", "rat_internal.h"],
                  "attention_f32": ["prefill_attn.hip", "rat_internal.h"],
                  "decode": ["decode.hip", "kv_stream.h", "rat_internal.h"],
                  "topk_attend": ["topk.hip", "kv_stream.h", "rat_internal.h"],
                  "topk_stats": ["topk.hip", "rat_internal.h"], "topk_append": ["topk.hip", "rat_internal.h"],
                  "grid_to_col": ["chunk.hip", "rat_internal.h"], "ring_prefix": ["chunk.hip", "rat_internal.h"],
                  "topk_select": ["topk.hip", "rat_internal.h"]}


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload_key):
    """HBM bytes per launch from a committed rocprofv3 counter profile, or None
    if there is none for this kernel/workload or the kernel source changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_key}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        prof = json.load(fh)
    if prof.get("source_sha256") != source_hash(kernel):
        return None
    return prof.get("hbm_bytes_per_dispatch")


# ---------------------------------------------------------------------------
# work model (algorithmic bytes and flops; counts from the key-set ranges)
# ---------------------------------------------------------------------------

def prefill_pairs(T, D, W):
    import numpy as np
    t = np.arange(T, dtype=np.int64)
    grid = np.maximum(0, t - W + 1) // D
    win = np.minimum(W, t + 1)
    return int(grid.sum() + win.sum())


def prefill_work(c):
    B, H, Dh, T, D, W = c["B"], c["H"], c["Dh"], c["T"], c["D"], c["W"]
    Ds = D if isinstance(D, list) else [D] * H     # dilation per head
    e = 2 if c["dtype"] == "bf16" else 4
    n = B * T * H * Dh
    scan_read = 2 * n * (e + 4)                    # x and fp32 logits, keys and values
    scan_write = 2 * n * e if W > 0 else 2 * B * sum(T // d for d in Ds) * Dh * e
    pairs = sum(prefill_pairs(T, d, W) for d in Ds) * B
    flops = 4 * Dh * pairs
    return dict(scan_bytes=scan_read + scan_write, attn_flops=flops, pairs=pairs)


def decode_step_bytes(c, t):
    """Algorithmic HBM bytes of one decode step with every sequence at position t."""
    B, H, Dh, W = c["B"], c["H"], c["Dh"], c["W"]
    e = 2
    total = 0
    for D in c["D"]:
        n_g = max(0, t - W + 1) // D
        n_w = min(W, t + 1) if W > 0 else 0
        rows = n_g + max(0, n_w - 1)           # the newest state comes from registers
        kv = rows * Dh * e * 2
        state = Dh * 4 * 2 * 2                  # fp32 state read + write, keys and values
        new = Dh * (3 * e + 2 * 4)              # q, k, v, zk, zv
        writes = Dh * e * 2 * ((1 if W > 0 else 0) + (1 if (t + 1) % D == 0 else 0))
        out = Dh * e
        total += kv + state + new + writes + out
    return B * total


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------

def time_loop(fn, steps, torch):
    """Average ms per call of fn() with HIP events on the current stream."""
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / steps


def bench_prefill(c, steps, warmup, torch, R, inputs):
    dev = "cuda:0"
    dt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    log(f"[bench] prefill inputs B={c['B']} T={c['T']} H={c['H']} Dh={c['Dh']} D={c['D']} W={c['W']}")
    x = inputs.prefill_inputs(c["B"], c["T"], c["H"], c["Dh"], dtype=dt, mu=c["mu"], seed=2, device=dev)
    out = torch.empty_like(x["q"])
    ws_bytes = R.rat_dilated_prefill_workspace_size(c["B"], c["T"], c["H"], c["Dh"], c["D"], c["W"], dt)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    args = (x["q"], x["k"], x["v"], x["zk"], x["zv"], c["D"], c["W"])

    def step():
        R.rat_dilated_prefill(*args, out=out, ws=ws)

    def scan_only():
        R.rat_dilated_prefill_stage(1, *args, out=out, ws=ws)

    def attn_only():
        R.rat_dilated_prefill_stage(2, *args, out=out, ws=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # single-call API (both kernels behind one rat_dilated_prefill call)
    ms_call = time_loop(step, steps, torch)

    # Timed region: the same two launches issued stage by stage, with HIP
    # events between them on the stream they run on, so each kernel's
    # duration is measured inside the region that gives the step time.
    # One event per step boundary (a step ends where the next begins) and
    # one between the two launches of a step.
    s = torch.cuda.current_stream()
    eb = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    em = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    eb[0].record(s)
    for i in range(steps):
        scan_only()
        em[i].record(s)
        attn_only()
        eb[i + 1].record(s)
    eb[-1].synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    ms = eb[0].elapsed_time(eb[-1]) / steps
    ms_scan = sum(eb[i].elapsed_time(em[i]) for i in range(steps)) / steps
    ms_attn = sum(em[i].elapsed_time(eb[i + 1]) for i in range(steps)) / steps
    # the single-call API once more, now as warm as the staged loop
    ms_call_after = time_loop(step, steps, torch)
    err = R.workspace_error(ws)
    log(f"[bench] prefill {ms:.3f} ms/step (wall {wall:.3f}; single call {ms_call:.3f} before, "
        f"{ms_call_after:.3f} after); scan {ms_scan:.3f} ms, attention {ms_attn:.3f} ms per launch; ws error {err}")
    return dict(ms=ms, ms_call=ms_call, ms_call_after=ms_call_after, wall_ms=wall, ms_scan=ms_scan, ms_attn=ms_attn,
                x=x, out=out,
                ws_error=err, inputs_sha256=inputs.sha256_of(x["q"], x["k"], x["v"], x["zk"], x["zv"]))


def bench_decode(c, steps, warmup, torch, R, inputs):
    dev = "cuda:0"
    B, H, Dh, W = c["B"], c["H"], c["Dh"], c["W"]
    dil = c["D"]
    max_pos = c["ctx"] + max(steps, warmup)
    off, cap, rows = R.rat_grid_layout(H, dil, max_pos)
    log(f"[bench] decode cache B={B} H={H} ctx={c['ctx']} rows/seq={rows} "
        f"({2 * B * rows * Dh * 2 / 1e9:.1f} GB)")
    cache = inputs.decode_cache(B, H, Dh, dil, W, c["ctx"], max(steps, warmup), seed=4, device=dev)
    assert cache["layout"].cap == cap and cache["layout"].off == off
    n_in = max(steps, warmup)
    st = inputs.decode_step_inputs(B, H, Dh, n_in, mu=c["mu"], seed=5, device=dev)
    pos = torch.full((B,), c["ctx"], dtype=torch.int32, device=dev)
    out = torch.empty((B, H, Dh), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(R.rat_decode_workspace_size(B, H, Dh, dil, W, max_pos), dtype=torch.uint8, device=dev)

    def run(n):
        for i in range(n):
            R.rat_decode_step(st["q"][i], st["k"][i], st["v"][i], st["zk"][i], st["zv"][i],
                              cache["state_k"], cache["state_v"], cache["grid_k"], cache["grid_v"],
                              off, cap, cache["ring_k"], cache["ring_v"], pos, max_pos, dil, W,
                              out=out, ws=ws)
            pos.add_(1)

    run(warmup)
    torch.cuda.synchronize()
    pos.fill_(c["ctx"])
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s)
    run(steps)
    e1.record(s)
    e1.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    err = R.workspace_error(ws)
    bytes_avg = sum(decode_step_bytes(c, c["ctx"] + i) for i in range(steps)) / steps
    log(f"[bench] decode {ms:.3f} ms/step, {bytes_avg / (ms * 1e-3) / 1e9:.0f} GB/s, ws error {err}")
    return dict(ms=ms, wall_s=wall, bytes_per_step=bytes_avg, ws_error=err, steps=steps)


# ---------------------------------------------------------------------------
# auxiliary workloads: chunked prefill, top-k block attention, chunk-local
# ---------------------------------------------------------------------------

def bench_chunked(c, steps, warmup, torch, R, inputs):
    """Config-2 sequence prefilled in chunks into a decode cache (handoff)."""
    dev = "cuda:0"
    B, H, Dh, T, D, W, ch = c["B"], c["H"], c["Dh"], c["T"], c["D"], c["W"], c["chunk"]
    x = inputs.prefill_inputs(B, T, H, Dh, dtype=torch.bfloat16, mu=c["mu"], seed=2, device=dev)
    max_pos = T + 1024
    off, cap, rows = R.rat_grid_layout(H, [D] * H, max_pos)
    gk = torch.zeros(B * rows * Dh, dtype=torch.bfloat16, device=dev)
    gv = torch.zeros_like(gk)
    rk = torch.zeros((B, H, W, Dh), dtype=torch.bfloat16, device=dev)
    rv = torch.zeros_like(rk)
    sk = torch.zeros((B, H, Dh), dtype=torch.float32, device=dev)
    sv = torch.zeros_like(sk)
    parts = [{n: t[:, p0:p0 + ch].contiguous() for n, t in x.items()} for p0 in range(0, T, ch)]
    out = torch.empty((B, ch, H, Dh), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(max(R.rat_prefill_chunk_workspace_size(B, ch, H, Dh, [D] * H, W, p0) for p0 in range(0, T, ch)),
                     dtype=torch.uint8, device=dev)

    def step():
        sk.zero_()
        sv.zero_()
        for i, d in enumerate(parts):
            R.rat_prefill_chunk(d["q"], d["k"], d["v"], d["zk"], d["zv"], sk, sv, gk, gv, off, cap, rk, rv, i * ch,
                                max_pos, [D] * H, W, out=out, ws=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms = time_loop(step, steps, torch)
    log(f"[bench] chunked prefill ({T // ch} chunks of {ch}) {ms:.3f} ms/sequence")
    return ms


def topk_decode_bytes(c, t):
    """Algorithmic HBM bytes of one top-k decode step at position t."""
    B, H, Dh, blk, k = c["B"], c["H"], c["Dh"], c["block"], c["topk"]
    local = t // blk
    ncand = max(0, local - 1)
    nstats = 2 if c["score"] == 0 else 1                  # Quest reads min and max, MoBA the mean
    kept = min(k, ncand) * blk + (blk if local > 0 else 0) + (t - local * blk + 1)
    per = (3 * Dh * 2 + 2 * Dh * 4          # q, k, v, zk, zv
           + 2 * 2 * Dh * 4                 # fp32 states read and written
           + 2 * Dh * 2                     # the new cache rows
           + ncand * nstats * Dh * 4        # summaries of the candidate blocks
           + kept * Dh * 2 * 2              # key and value rows of the kept blocks
           + Dh * 2)                        # output
    if (t + 1) % blk == 0:
        per += blk * Dh * 2 + 3 * Dh * 4    # summary of the completed block
    return B * H * per


def bench_topk_decode(c, steps, warmup, torch, R):
    dev = "cuda:0"
    B, H, Dh, blk, k, ctx = c["B"], c["H"], c["Dh"], c["block"], c["topk"], c["ctx"]
    max_pos = ctx + max(steps, warmup) + blk
    max_pos = (max_pos + blk - 1) // blk * blk
    cache = R.topk_cache(B, H, Dh, max_pos, blk, torch.bfloat16, dev)
    from recurrence_augmented_dilated_amd import inputs
    inputs.fill_topk_cache(cache, seed=7)
    R.rat_topk_summarize(cache, 0, ctx // blk, max_pos, blk)
    n_in = max(steps, warmup)
    st = inputs.decode_step_inputs(B, H, Dh, n_in, mu=c["mu"], seed=5, device=dev)
    pos = torch.full((B,), ctx, dtype=torch.int32, device=dev)
    out = torch.empty((B, H, Dh), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(R.lib().rat_topk_decode_workspace_size(), dtype=torch.uint8, device=dev)

    def run(n):
        for i in range(n):
            R.rat_topk_decode_step(st["q"][i], st["k"][i], st["v"][i], st["zk"][i], st["zv"][i], cache, pos, max_pos,
                                   blk, k, c["score"], out=out, ws=ws)
            pos.add_(1)

    run(warmup)
    torch.cuda.synchronize()
    pos.fill_(ctx)
    ms = time_loop(lambda: run(1), steps, torch)
    err = R.workspace_error(ws)
    nbytes = sum(topk_decode_bytes(c, ctx + i) for i in range(steps)) / steps
    log(f"[bench] top-k decode {ms:.3f} ms/step, {nbytes / (ms * 1e-3) / 1e9:.0f} GB/s, ws error {err}")
    return ms, nbytes, err


def topk_prefill_flops(c):
    """Flops of top-k block prefill: (scoring every candidate block, the
    softmax attention over the kept positions, 4 Dh per kept pair)."""
    B, H, Dh, T, blk, k = c["B"], c["H"], c["Dh"], c["T"], c["block"], c["topk"]
    score = attn = 0
    for t in range(T):
        local = t // blk
        ncand = max(0, local - 1)
        kept = min(k, ncand) * blk + (blk if local > 0 else 0) + (t - local * blk + 1)
        score += (2 * Dh if c["score"] == 1 else 3 * Dh) * ncand
        attn += 4 * Dh * kept
    return B * H * score, B * H * attn


def bench_topk_prefill(c, steps, warmup, torch, R, inputs):
    dev = "cuda:0"
    B, H, Dh, T, blk, k = c["B"], c["H"], c["Dh"], c["T"], c["block"], c["topk"]
    x = inputs.prefill_inputs(B, T, H, Dh, dtype=torch.bfloat16, mu=c["mu"], seed=2, device=dev)
    max_pos = (T + blk - 1) // blk * blk
    cache = R.topk_cache(B, H, Dh, max_pos, blk, torch.bfloat16, dev)
    out = torch.empty_like(x["q"])
    ws = torch.zeros(R.lib().rat_topk_prefill_workspace_size(B, T, H, Dh), dtype=torch.uint8, device=dev)

    def step():
        cache["state_k"].zero_()
        cache["state_v"].zero_()
        R.rat_topk_prefill(x["q"], x["k"], x["v"], x["zk"], x["zv"], cache, 0, max_pos, blk, k, c["score"], out=out,
                           ws=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms = time_loop(step, steps, torch)
    log(f"[bench] top-k prefill {ms:.3f} ms/step")
    return ms


def bench_local(c, steps, warmup, torch, R, inputs):
    dev = "cuda:0"
    B, H, Dh, T, L = c["B"], c["H"], c["Dh"], c["T"], c["L"]
    x = inputs.prefill_inputs(B, T, H, Dh, dtype=torch.bfloat16, mu=c["mu"], seed=2, device=dev)
    max_pos = T + 64
    off, cap, rows = R.rat_grid_layout(H, [L] * H, max_pos)
    gk = torch.zeros(B * rows * Dh, dtype=torch.bfloat16, device=dev)
    gv = torch.zeros_like(gk)
    rk = torch.zeros((B, H, 1, Dh), dtype=torch.bfloat16, device=dev)
    rv = torch.zeros_like(rk)
    sk = torch.zeros((B, H, Dh), dtype=torch.float32, device=dev)
    sv = torch.zeros_like(sk)
    out = torch.empty_like(x["q"])

    def step():
        R.rat_local_prefill_chunk(x["q"], x["k"], x["v"], x["zk"], x["zv"], sk, sv, gk, gv, off, cap, rk, rv, 0,
                                  max_pos, L, out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms = time_loop(step, steps, torch)
    log(f"[bench] chunk-local prefill (L={L}) {ms:.3f} ms/step")
    return ms


def aux_result(cfg_id, c, a, torch, R, inputs):
    """One JSON result for an auxiliary workload (configs 6-9)."""
    res = {"unit": "tokens/s", "n_gpus": 1, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "data": "synthetic", "dtype": c["dtype"], "steps": a.steps, "warmup": a.warmup}
    kind = c["kind"]
    if kind in ("chunked", "local"):
        if kind == "chunked":
            ms = bench_chunked(c, a.steps, a.warmup, torch, R, inputs)
            w = prefill_work(c)
            wl = (f"chunked prefill B={c['B']} H={c['H']} Dh={c['Dh']} T={c['T']} in chunks of {c['chunk']} "
                  f"D={c['D']} W={c['W']} bf16 into a decode cache")
            metric = "chunked prefill tokens/s (prefill continuing a decode cache)"
        else:
            ms = bench_local(c, a.steps, a.warmup, torch, R, inputs)
            w = prefill_work(dict(c, D=c["L"], W=1))
            wl = f"RAT chunk-local prefill B={c['B']} H={c['H']} Dh={c['Dh']} T={c['T']} L={c['L']} bf16"
            metric = "chunk-local (RAT) prefill tokens/s"
        tfs = w["attn_flops"] / (ms * 1e-3)
        res.update(metric=metric, value=c["B"] * c["T"] / (ms * 1e-3), ms_per_step=ms,
                   config={"workload": wl, "config_id": cfg_id},
                   roofline={"kernel": "whole step (recurrence + attention)", "bound": "mfma",
                             "achieved": tfs / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                             "frac": tfs / PEAK_BF16, "traffic": None,
                             "note": "attention flops over the whole step time"})
    elif kind == "topk_decode":
        ms, nbytes, err = bench_topk_decode(c, a.steps, a.warmup, torch, R)
        gbs = nbytes / (ms * 1e-3)
        res.update(metric="top-k block attention decode tokens/s", value=c["B"] / (ms * 1e-3), ms_per_step=ms,
                   config={"workload": f"top-k decode B={c['B']} H={c['H']} Dh={c['Dh']} ctx={c['ctx']} "
                                       f"block={c['block']} topk={c['topk']} {'quest' if c['score'] == 0 else 'moba'}",
                           "config_id": cfg_id},
                   roofline={"kernel": "whole step (append + select + attend)", "bound": "hbm",
                             "achieved": gbs / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": gbs / PEAK_HBM,
                             "traffic": measured_traffic("topk_attend", f"topk_decode_config{cfg_id}")},
                   ws_error=err)
    elif kind == "topk_prefill":
        ms = bench_topk_prefill(c, a.steps, a.warmup, torch, R, inputs)
        _, fl = topk_prefill_flops(c)
        res.update(metric="top-k block attention prefill tokens/s", value=c["B"] * c["T"] / (ms * 1e-3),
                   ms_per_step=ms,
                   config={"workload": f"top-k prefill B={c['B']} H={c['H']} Dh={c['Dh']} T={c['T']} "
                                       f"block={c['block']} topk={c['topk']} {'quest' if c['score'] == 0 else 'moba'}",
                           "config_id": cfg_id},
                   roofline={"kernel": "whole step (recurrence + summaries + select + attend)", "bound": "mfma",
                             "achieved": fl / (ms * 1e-3) / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                             "frac": fl / (ms * 1e-3) / PEAK_BF16, "traffic": None,
                             "note": "attention flops of the kept (query, key) pairs over the whole step time"})
    return res


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle as it stands, over a pool of host cores
# ---------------------------------------------------------------------------

def cpu_workers():
    """Worker processes of the CPU baseline: the cores this process may run
    on, at most 16 (one GPU's share of the host)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_prefill_head(task):
    """Worker: one head of a prefill workload through the fp64 oracle, on
    inputs drawn here with the workload's shapes and distributions.  Times
    the full-length recurrence of keys and values and the attention of the
    sampled query rows (one BLAS thread).  Returns (scan s, attention s,
    sampled rows)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    T, Dh, D, W, mu, seed, n_rows = task
    with threadpool_limits(limits=1):
        rng = np.random.default_rng(seed)
        shp = (1, T, 1, Dh)
        q, k, v = (rng.standard_normal(shp) for _ in range(3))
        zk, zv = (mu + rng.standard_normal(shp) for _ in range(2))
        t0 = time.perf_counter()
        Kt = oracle.scan(k, zk)
        Vt = oracle.scan(v, zv)
        t1 = time.perf_counter()
        rows = list(range(T)) if n_rows >= T else sorted(int(r) for r in rng.choice(T, n_rows, replace=False))
        oracle.prefill(q, None, None, None, None, D, W, rows=rows, states=(Kt, Vt))
        t2 = time.perf_counter()
    return t1 - t0, t2 - t1, rows


def _oracle_decode_seq(task):
    """Worker: one sequence of a decode workload through the fp64 oracle's
    DecodeCache (every head; caches filled from N(0, 1) here with the
    workload's layout), `steps` steps from position ctx.  Returns the seconds
    of the steps."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    H, Dh, dil, W, ctx, max_pos, steps, mu, seed = task
    with threadpool_limits(limits=1):
        rng = np.random.default_rng(seed)
        n = lambda *s: rng.standard_normal(s)  # noqa: E731
        cache = oracle.DecodeCache(n(1, H, Dh), n(1, H, Dh), n(1, H, W, Dh), n(1, H, W, Dh),
                                   [np.zeros((1, 1, Dh))] * H, [np.zeros((1, 1, Dh))] * H, dil, W)
        # the grids are handed over as drawn (no second copy of ~2 GB)
        cache.grid_k = [n(1, max_pos // d, Dh) for d in dil]
        cache.grid_v = [n(1, max_pos // d, Dh) for d in dil]
        xs = [(n(1, H, Dh), n(1, H, Dh), n(1, H, Dh), mu + n(1, H, Dh), mu + n(1, H, Dh)) for _ in range(steps)]
        t0 = time.perf_counter()
        for i, (q, k, v, zk, zv) in enumerate(xs):
            cache.step(q, k, v, zk, zv, [ctx + i])
        return time.perf_counter() - t0


def _pool_map(fn, tasks, n):
    import multiprocessing as mp
    with mp.get_context("spawn").Pool(n) as pool:
        return pool.map(fn, tasks, chunksize=1)


def cpu_baseline_prefill(c, n_rows):
    """The fp64 oracle on every head of a prefill workload over a pool of
    worker processes (one head per task): the full-length recurrence and
    n_rows sampled query rows per head (every row if n_rows >= T), the
    attention time extrapolated by the key-set pairs to every row.  tokens/s
    = B T / (summed per-head seconds / workers)."""
    import numpy as np
    B, H, Dh, T, W = c["B"], c["H"], c["Dh"], c["T"], c["W"]
    Ds = c["D"] if isinstance(c["D"], list) else [c["D"]] * H
    tasks = [(T, Dh, Ds[h], W, c["mu"], 1000 + h, n_rows) for h in range(H)]
    n = min(cpu_workers(), len(tasks))
    t0 = time.perf_counter()
    res = _pool_map(_oracle_prefill_head, tasks, n)
    wall = time.perf_counter() - t0
    total = 0.0
    scan_s = attn_s = 0.0
    for (ts, ta, rows), d in zip(res, Ds):
        r = np.asarray(rows, dtype=np.int64)
        sampled = int((np.maximum(0, r - W + 1) // d + np.minimum(W, r + 1)).sum())
        full = prefill_pairs(T, d, W)
        total += ts + ta * full / max(sampled, 1)
        scan_s += ts
        attn_s += ta
    sec = B * total / n
    measured = n_rows >= T
    log(f"[bench] cpu baseline prefill: {H} heads over {n} workers, {wall:.1f} s wall "
        f"(scan {scan_s:.1f} s, attention {attn_s:.1f} s summed)")
    return dict(value=B * T / sec, unit="tokens/s", cores=n, kind="oracle", cpu_model=cpu_model(),
                sample=(f"fp64 oracle, {n} worker processes x 1 BLAS thread, one head per task, all {H} heads: "
                        f"the full {T}-step recurrence of keys and values and "
                        + ("every query row (measured)" if measured else
                           f"{n_rows} random query rows per head, the attention time scaled by key-set pairs "
                           f"to all {T} rows (extrapolated)")
                        + (f"; x B={B}" if B > 1 else "") + f"; inputs drawn on the host with the workload's "
                        f"shapes and distributions; {wall:.1f} s wall"))


def cpu_baseline_decode(c, n_seq, steps):
    """The fp64 oracle's decode step for n_seq sequences (every head) over a
    pool of worker processes, `steps` steps each from the workload's first
    position.  tokens/s = sequence-steps / (summed step seconds / workers)."""
    H, Dh, W, ctx = c["H"], c["Dh"], c["W"], c["ctx"]
    max_pos = ctx + c["steps"]
    tasks = [(H, Dh, c["D"], W, ctx, max_pos, steps, c["mu"], 2000 + i) for i in range(n_seq)]
    n = min(cpu_workers(), len(tasks))
    t0 = time.perf_counter()
    secs = _pool_map(_oracle_decode_seq, tasks, n)
    wall = time.perf_counter() - t0
    rate = n_seq * steps / (sum(secs) / n)
    log(f"[bench] cpu baseline decode: {n_seq} sequences x {steps} steps over {n} workers, {wall:.1f} s wall")
    return dict(value=rate, unit="tokens/s", cores=n, kind="oracle", cpu_model=cpu_model(),
                sample=(f"fp64 oracle DecodeCache.step, {n} worker processes x 1 BLAS thread: {n_seq} sequences "
                        f"(all {H} heads, caches of context {ctx} drawn from N(0,1) on the host in the workload's "
                        f"layout) x {steps} steps from position {ctx}; tokens/s = sequence-steps per summed "
                        f"worker second x {n} workers (measured); {wall:.1f} s wall"))


def measure_copy(torch):
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ms = time_loop(lambda: dst.copy_(src), 5, torch)
    del src, dst
    return 2 * n * 4 / (ms * 1e-3) / 1e9


# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# offline: rocprofv3 CSV output -> short summaries under profiles/ (CPU only)
# ---------------------------------------------------------------------------

KERNEL_PATTERNS = {"scan": ("scan_kernel", "scan_seg_kernel"), "attention": ("attn_bf16_kernel", "attn_bf16_stream_kernel"),
                   "attention_f32": "attn_f32_kernel",
                   "decode": "decode_kernel",
                   "topk_attend": "topk_attend_kernel", "topk_stats": "topk_stats_kernel",
                   "topk_append": "topk_append_kernel", "grid_to_col": "grid_to_col_kernel",
                   "ring_prefix": "ring_prefix_kernel", "topk_select": "topk_select_tile_kernel"}
COPY_BYTES = 1 << 30   # --calibrate-copy: bytes read and bytes written by one copy


def _pat_text(pat):
    """The kernel-name pattern(s) as text."""
    return pat if isinstance(pat, str) else " or ".join(pat)


def _matches(name, pat):
    """Whether a kernel name holds the pattern (or one of a tuple of them)."""
    return any(p in name for p in ((pat,) if isinstance(pat, str) else pat))


def _find_csv(d, suffix):
    import glob
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def _counter_rows(d, counter):
    import csv
    rows = []
    with open(_find_csv(d, "counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def summarize_pmc(kernel, workload, fetch_dir, write_dir, cfetch_dir, cwrite_dir, bench_args):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of `kernel`, scaled by what
    the same counters read for a plain copy of known size, into
    profiles/<kernel>_<workload>_pmc.json (+ .txt)."""
    pat = KERNEL_PATTERNS[kernel]
    fetch = [v for n, v in _counter_rows(fetch_dir, "FETCH_SIZE") if _matches(n, pat)]
    write = [v for n, v in _counter_rows(write_dir, "WRITE_SIZE") if _matches(n, pat)]
    # the calibration run's largest dispatch is the 1 GiB copy
    cf = max(v for _, v in _counter_rows(cfetch_dir, "FETCH_SIZE"))
    cw = max(v for _, v in _counter_rows(cwrite_dir, "WRITE_SIZE"))
    f_fetch = COPY_BYTES / (cf * 1024.0)
    f_write = COPY_BYTES / (cw * 1024.0)
    fk = sum(fetch) / len(fetch)
    wk = sum(write) / len(write)
    hbm = fk * 1024.0 * f_fetch + wk * 1024.0 * f_write
    cmds = [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o pmc -- python3 bench.py {bench_args}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o pmc -- python3 bench.py {bench_args}",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {cfetch_dir} -o pmc -- python3 bench.py --calibrate-copy",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {cwrite_dir} -o pmc -- python3 bench.py --calibrate-copy",
            f"python3 bench.py --summarize-pmc {kernel} {workload} {fetch_dir} {write_dir} {cfetch_dir} {cwrite_dir} "
            f"--pmc-bench-args '{bench_args}'"]
    out = {"kernel": kernel, "kernel_name_pattern": pat, "workload": workload, "source_sha256": source_hash(kernel),
           "dispatches": [len(fetch), len(write)], "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
           "copy_fetch_kib": cf, "copy_write_kib": cw, "factor_fetch": f_fetch, "factor_write": f_write,
           "hbm_bytes_per_dispatch": hbm, "commands": cmds}
    base = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc")
    with open(base + ".json", "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    with open(base + ".txt", "w") as fh:
        fh.write(f"HBM traffic of {kernel} ({_pat_text(pat)}) on workload {workload}\n\n")
        fh.write("\n".join("$ " + c for c in cmds) + "\n\n")
        fh.write(f"dispatches averaged: FETCH {len(fetch)}, WRITE {len(write)}\n")
        fh.write(f"FETCH_SIZE {fk:.1f} KiB/dispatch x {f_fetch:.3f} (1 GiB copy read {cf:.1f} KiB)\n")
        fh.write(f"WRITE_SIZE {wk:.1f} KiB/dispatch x {f_write:.3f} (1 GiB copy wrote {cw:.1f} KiB)\n")
        fh.write(f"HBM bytes per dispatch: {hbm:.4g}\n")
        fh.write(f"source sha256 of the kernel's files: {out['source_sha256']}\n")
    print(json.dumps(out))


def summarize_counters(kernel, workload, dirs, bench_args):
    """Every counter of one or more `rocprofv3 --pmc` runs (one counter set
    per directory, the sets named in each run's own log), averaged per
    dispatch of `kernel`, into profiles/<kernel>_<workload>_sq_counters.txt,
    with the ratios read from them."""
    import csv
    pat = KERNEL_PATTERNS[kernel]
    vals, cmds = {}, []
    for d in dirs:
        per = {}
        with open(_find_csv(d, "counter_collection.csv")) as fh:
            for r in csv.DictReader(fh):
                if _matches(r["Kernel_Name"], pat):
                    per.setdefault(r["Counter_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
                    per[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        for c, byd in per.items():
            vals[c] = sum(byd.values()) / len(byd)
        cmds.append(f"rocprofv3 --pmc {' '.join(sorted(per))} --output-format csv -d {d} -o pmc -- "
                    f"python3 bench.py {bench_args}")
    cmds.append(f"python3 bench.py --summarize-counters {kernel} {workload} {' '.join(dirs)} "
                f"--pmc-bench-args '{bench_args}'")
    lines = [f"SQ counters of {kernel} ({_pat_text(pat)}) on workload {workload}, per dispatch", ""]
    lines += ["$ " + c for c in cmds] + [""]
    lines += [f"{c:28s} {v:.4g}" for c, v in sorted(vals.items())]
    g = vals.get
    derived = []
    if g("SQ_WAVE_CYCLES"):
        for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU"):
            if g(c) is not None:
                derived.append(f"{c} / SQ_WAVE_CYCLES = {g(c) / g('SQ_WAVE_CYCLES'):.3f}")
    if g("SQ_VALU_MFMA_BUSY_CYCLES") and g("SQ_VALU_MFMA_COEXEC_CYCLES") is not None:
        derived.append("SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES = "
                       f"{g('SQ_VALU_MFMA_COEXEC_CYCLES') / g('SQ_VALU_MFMA_BUSY_CYCLES'):.3f}")
    if g("SQ_INSTS_MFMA"):
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VALU_TRANS_F32"):
            if g(c) is not None:
                derived.append(f"{c} / SQ_INSTS_MFMA = {g(c) / g('SQ_INSTS_MFMA'):.3f}")
    if derived:
        lines += ["", "derived:"] + derived
    lines += ["", f"source sha256 of the kernel's files: {source_hash(kernel)}"]
    with open(os.path.join(ROOT, "profiles", f"{kernel}_{workload}_sq_counters.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(trace_dir, kernel, workload, bench_args):
    """Launch statistics of `kernel` from a --kernel-trace --stats run into
    profiles/<kernel>_<workload>_kernel_trace.txt."""
    import csv
    path = _find_csv(trace_dir, "kernel_stats.csv")
    pat = KERNEL_PATTERNS[kernel]
    with open(path) as fh:
        rows = [r for r in csv.DictReader(fh) if _matches(r["Name"], pat)]
    lines = [f"rocprofv3 kernel statistics of {kernel} ({_pat_text(pat)}) on workload {workload}", "",
             f"$ rocprofv3 --kernel-trace --stats --output-format csv -d {trace_dir} -o kt -- python3 bench.py "
             f"{bench_args}",
             f"$ python3 bench.py --summarize-trace {trace_dir} {kernel} {workload} --pmc-bench-args '{bench_args}'",
             ""]
    # per-dispatch durations from the trace: the median, and the mean without
    # the first three (cold) dispatches, next to the --stats figures
    import statistics
    with open(_find_csv(trace_dir, "kernel_trace.csv")) as fh:
        trace = [r for r in csv.DictReader(fh) if _matches(r["Kernel_Name"], pat)]
    for r in rows:
        ds = [(int(t["End_Timestamp"]) - int(t["Start_Timestamp"])) / 1e3 for t in trace
              if t["Kernel_Name"] == r["Name"]]
        lines += [f"kernel: {r['Name']}",
                  f"calls {int(float(r['Calls']))}, average {float(r['AverageNs']) / 1e3:.2f} us, "
                  f"min {float(r['MinNs']) / 1e3:.2f} us, max {float(r['MaxNs']) / 1e3:.2f} us, "
                  f"{float(r['Percentage']):.2f}% of the run's kernel time"]
        if len(ds) > 3:
            lines += [f"per-dispatch trace: median {statistics.median(ds):.2f} us, "
                      f"mean after the first 3 dispatches {statistics.mean(ds[3:]):.2f} us"]
    with open(os.path.join(ROOT, "profiles", f"{kernel}_{workload}_kernel_trace.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="default line only: skip the T=1024, T=16384 and batch-256 decode sub-results")
    ap.add_argument("--config", type=int, default=0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--summarize-pmc", nargs=6, metavar=("KERNEL", "WORKLOAD", "FETCH_DIR", "WRITE_DIR",
                                                         "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="offline: write profiles/<KERNEL>_<WORKLOAD>_pmc.json from rocprofv3 counter CSVs")
    ap.add_argument("--summarize-counters", nargs="+", metavar="ARG",
                    help="offline: KERNEL WORKLOAD DIR [DIR ...]: average every counter of the given "
                         "rocprofv3 --pmc runs per dispatch of KERNEL into "
                         "profiles/<KERNEL>_<WORKLOAD>_sq_counters.txt")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("TRACE_DIR", "KERNEL", "WORKLOAD"),
                    help="offline: write profiles/<KERNEL>_<WORKLOAD>_kernel_trace.txt from a "
                         "--kernel-trace --stats run")
    ap.add_argument("--pmc-bench-args", default="", help="bench.py arguments of the profiled run (recorded)")
    a = ap.parse_args()
    if a.summarize_pmc:
        summarize_pmc(*a.summarize_pmc, a.pmc_bench_args)
        return
    if a.summarize_trace:
        summarize_trace(*a.summarize_trace, a.pmc_bench_args)
        return
    if a.summarize_counters:
        if len(a.summarize_counters) < 3:
            raise SystemExit("--summarize-counters KERNEL WORKLOAD DIR [DIR ...]")
        k, w, *dirs = a.summarize_counters
        summarize_counters(k, w, dirs, a.pmc_bench_args)
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(a sequence or batch split over GPUs would add carry and grid exchanges; none is built).", file=sys.stderr)
        sys.exit(2)

    import torch
    if a.calibrate_copy:
        n = (1 << 30) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        ms = time_loop(lambda: dst.copy_(src), 5, torch)
        print(json.dumps({"calibration": "copy", "bytes_read": n * 4, "bytes_written": n * 4, "ms": ms,
                          "GBps_read_plus_write": 2 * n * 4 / (ms * 1e-3) / 1e9}), flush=True)
        return
    import recurrence_augmented_dilated_amd as R
    from recurrence_augmented_dilated_amd import inputs
    R.lib()

    if a.config:
        c = CONFIGS[a.config]
        if c["kind"] not in ("prefill", "decode"):
            print(json.dumps(aux_result(a.config, c, a, torch, R, inputs)), flush=True)
            return
        fn = prefill_result if c["kind"] == "prefill" else decode_result
        result = fn(a.config, c, a, torch, R, inputs, not a.no_cpu_baseline)
        result["copy_GBps_measured"] = measure_copy(torch)
        print(json.dumps(result), flush=True)
        return

    # Default line: the longest prefill (T = 262144, the pages' prefill
    # length) gives `value`; the hybrid-head decode (batch 128, context
    # 131072) is reported under "decode"; the other three workloads under
    # "other_configs".  Every workload carries its own roofline and CPU
    # baseline.
    cpu = not a.no_cpu_baseline
    result = prefill_result(3, CONFIGS[3], a, torch, R, inputs, cpu)
    result["copy_GBps_measured"] = measure_copy(torch)
    if not a.no_decode:
        result["decode"] = decode_result(5, CONFIGS[5], a, torch, R, inputs, cpu)
    if not a.no_other_configs:
        others = {}
        for cid in (1, 2, 4):
            c = CONFIGS[cid]
            fn = prefill_result if c["kind"] == "prefill" else decode_result
            others[str(cid)] = fn(cid, c, a, torch, R, inputs, cpu)
        result["other_configs"] = others
    print(json.dumps(result), flush=True)


METRIC = "prefill & decode tokens/s of RAT+ dilated op; % HBM/MFMA roofline"
CPU_PREFILL_ROWS = {1: 1 << 30, 2: 1 << 30, 3: 2048, 10: 2048}   # query rows per head (>= T: all)
CPU_DECODE_SAMPLE = {4: (16, 8), 5: (16, 2)}                      # (sequences, steps)


def _free(torch):
    import gc
    gc.collect()
    torch.cuda.empty_cache()


def prefill_result(cfg_id, c, a, torch, R, inputs, cpu):
    """One prefill workload: tokens/s of the whole call, each kernel's
    roofline, the dominant kernel's as `roofline`, and the CPU baseline."""
    p = bench_prefill(c, a.steps, a.warmup, torch, R, inputs)
    w = prefill_work(c)
    tok_s = c["B"] * c["T"] / (p["ms"] * 1e-3)
    scan_gbs = w["scan_bytes"] / (p["ms_scan"] * 1e-3)
    attn_tfs = w["attn_flops"] / (p["ms_attn"] * 1e-3)
    bf16 = c["dtype"] == "bf16"
    attn_peak = PEAK_BF16 if bf16 else PEAK_F32_VALU
    # a per-head dilation list is named by its (dilation x heads) groups
    dname = (c["D"] if not isinstance(c["D"], list) else
             ",".join(f"{d}x{c['D'].count(d)}" for d in sorted(set(c["D"]))))
    wkey = f"prefill_T{c['T']}_D{str(dname).replace(',', '-')}_W{c['W']}"
    kernels = {
        "scan": {"bound": "hbm", "ms": p["ms_scan"], "achieved": scan_gbs / 1e9, "peak": PEAK_HBM / 1e9,
                 "unit": "GB/s", "frac": scan_gbs / PEAK_HBM, "algorithmic_bytes": w["scan_bytes"],
                 "traffic": measured_traffic("scan", wkey)},
        "attention": {"bound": "mfma" if bf16 else "alu", "ms": p["ms_attn"], "achieved": attn_tfs / 1e12,
                      "peak": attn_peak / 1e12, "unit": "TFLOP/s", "frac": attn_tfs / attn_peak,
                      "algorithmic_flops": w["attn_flops"],
                      "traffic": measured_traffic("attention" if bf16 else "attention_f32", wkey)},
    }
    dom = "scan" if p["ms_scan"] >= p["ms_attn"] else "attention"
    k = kernels[dom]
    res = {"metric": METRIC, "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "data": "synthetic",
           "value": tok_s, "steps": a.steps, "warmup": a.warmup, "ms_per_step": p["ms"],
           "single_call_ms_per_step": p["ms_call"], "single_call_ms_per_step_after": p["ms_call_after"],
           "dtype": c["dtype"],
           "config": {"workload": f"prefill B={c['B']} H={c['H']} Dh={c['Dh']} T={c['T']} D={dname} "
                                  f"W={c['W']} {c['dtype']}", "config_id": cfg_id, "B": c["B"], "T": c["T"],
                      "heads": c["H"], "head_dim": c["Dh"], "dilation": c["D"], "window": c["W"]},
           "roofline": {"kernel": dom, "bound": k["bound"], "achieved": k["achieved"], "peak": k["peak"],
                        "unit": k["unit"], "frac": k["frac"], "traffic": k["traffic"]},
           "kernels": kernels, "ws_error": p["ws_error"], "inputs_sha256": p["inputs_sha256"]}
    del p
    _free(torch)
    if cpu:
        res["cpu_baseline"] = cpu_baseline_prefill(c, CPU_PREFILL_ROWS.get(cfg_id, 2048))
    return res


def decode_result(cfg_id, c, a, torch, R, inputs, cpu):
    """One decode workload: tokens/s over the timed steps, the HBM roofline
    of the step and the CPU baseline."""
    d = bench_decode(c, a.decode_steps, 8, torch, R, inputs)
    _free(torch)
    gbs = d["bytes_per_step"] / (d["ms"] * 1e-3)
    dname = ",".join(f"{x}x{c['D'].count(x)}" for x in sorted(set(c["D"])))
    res = {"metric": METRIC, "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "data": "synthetic",
           "value": c["B"] / (d["ms"] * 1e-3), "steps": d["steps"], "warmup": 8, "ms_per_step": d["ms"],
           "dtype": "bf16",
           "config": {"workload": f"decode B={c['B']} H={c['H']} Dh={c['Dh']} ctx={c['ctx']} W={c['W']} "
                                  f"dilation={dname} bf16, {d['steps']} steps", "config_id": cfg_id},
           "roofline": {"kernel": "decode", "bound": "hbm", "achieved": gbs / 1e9, "peak": PEAK_HBM / 1e9,
                        "unit": "GB/s", "frac": gbs / PEAK_HBM, "algorithmic_bytes_per_step": d["bytes_per_step"],
                        "traffic": measured_traffic("decode", f"decode_config{cfg_id}")},
           "ws_error": d["ws_error"]}
    if cpu:
        n_seq, steps = CPU_DECODE_SAMPLE.get(cfg_id, (8, 4))
        res["cpu_baseline"] = cpu_baseline_decode(c, n_seq, steps)
    return res


if __name__ == "__main__":
    main()
