"""Seeded synthetic inputs for the RAT+ operator.

This module only draws random numbers; it holds none of the operator's
arithmetic.  Both the HIP path (through the tests and the benchmark) and the
fp64 oracle (through the tests) take their inputs from here.

Recipe: q, k, v ~ N(0, 1), drawn in fp32 and cast to the compute dtype with
round-to-nearest-even; gate logits z ~ N(mu, 1) in fp32 (one set for keys,
one for values); decode caches (fp32 state, bf16 grid and ring) and top-k
state caches ~ N(0, 1).
Draw order is fixed: q, k, v, zk, zv, then caches, then per-step inputs.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import torch


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, g, device, mean=0.0):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if mean:
        x.add_(mean)
    return x


def prefill_inputs(B, T, H, Dh, dtype=torch.bfloat16, mu=2.0, seed=0, device="cpu"):
    """q, k, v in `dtype`; zk, zv fp32 with mean `mu`.  Shapes [B, T, H, Dh]."""
    g = _gen(seed, device)
    shape = (B, T, H, Dh)
    q = _normal(shape, g, device).to(dtype)
    k = _normal(shape, g, device).to(dtype)
    v = _normal(shape, g, device).to(dtype)
    zk = _normal(shape, g, device, mu)
    zv = _normal(shape, g, device, mu)
    return dict(q=q, k=k, v=v, zk=zk, zv=zv)


@dataclass
class GridLayout:
    """Ragged per-head grid cache layout: head h occupies elements
    [B * off[h] * Dh, B * (off[h] + cap[h]) * Dh) laid out [B, cap[h], Dh]."""
    off: list
    cap: list

    @property
    def total_rows(self) -> int:
        return int(self.off[-1] + self.cap[-1]) if self.cap else 0


def grid_layout(dilation, context: int, steps: int) -> GridLayout:
    """Capacity per head = grid entries after context + steps tokens."""
    cap = [(context + steps) // int(d) for d in dilation]
    off, acc = [], 0
    for c in cap:
        off.append(acc)
        acc += c
    return GridLayout(off=off, cap=cap)


def decode_cache(B, H, Dh, dilation, W, context, steps, dtype=torch.bfloat16, seed=0,
                 device="cpu"):
    """Random-filled decode cache for sequences that hold `context` tokens.

    Returns dict(state_k, state_v [B,H,Dh] fp32; ring_k, ring_v [B,H,W,Dh];
    grid_k, grid_v flat ragged buffers; layout).  Every buffer is N(0, 1)
    (grid rows beyond the filled ones too; they are overwritten by appends).
    """
    g = _gen(seed, device)
    lay = grid_layout(dilation, context, steps)
    state_k = _normal((B, H, Dh), g, device)
    state_v = _normal((B, H, Dh), g, device)
    ring_k = _normal((B, H, max(W, 0), Dh), g, device).to(dtype)
    ring_v = _normal((B, H, max(W, 0), Dh), g, device).to(dtype)
    n = B * lay.total_rows * Dh
    grid_k = torch.empty(n, dtype=dtype, device=device)
    grid_v = torch.empty(n, dtype=dtype, device=device)
    chunk = 1 << 28
    for buf in (grid_k, grid_v):
        for s in range(0, n, chunk):
            e = min(n, s + chunk)
            buf[s:e] = _normal((e - s,), g, device).to(dtype)
    return dict(state_k=state_k, state_v=state_v, ring_k=ring_k, ring_v=ring_v,
                grid_k=grid_k, grid_v=grid_v, layout=lay)


def fill_topk_cache(cache, seed=7):
    """Fill the state caches of a top-k cache dict (cache_k, cache_v [H, B,
    max_pos, Dh]; state_k, state_v [B, H, Dh] fp32) with N(0, 1) values:
    cache_k head by head, then cache_v, then state_k, state_v.  Summaries are
    left alone (the caller computes them)."""
    device = cache["cache_k"].device
    g = _gen(seed, device)
    for name in ("cache_k", "cache_v"):
        buf = cache[name]
        for h in range(buf.shape[0]):
            buf[h].copy_(torch.randn(buf[h].shape, generator=g, device=device).to(buf.dtype))
    cache["state_k"].normal_(generator=g)
    cache["state_v"].normal_(generator=g)


def decode_step_inputs(B, H, Dh, steps, dtype=torch.bfloat16, mu=2.0, seed=0, device="cpu"):
    """Per-step q, k, v ([steps, B, H, Dh] in dtype) and zk, zv (fp32, mean mu)."""
    g = _gen(seed, device)
    shape = (steps, B, H, Dh)
    q = _normal(shape, g, device).to(dtype)
    k = _normal(shape, g, device).to(dtype)
    v = _normal(shape, g, device).to(dtype)
    zk = _normal(shape, g, device, mu)
    zv = _normal(shape, g, device, mu)
    return dict(q=q, k=k, v=v, zk=zk, zv=zv)


def sha256_of(*tensors) -> str:
    """Hash of host copies of tensors (bytes in memory order)."""
    h = hashlib.sha256()
    for t in tensors:
        t = t.detach().contiguous().cpu()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        h.update(t.numpy().tobytes())
    return h.hexdigest()
