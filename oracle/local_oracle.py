"""Plain fp64 CPU oracle of RAT's chunk-local variant of the operator.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the package's smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code, header, table or
constant with the HIP library.

What it computes (sources are the pages' titles plus the section named):

* "RAT: Bridging RNN Efficiency and Attention Accuracy via Chunk-based
  Sequence Modeling" (approach): the sequence is cut into chunks of L
  positions; a gated linear recurrence runs inside each chunk, and softmax
  attention over chunk-level keys and values gives long-range access, with
  the query's own chunk entering hierarchically, through its recurrent
  state.  "RAT+: Train Dense, Infer Sparse" (Fig. 1a) takes the same
  recurrence to the extreme L = T.
* Readings taken where the pages are silent:
    - inside a chunk the recurrence is the RAT+ one (rat_oracle.scan: per
      channel, g = sigmoid(z), separately for keys and values); it restarts
      from a zero state at every chunk start (positions t with t mod L == 0),
      so that L = T is the RAT+ recurrence exactly;
    - the keys and values of a completed chunk are its last states
      (positions (j + 1) L - 1): the RAT+ grid with D = L;
    - the query at position t attends over those of the chunks before its
      own plus its own current state: the RAT+ key set with D = L and a
      window of W = 1.
"""
from __future__ import annotations

import numpy as np

from .rat_oracle import DecodeCache, gates, key_set, prefill


def scan_local(x, z, L: int):
    """Chunk-local recurrence: h_t = g_t h_{t-1} + (1 - g_t) x_t with
    h_{t-1} taken as 0 whenever t mod L == 0.  x, z [B, T, H, Dh]."""
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    B, T, H, Dh = x.shape
    h = np.zeros((B, H, Dh))
    out = np.empty((B, T, H, Dh))
    for t in range(T):
        if t % L == 0:
            h = np.zeros((B, H, Dh))
        g, c = gates(z[:, t])
        h = g * h + c * x[:, t]
        out[:, t] = h
    return out


def key_positions(t: int, L: int) -> np.ndarray:
    """Keys of the query at t: final states of earlier chunks, and t."""
    return key_set(t, L, 1)


def local_prefill(q, k, v, zk, zv, L: int, scale=None, rows=None):
    """RAT chunk-local operator over a whole sequence: out [B, T, H, Dh]."""
    Kt = scan_local(k, zk, L)
    Vt = scan_local(v, zv, L)
    return prefill(q, None, None, None, None, L, 1, scale=scale, rows=rows, states=(Kt, Vt))


def local_cache_from_prefill(k, v, zk, zv, L: int, cap):
    """Decode cache (rat_oracle.DecodeCache with D = L, W = 1) after the
    chunk-local prefill of positions 0 .. T-1."""
    k = np.asarray(k, dtype=np.float64)
    B, T, H, Dh = k.shape
    Kt = scan_local(k, zk, L)
    Vt = scan_local(v, zv, L)
    ring_k = np.zeros((B, H, 1, Dh))
    ring_v = np.zeros((B, H, 1, Dh))
    if T:
        ring_k[:, :, 0] = Kt[:, T - 1]
        ring_v[:, :, 0] = Vt[:, T - 1]
    grid_k, grid_v = [], []
    for h in range(H):
        gk = np.zeros((B, cap[h], Dh))
        gv = np.zeros((B, cap[h], Dh))
        for i in range(T // L):
            gk[:, i] = Kt[:, (i + 1) * L - 1, h]
            gv[:, i] = Vt[:, (i + 1) * L - 1, h]
        grid_k.append(gk)
        grid_v.append(gv)
    state_k = Kt[:, T - 1] if T else np.zeros((B, H, Dh))
    state_v = Vt[:, T - 1] if T else np.zeros((B, H, Dh))
    return DecodeCache(state_k, state_v, ring_k, ring_v, grid_k, grid_v, L, 1)


def local_decode_step(cache: DecodeCache, q, k, v, zk, zv, pos, L: int, scale=None, compute=True):
    """One chunk-local decode step: a sequence whose new position starts a
    chunk restarts from a zero state, then the RAT+ step (D = L, W = 1)."""
    for b, t in enumerate(pos):
        if int(t) % L == 0:
            cache.state_k[b] = 0.0
            cache.state_v[b] = 0.0
    return cache.step(q, k, v, zk, zv, pos, scale=scale, compute=compute)
