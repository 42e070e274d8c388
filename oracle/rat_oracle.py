"""Plain fp64 CPU oracle of the RAT+ temporal-mixing operator.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the package's smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code, header, table or
constant with the HIP library; it is deliberately slow and written so that
each step can be checked against the pages by eye.

What it computes (sources are the pages' titles plus the section named):

* Recurrence.  "RAT+: Train Dense, Infer Sparse -- Recurrence Augmented
  Attention for Dilated Inference" (abstract; Fig. 1a: full-sequence
  recurrence, L = T) and "Augmenting Attention with Exponentially Decaying
  Memory Improves Query-Aware KV Sparsity" (section 2.1: keys and values are
  updated by an input-dependent gate into an exponentially decaying memory
  with O(1) cost per token).  The plainest reading, taken here, is the gated
  linear recurrence applied per channel to keys and to values separately:
      g_t = sigmoid(z_t),   h_t = g_t * h_{t-1} + (1 - g_t) * x_t,
  with h_{-1} = h0 (zero unless given; a non-zero initial cell state is
  discussed with RAT+ Fig. 9).  (1 - g_t) is evaluated as sigmoid(-z_t).
* Dilated attention.  RAT+ abstract and Fig. 1c: attention over every D-th
  state (FLOPs and KV cache shrink by D), optionally plus a local window.
  Section 2.2 of the follow-up page: attention runs over the memory states
  (K~, V~), not the raw keys and values.  Query t (0-based) attends to
      S_t = { j <= t : (j + 1) mod D == 0 }  U  { j : max(0, t-W+1) <= j <= t }
  (a set: a position in both parts counts once) with softmax weights
  proportional to exp(scale * <q_t, k~_j>).  An empty S_t gives o_t = 0.
* Decode.  RAT+ Fig. 2: decoding updates the recurrence one step at a time
  and attends over the cached states.  The cache holds the fp state, a ring
  of the last W states (slot p mod W holds position p) and the grid of
  states at (j + 1) mod D == 0 (entry i holds position (i + 1) * D - 1).
  One step at position t: update the state; if W > 0 write it to ring slot
  t mod W; if (t + 1) mod D == 0 append it as grid entry (t + 1) / D - 1;
  then attend over grid entries strictly older than the window
  (i < floor((t - W + 1) / D), none if negative) plus the ring slots of
  positions max(0, t-W+1) .. t.  With W = 0 the grid part is
  i < floor((t + 1) / D), which includes the entry just appended.
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# gate
# ---------------------------------------------------------------------------

def gates(z):
    """Return (g, 1 - g) for gate logits z, both in fp64.

    g = 1 / (1 + exp(-z)) and 1 - g = 1 / (1 + exp(z)).  The complement is
    evaluated from its own formula so that g -> 1 loses no precision and
    z = +-inf gives exactly (1, 0) / (0, 1).
    """
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        g = 1.0 / (1.0 + np.exp(-z))
        c = 1.0 / (1.0 + np.exp(z))
    return g, c


# ---------------------------------------------------------------------------
# recurrence (prefill form)
# ---------------------------------------------------------------------------

def scan(x, z, h0=None):
    """Gated linear recurrence over time for every channel.

    x, z: [B, T, H, Dh] (any real dtype; promoted to fp64).
    h0:   [B, H, Dh] or None (zeros).
    Returns the states h: [B, T, H, Dh] fp64, where
        h[:, t] = g_t * h[:, t-1] + (1 - g_t) * x[:, t]   and h[:, -1] = h0.
    A sequential loop over t, vectorised over the channels.
    """
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    B, T, H, Dh = x.shape
    h = np.zeros((B, H, Dh)) if h0 is None else np.array(h0, dtype=np.float64)
    out = np.empty((B, T, H, Dh))
    for t in range(T):
        g, c = gates(z[:, t])
        h = g * h + c * x[:, t]
        out[:, t] = h
    return out


# ---------------------------------------------------------------------------
# key sets
# ---------------------------------------------------------------------------

def key_set(t: int, D: int, W: int) -> np.ndarray:
    """Sorted positions that query t attends to with dilation D and window W.

    The union of the dilated grid {j <= t : (j + 1) mod D == 0} and the
    window {max(0, t - W + 1) .. t}; both parts are enumerated directly.
    """
    if D < 1 or W < 0 or t < 0:
        raise ValueError("need D >= 1, W >= 0, t >= 0")
    grid = np.arange(D - 1, t + 1, D, dtype=np.int64)
    window = np.arange(max(0, t - W + 1), t + 1, dtype=np.int64)
    return np.union1d(grid, window)


# ---------------------------------------------------------------------------
# attention of one query over an explicit key list
# ---------------------------------------------------------------------------

def attend(q, K, V, scale: float):
    """Softmax attention of one query over rows of K, V (fp64).

    q: [Dh]; K, V: [n, Dh].  Returns sum_j p_j V_j with
    p = softmax(scale * K q).  n == 0 returns zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1] if V.ndim == 2 else q.shape[0])
    s = scale * (K @ q)
    p = np.exp(s - s.max())
    p /= p.sum()
    return p @ V


def default_scale(Dh: int) -> float:
    return 1.0 / math.sqrt(Dh)


def _per_head(dilation, H):
    if np.isscalar(dilation):
        return [int(dilation)] * H
    d = [int(v) for v in dilation]
    if len(d) != H:
        raise ValueError("dilation must be a scalar or one value per head")
    return d


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def prefill(q, k, v, zk, zv, dilation, W: int, scale=None, h0k=None, h0v=None,
            rows=None, states=None):
    """Dilated attention over recurrent states for a whole sequence.

    q, k, v, zk, zv: [B, T, H, Dh].  dilation: int or one int per head.
    rows: optional iterable of query positions to evaluate (others stay 0).
    states: optional precomputed (K~, V~) from scan(), to reuse.
    Returns out [B, T, H, Dh] fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    B, T, H, Dh = q.shape
    if scale is None:
        scale = default_scale(Dh)
    Ds = _per_head(dilation, H)
    if states is None:
        Kt = scan(k, zk, h0k)
        Vt = scan(v, zv, h0v)
    else:
        Kt, Vt = states
    out = np.zeros((B, T, H, Dh))
    ts = range(T) if rows is None else rows
    for t in ts:
        for h in range(H):
            idx = key_set(int(t), Ds[h], W)
            for b in range(B):
                out[b, t, h] = attend(q[b, t, h], Kt[b, idx, h], Vt[b, idx, h], scale)
    return out


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

class DecodeCache:
    """fp64 decode cache for one batch of sequences.

    state_k, state_v: [B, H, Dh]
    ring_k, ring_v:   [B, H, W, Dh]   (slot p mod W holds position p)
    grid_k, grid_v:   list over heads of [B, cap_h, Dh] (entry i holds
                      position (i + 1) * D_h - 1)
    """

    def __init__(self, state_k, state_v, ring_k, ring_v, grid_k, grid_v, dilation, W):
        self.state_k = np.array(state_k, dtype=np.float64)
        self.state_v = np.array(state_v, dtype=np.float64)
        self.ring_k = np.array(ring_k, dtype=np.float64)
        self.ring_v = np.array(ring_v, dtype=np.float64)
        self.grid_k = [np.array(g, dtype=np.float64) for g in grid_k]
        self.grid_v = [np.array(g, dtype=np.float64) for g in grid_v]
        B, H, Dh = self.state_k.shape
        self.dilation = _per_head(dilation, H)
        self.W = int(W)

    @classmethod
    def from_prefill(cls, k, v, zk, zv, dilation, W, cap=None, h0k=None, h0v=None):
        """Cache contents after prefilling positions 0..T-1 (for continuation)."""
        k = np.asarray(k, dtype=np.float64)
        B, T, H, Dh = k.shape
        Ds = _per_head(dilation, H)
        Kt = scan(k, zk, h0k)
        Vt = scan(v, zv, h0v)
        ring_k = np.zeros((B, H, W, Dh))
        ring_v = np.zeros((B, H, W, Dh))
        for p in range(max(0, T - W), T):
            ring_k[:, :, p % W] = Kt[:, p]
            ring_v[:, :, p % W] = Vt[:, p]
        grid_k, grid_v = [], []
        for h in range(H):
            D = Ds[h]
            n = T // D
            c = n if cap is None else cap[h]
            gk = np.zeros((B, c, Dh))
            gv = np.zeros((B, c, Dh))
            for i in range(n):
                gk[:, i] = Kt[:, (i + 1) * D - 1, h]
                gv[:, i] = Vt[:, (i + 1) * D - 1, h]
            grid_k.append(gk)
            grid_v.append(gv)
        return cls(Kt[:, T - 1] if T else np.zeros((B, H, Dh)),
                   Vt[:, T - 1] if T else np.zeros((B, H, Dh)),
                   ring_k, ring_v, grid_k, grid_v, dilation, W)

    def step(self, q, k, v, zk, zv, pos, scale=None, compute=True):
        """One decode step.  q, k, v, zk, zv: [B, H, Dh]; pos: [B] ints.

        Mutates the cache in place.  Returns out [B, H, Dh] (zeros when
        compute is False: the state and cache are still updated).
        """
        q = np.asarray(q, dtype=np.float64)
        B, H, Dh = q.shape
        W = self.W
        if scale is None:
            scale = default_scale(Dh)
        gk, ck = gates(zk)
        gv, cv = gates(zv)
        self.state_k = gk * self.state_k + ck * np.asarray(k, dtype=np.float64)
        self.state_v = gv * self.state_v + cv * np.asarray(v, dtype=np.float64)
        out = np.zeros((B, H, Dh))
        for b in range(B):
            t = int(pos[b])
            for h in range(H):
                D = self.dilation[h]
                if W > 0:
                    self.ring_k[b, h, t % W] = self.state_k[b, h]
                    self.ring_v[b, h, t % W] = self.state_v[b, h]
                if (t + 1) % D == 0:
                    i = (t + 1) // D - 1
                    self.grid_k[h][b, i] = self.state_k[b, h]
                    self.grid_v[h][b, i] = self.state_v[b, h]
                if not compute:
                    continue
                # grid entries strictly older than the window: position <= t - W
                gpos = (np.arange(self.grid_k[h].shape[1]) + 1) * D - 1
                sel = np.nonzero(gpos <= t - W)[0]
                keys = [self.grid_k[h][b, sel]]
                vals = [self.grid_v[h][b, sel]]
                if W > 0:
                    win = np.arange(max(0, t - W + 1), t + 1)
                    keys.append(self.ring_k[b, h, win % W])
                    vals.append(self.ring_v[b, h, win % W])
                out[b, h] = attend(q[b, h], np.concatenate(keys), np.concatenate(vals), scale)
        return out


# ---------------------------------------------------------------------------
# counting helpers (used by the pins and by the benchmark's work model)
# ---------------------------------------------------------------------------

def pairs(T: int, D: int, W: int) -> int:
    """Number of (query, key) pairs of one head, by enumeration of key sets."""
    return int(sum(len(key_set(t, D, W)) for t in range(T)))
