"""Plain fp64 CPU oracle of top-k block attention over RAT+ states.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the package's smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code, header, table or
constant with the HIP library.

What it computes (sources are the pages' titles plus the section named):

* "Augmenting Attention with Exponentially Decaying Memory Improves
  Query-Aware KV Sparsity", section 2.2: query-aware sparse inference first
  scores candidate KV blocks and then attends only over the selected ones;
  applied to RAT+ it works on the memory states (K~, V~) -- here the states
  of rat_oracle.scan -- rather than on raw keys and values.
* Blocks: positions are cut into blocks of `block` positions, block j
  holding positions j*block .. (j+1)*block - 1 (block size D and K selected
  blocks: "RAT+: Train Dense, Infer Sparse", Fig. 3).
* Block representatives of a complete block, over its key states
  (follow-up page, sparse inference settings; RAT+ Tables 17 and 18):
    Quest -- the dimension-wise minimum and maximum; the score of query q is
             sum_d max(q_d * min_d, q_d * max_d), the largest value q.k~ can
             take for a key inside the box [min, max];
    MoBA  -- the mean (mean-pooled keys); the score is q . mean.
* Key set of the query at position t.  The first block and the query's own
  (local) block l = t // block, the latter up to position t, are always kept,
  as each selection method does in its own design.  Among the
  complete blocks strictly between them, 1 .. l-1, the `topk` with the
  highest scores are added.  Readings taken where the pages are silent: the
  K selected blocks come in addition to the first and local blocks; ties go
  to the lower block index; with at most `topk` candidates all are kept;
  the scores use the query as given (the softmax scale does not change a
  ranking).
* Attention over the key set: softmax(scale * q.k~) weights on v~, as in
  rat_oracle.attend; the key set is never empty (it holds position t).
"""
from __future__ import annotations

import numpy as np

from .rat_oracle import attend, default_scale, scan

QUEST = "quest"
MOBA = "moba"


def block_stats(Kt, block: int):
    """Minimum, maximum and mean of the key states over every complete block.

    Kt [B, T, H, Dh] -> three arrays [B, nb, H, Dh], nb = T // block.
    """
    Kt = np.asarray(Kt, dtype=np.float64)
    B, T, H, Dh = Kt.shape
    nb = T // block
    kmin = np.zeros((B, nb, H, Dh))
    kmax = np.zeros((B, nb, H, Dh))
    kmean = np.zeros((B, nb, H, Dh))
    for j in range(nb):
        rows = Kt[:, j * block:(j + 1) * block]        # [B, block, H, Dh]
        kmin[:, j] = rows.min(axis=1)
        kmax[:, j] = rows.max(axis=1)
        kmean[:, j] = rows.sum(axis=1) / block
    return kmin, kmax, kmean


def block_score(q, kmin, kmax, kmean, method: str) -> float:
    """Score of one block for one query vector (all arguments [Dh])."""
    if method == QUEST:
        return float(np.sum(np.maximum(q * kmin, q * kmax)))
    if method == MOBA:
        return float(np.dot(q, kmean))
    raise ValueError(method)


def select_blocks(t: int, block: int, topk: int, scores) -> list:
    """Candidate blocks chosen for the query at position t, ascending.

    scores[j] is the score of complete block j (entries for j >= t // block
    are ignored).  The first and local blocks are not part of the result:
    they are always kept.
    """
    local = t // block
    cand = list(range(1, local))
    if len(cand) <= topk:
        return cand
    ranked = sorted(cand, key=lambda j: (-scores[j], j))   # highest score first, then lower index
    return sorted(ranked[:topk])


def key_positions(t: int, block: int, chosen) -> np.ndarray:
    """Positions of the key set: first block, chosen blocks, local block up to t."""
    local = t // block
    blocks = sorted(set([0, local]) | set(chosen))
    pos = []
    for j in blocks:
        hi = min((j + 1) * block - 1, t)
        pos.extend(range(j * block, hi + 1))
    return np.asarray(pos, dtype=np.int64)


def attend_selected(q, Kt, Vt, t: int, block: int, chosen, scale: float):
    """Attention of one query (q [Dh]) at position t over the key set that
    `chosen` defines; Kt, Vt [T', Dh] are the states of one (b, h)."""
    pos = key_positions(t, block, chosen)
    return attend(q, Kt[pos], Vt[pos], scale)


def topk_prefill(q, k, v, zk, zv, block: int, topk: int, method: str, scale=None, h0k=None, h0v=None,
                 rows=None, states=None, chosen_fn=None):
    """Top-k block attention over the recurrent states for every query row.

    Returns (out [B, T, H, Dh], chosen) where chosen[(b, t, h)] lists the
    selected candidate blocks.  rows restricts the computed query rows;
    states = (Kt, Vt) skips the recurrence; chosen_fn(b, t, h), if given,
    replaces the oracle's selection (to evaluate another valid selection).
    """
    q = np.asarray(q, dtype=np.float64)
    B, T, H, Dh = q.shape
    if scale is None:
        scale = default_scale(Dh)
    if states is None:
        Kt = scan(k, zk, h0k)
        Vt = scan(v, zv, h0v)
    else:
        Kt, Vt = states
    kmin, kmax, kmean = block_stats(Kt, block)
    out = np.zeros((B, T, H, Dh))
    chosen = {}
    for b in range(B):
        for h in range(H):
            for t in (range(T) if rows is None else rows):
                local = t // block
                scores = np.full(max(local, 1), -np.inf)
                for j in range(1, local):
                    scores[j] = block_score(q[b, t, h], kmin[b, j, h], kmax[b, j, h], kmean[b, j, h], method)
                sel = chosen_fn(b, t, h) if chosen_fn else select_blocks(t, block, topk, scores)
                chosen[(b, t, h)] = list(sel)
                out[b, t, h] = attend_selected(q[b, t, h], Kt[b, :, h], Vt[b, :, h], t, block, sel, scale)
    return out, chosen

