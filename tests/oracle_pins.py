"""Checks that pin the fp64 oracle to facts other than itself.

Every function takes the oracle module `O` as its argument so that the same
checks can run against deliberately broken copies of the oracle (see
test_oracle_mutants.py): each plausible mistake must make one of them fail.

The facts come from closed forms, textbook special cases, a library routine
(torch's scaled_dot_product_attention on the CPU in fp64), brute-force
enumeration, and hand-worked fixtures in tests/golden/.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err} > {tol}"


def _col(vals):
    """[T] list -> [1, T, 1, 1] array."""
    return np.asarray(vals, dtype=np.float64).reshape(1, -1, 1, 1)


# ---------------------------------------------------------------------------
# gate and recurrence
# ---------------------------------------------------------------------------

def pin_gates(O):
    g, c = O.gates(np.array([0.0, math.log(3.0), -math.log(3.0), np.inf, -np.inf]))
    _close(g, [0.5, 0.75, 0.25, 1.0, 0.0], 1e-15, "sigmoid values")
    _close(c, [0.5, 0.25, 0.75, 0.0, 1.0], 1e-15, "complement values")
    z = _rng(1).normal(0, 4, size=1000)
    g, c = O.gates(z)
    _close(g + c, np.ones_like(z), 1e-15, "g + (1-g) == 1")


def pin_scan_golden(O):
    f = _golden("scan_half_gate.json")
    T = len(f["x"])
    h = O.scan(_col(f["x"]), np.full((1, T, 1, 1), f["z"]), np.full((1, 1, 1), f["h0"]))
    _close(h.reshape(-1), f["expected"], 1e-15, "scan golden (g=1/2)")
    T = len(f["x_b"])
    h = O.scan(_col(f["x_b"]), np.full((1, T, 1, 1), f["z_b"]), np.full((1, 1, 1), f["h0_b"]))
    _close(h.reshape(-1), f["expected_b"], 1e-13, "scan golden (g=3/4, h0=8)")


def pin_scan_closed_form(O):
    """h_t = sum_j (prod_{s=j+1..t} g_s)(1-g_j) x_j + (prod_{s<=t} g_s) h0, T <= 48."""
    r = _rng(2)
    B, T, H, Dh = 2, 48, 2, 3
    x = r.normal(size=(B, T, H, Dh))
    z = r.normal(1.5, 1.5, size=(B, T, H, Dh))
    h0 = r.normal(size=(B, H, Dh))
    got = O.scan(x, z, h0)
    g = 1.0 / (1.0 + np.exp(-z))
    for t in range(T):
        ref = np.prod(g[:, : t + 1], axis=1) * h0
        for j in range(t + 1):
            ref = ref + np.prod(g[:, j + 1: t + 1], axis=1) * (1.0 - g[:, j]) * x[:, j]
        _close(got[:, t], ref, 1e-12, f"closed form t={t}")


def pin_scan_geometric(O):
    """Constant gate a and input x: h_t = x (1 - a^{t+1}) + a^{t+1} h0."""
    T, a, x, h0 = 200, 0.9, 0.7, -1.3
    z = math.log(a / (1 - a))
    h = O.scan(np.full((1, T, 1, 1), x), np.full((1, T, 1, 1), z), np.full((1, 1, 1), h0))
    t = np.arange(T)
    _close(h.reshape(-1), x * (1 - a ** (t + 1)) + a ** (t + 1) * h0, 1e-12, "geometric")


def pin_scan_extreme_gates(O):
    r = _rng(3)
    x = r.normal(size=(1, 16, 2, 4))
    h0 = r.normal(size=(1, 2, 4))
    _close(O.scan(x, np.full(x.shape, -np.inf), h0), x, 0.0, "g = 0 copies the input")
    h = O.scan(x, np.full(x.shape, np.inf), h0)
    _close(h, np.broadcast_to(h0[:, None], x.shape), 0.0, "g = 1 keeps h0")


# ---------------------------------------------------------------------------
# key sets
# ---------------------------------------------------------------------------

def pin_key_set_bruteforce(O):
    """Every position j of [0, T) against the predicate, for all D, W."""
    T = 24
    for D in range(1, T + 1):
        for W in range(0, T + 2):
            for t in range(T):
                want = [j for j in range(T)
                        if j <= t and ((j + 1) % D == 0 or j >= t - W + 1)]
                got = list(O.key_set(t, D, W))
                assert got == want, (t, D, W, got, want)
                # count: grid part strictly older than the window plus window
                n = max(0, (t - W + 1)) // D + min(W, t + 1)
                assert len(got) == n, (t, D, W, len(got), n)


def pin_kv_reduction(O):
    """Abstract: KV cache and attention work shrink by the dilation size D."""
    f = _golden("kv_reduction.json")
    D, T = f["D"], f["T"]
    grid = len(O.key_set(T - 1, D, 0))
    assert T // grid == f["reduction"], (T, grid)
    Ts = 4096
    dense = Ts * (Ts + 1) // 2
    ratio = dense / O.pairs(Ts, D, 0)
    assert abs(ratio - f["reduction"]) / f["reduction"] < 0.02, ratio


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def pin_attention_golden(O):
    for case in _golden("dilated_tiny.json")["cases"]:
        T = case["T"]
        q, k, v = _col(case["q"]), _col(case["k"]), _col(case["v"])
        zinf = np.full((1, T, 1, 1), -np.inf)
        out = O.prefill(q, k, v, zinf, zinf, case["D"], case["W"], scale=case.get("scale", 1.0))
        _close(out.reshape(-1), case["expected"], 1e-12, f"golden {case['derivation']}")


def _sdpa_causal(q, k, v, scale):
    """torch's fused attention routine, fp64 on the CPU: [B,T,H,Dh] layout."""
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def pin_d1_is_causal_attention(O):
    """D = 1 with gates closed (g = 0) is ordinary causal softmax attention."""
    r = _rng(4)
    B, T, H, Dh = 2, 40, 3, 8
    q, k, v = (r.normal(size=(B, T, H, Dh)) for _ in range(3))
    zinf = np.full((B, T, H, Dh), -np.inf)
    out = O.prefill(q, k, v, zinf, zinf, 1, 0, scale=0.5)
    _close(out, _sdpa_causal(q, k, v, 0.5), 1e-12, "D=1 vs SDPA")


def _masked_softmax_attention(q, K, V, mask, scale):
    """Dense [T, T] score matrix with a boolean mask, fp64; empty rows -> 0."""
    s = scale * (q @ K.T)
    s = np.where(mask, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.where(mask, np.exp(s - m), 0.0)
    den = p.sum(axis=1, keepdims=True)
    den = np.where(den > 0, den, 1.0)
    return (p / den) @ V


def pin_dilated_raw_matches_mask(O):
    """g = 0 and D > 1: plain absolute-grid dilated attention on raw k, v."""
    r = _rng(5)
    T, Dh = 37, 6
    q, k, v = (r.normal(size=(1, T, 1, Dh)) for _ in range(3))
    zinf = np.full((1, T, 1, Dh), -np.inf)
    t = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    for D, W in [(2, 0), (3, 0), (5, 2), (4, 4), (7, 1), (37, 0), (6, 9)]:
        mask = (j <= t) & (((j + 1) % D == 0) | (j >= t - W + 1))
        ref = _masked_softmax_attention(q[0, :, 0], k[0, :, 0], v[0, :, 0], mask, 0.7)
        out = O.prefill(q, k, v, zinf, zinf, D, W, scale=0.7)
        _close(out[0, :, 0], ref, 1e-12, f"dilated raw D={D} W={W}")


def pin_dilated_states_matches_mask(O):
    """Finite gates: attention over the recurrent states under the same mask."""
    r = _rng(6)
    T, Dh = 33, 4
    q, k, v = (r.normal(size=(1, T, 1, Dh)) for _ in range(3))
    zk = r.normal(2, 1, size=(1, T, 1, Dh))
    zv = r.normal(2, 1, size=(1, T, 1, Dh))
    gk = 1 / (1 + np.exp(-zk[0, :, 0]))
    gv = 1 / (1 + np.exp(-zv[0, :, 0]))
    Ks = np.zeros((T, Dh))
    Vs = np.zeros((T, Dh))
    hk = np.zeros(Dh)
    hv = np.zeros(Dh)
    for s in range(T):  # independent recurrence written with g and 1 - g
        hk = gk[s] * hk + (1 - gk[s]) * k[0, s, 0]
        hv = gv[s] * hv + (1 - gv[s]) * v[0, s, 0]
        Ks[s], Vs[s] = hk, hv
    t = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    for D, W in [(4, 0), (3, 5), (1, 0), (8, 3)]:
        mask = (j <= t) & (((j + 1) % D == 0) | (j >= t - W + 1))
        ref = _masked_softmax_attention(q[0, :, 0], Ks, Vs, mask, 0.5)
        out = O.prefill(q, k, v, zk, zv, D, W, scale=0.5)
        _close(out[0, :, 0], ref, 1e-10, f"states D={D} W={W}")


def pin_d_equals_t(O):
    """D = T, W = 0: only the last state is a key; every earlier row is empty."""
    r = _rng(7)
    B, T, H, Dh = 1, 20, 2, 5
    q, k, v = (r.normal(size=(B, T, H, Dh)) for _ in range(3))
    zk, zv = (r.normal(2, 1, size=(B, T, H, Dh)) for _ in range(2))
    out = O.prefill(q, k, v, zk, zv, T, 0)
    _close(out[:, : T - 1], np.zeros((B, T - 1, H, Dh)), 0.0, "rows before T-1 empty")
    Vt = O.scan(v, zv)
    _close(out[:, T - 1], Vt[:, T - 1], 1e-14, "single key -> its value")


def pin_full_window_ignores_d(O):
    """W >= T: the window covers every j <= t, so D has no effect."""
    r = _rng(8)
    B, T, H, Dh = 1, 18, 1, 4
    q, k, v = (r.normal(size=(B, T, H, Dh)) for _ in range(3))
    zk, zv = (r.normal(2, 1, size=(B, T, H, Dh)) for _ in range(2))
    ref = O.prefill(q, k, v, zk, zv, 1, T)
    for D in (2, 5, 18):
        _close(O.prefill(q, k, v, zk, zv, D, T), ref, 1e-14, f"W=T D={D}")


def pin_per_head_dilation(O):
    """Per-head dilation equals the homogeneous runs head by head."""
    r = _rng(9)
    B, T, H, Dh = 2, 30, 3, 4
    q, k, v = (r.normal(size=(B, T, H, Dh)) for _ in range(3))
    zk, zv = (r.normal(2, 1, size=(B, T, H, Dh)) for _ in range(2))
    Ds, W = [1, 4, 16], 3
    out = O.prefill(q, k, v, zk, zv, Ds, W)
    for h, D in enumerate(Ds):
        ref = O.prefill(q, k, v, zk, zv, D, W)
        _close(out[:, :, h], ref[:, :, h], 1e-14, f"head {h}")


def pin_convexity(O):
    """Outputs are convex combinations of the selected values."""
    r = _rng(10)
    B, T, H, Dh = 1, 30, 1, 6
    q, k, v = (r.normal(0, 3, size=(B, T, H, Dh)) for _ in range(3))
    zk, zv = (r.normal(1, 1, size=(B, T, H, Dh)) for _ in range(2))
    D, W = 4, 3
    out = O.prefill(q, k, v, zk, zv, D, W)
    Vt = O.scan(v, zv)
    for t in range(T):
        idx = O.key_set(t, D, W)
        lo, hi = Vt[0, idx, 0].min(0), Vt[0, idx, 0].max(0)
        assert np.all(out[0, t, 0] >= lo - 1e-12) and np.all(out[0, t, 0] <= hi + 1e-12), t


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def pin_decode_continuation(O):
    """Prefill of T + s tokens equals prefill of T followed by s decode steps."""
    r = _rng(11)
    B, H, Dh = 2, 3, 4
    T0, s = 21, 13
    Ds = [1, 3, 8]
    for W in (0, 4):
        q, k, v = (r.normal(size=(B, T0 + s, H, Dh)) for _ in range(3))
        zk, zv = (r.normal(2, 1, size=(B, T0 + s, H, Dh)) for _ in range(2))
        ref = O.prefill(q, k, v, zk, zv, Ds, W)
        cap = [(T0 + s) // D for D in Ds]
        cache = O.DecodeCache.from_prefill(k[:, :T0], v[:, :T0], zk[:, :T0], zv[:, :T0],
                                           Ds, W, cap=cap)
        for i in range(s):
            t = T0 + i
            out = cache.step(q[:, t], k[:, t], v[:, t], zk[:, t], zv[:, t], [t] * B)
            _close(out, ref[:, t], 1e-12, f"continuation W={W} t={t}")
            assert cache.state_k.shape == (B, H, Dh)  # O(1) state per token


def pin_decode_from_empty(O):
    """Decoding from position 0 with an empty cache reproduces prefill."""
    r = _rng(12)
    B, T, H, Dh = 1, 17, 2, 3
    q, k, v = (r.normal(size=(B, T, H, Dh)) for _ in range(3))
    zk, zv = (r.normal(2, 1, size=(B, T, H, Dh)) for _ in range(2))
    for D, W in [(2, 0), (4, 2), (1, 1)]:
        ref = O.prefill(q, k, v, zk, zv, D, W)
        cache = O.DecodeCache(np.zeros((B, H, Dh)), np.zeros((B, H, Dh)),
                              np.zeros((B, H, W, Dh)), np.zeros((B, H, W, Dh)),
                              [np.zeros((B, T // D, Dh))] * H, [np.zeros((B, T // D, Dh))] * H,
                              D, W)
        for t in range(T):
            out = cache.step(q[:, t], k[:, t], v[:, t], zk[:, t], zv[:, t], [t])
            _close(out, ref[:, t], 1e-12, f"from empty D={D} W={W} t={t}")


def pin_decode_slots(O):
    """Slot semantics on a random (inconsistent) cache, checked by hand."""
    r = _rng(13)
    B, H, Dh, W, D = 1, 1, 3, 4, 2
    t = 9
    cap = 6
    gk, gv = r.normal(size=(B, cap, Dh)), r.normal(size=(B, cap, Dh))
    rk, rv = r.normal(size=(B, H, W, Dh)), r.normal(size=(B, H, W, Dh))
    sk, sv = r.normal(size=(B, H, Dh)), r.normal(size=(B, H, Dh))
    q, k, v = (r.normal(size=(B, H, Dh)) for _ in range(3))
    zk, zv = (r.normal(size=(B, H, Dh)) for _ in range(2))
    cache = O.DecodeCache(sk, sv, rk, rv, [gk], [gv], D, W)
    out = cache.step(q, k, v, zk, zv, [t], scale=1.0)
    ak = 1 / (1 + np.exp(-zk))
    av = 1 / (1 + np.exp(-zv))
    nk = ak * sk + (1 - ak) * k
    nv = av * sv + (1 - av) * v
    # t = 9, D = 2: (t+1) % D == 0 -> grid entry 4 written; window = 6..9
    # grid keys strictly older than the window: positions 1, 3, 5 -> entries 0, 1, 2
    _close(cache.grid_k[0][0, 4], nk[0, 0], 1e-15, "grid append")
    _close(cache.ring_k[0, 0, t % W], nk[0, 0], 1e-15, "ring write")
    Ks = np.concatenate([gk[0, :3], rk[0, 0, [6 % W, 7 % W, 8 % W]], nk[0]])
    Vs = np.concatenate([gv[0, :3], rv[0, 0, [6 % W, 7 % W, 8 % W]], nv[0]])
    s = Ks @ q[0, 0]
    p = np.exp(s - s.max())
    p /= p.sum()
    _close(out[0, 0], p @ Vs, 1e-12, "decode slot semantics")


ALL_PINS = [
    pin_gates, pin_scan_golden, pin_scan_closed_form, pin_scan_geometric,
    pin_scan_extreme_gates, pin_key_set_bruteforce, pin_kv_reduction,
    pin_attention_golden, pin_d1_is_causal_attention, pin_dilated_raw_matches_mask,
    pin_dilated_states_matches_mask, pin_d_equals_t, pin_full_window_ignores_d,
    pin_per_head_dilation, pin_convexity, pin_decode_continuation,
    pin_decode_from_empty, pin_decode_slots,
]


def run_all(O):
    """Run every pin; return the names of those that fail."""
    failed = []
    for pin in ALL_PINS:
        try:
            pin(O)
        except Exception:  # noqa: BLE001 - a mutant may fail in any way
            failed.append(pin.__name__)
    return failed



# ---------------------------------------------------------------------------
# top-k block attention over the memory states (oracle.topk_oracle)
# ---------------------------------------------------------------------------

def tpin_golden(T):
    f = _golden("topk_hand.json")
    K = np.asarray(f["keys"], dtype=np.float64)
    blk, t, q = f["block"], f["t"], np.asarray(f["q"])
    kmin, kmax, kmean = T.block_stats(K.reshape(1, -1, 1, 2), blk)
    for meth, name in ((T.QUEST, "quest"), (T.MOBA, "moba")):
        for j, want in f[f"{name}_scores"].items():
            j = int(j)
            got = T.block_score(q, kmin[0, j, 0], kmax[0, j, 0], kmean[0, j, 0], meth)
            _close(got, want, 1e-15, f"{name} score of block {j}")
        scores = [T.block_score(q, kmin[0, j, 0], kmax[0, j, 0], kmean[0, j, 0], meth) for j in range(t // blk)]
        chosen = T.select_blocks(t, blk, f["topk"], scores)
        assert chosen == f[f"{name}_chosen"], (name, chosen)
        assert list(T.key_positions(t, blk, chosen)) == f[f"{name}_positions"], name


def tpin_quest_is_box_maximum(T):
    """Quest's score is the maximum of q.k over the corners of the block's
    bounding box (brute force over the 2^Dh corners), hence an upper bound of
    q.k for every key in the block."""
    rng = _rng(21)
    Dh, blk = 4, 5
    K = rng.normal(size=(1, 3 * blk, 1, Dh))
    kmin, kmax, kmean = T.block_stats(K, blk)
    for trial in range(20):
        q = rng.normal(size=Dh)
        for j in range(3):
            s = T.block_score(q, kmin[0, j, 0], kmax[0, j, 0], kmean[0, j, 0], T.QUEST)
            corners = [np.where([(c >> d) & 1 for d in range(Dh)], kmax[0, j, 0], kmin[0, j, 0]) for c in range(2 ** Dh)]
            _close(s, max(float(q @ c) for c in corners), 1e-12, "quest == max over box corners")
            rows = K[0, j * blk:(j + 1) * blk, 0]
            assert s >= np.max(rows @ q) - 1e-12, "quest is an upper bound"


def tpin_moba_is_mean_dot(T):
    """MoBA's score is the average of the block's per-key dot products."""
    rng = _rng(22)
    Dh, blk = 6, 4
    K = rng.normal(size=(2, 3 * blk + 1, 1, Dh))
    kmin, kmax, kmean = T.block_stats(K, blk)
    assert kmean.shape[1] == 3                 # the incomplete last block has no representative
    for b in range(2):
        for j in range(3):
            q = rng.normal(size=Dh)
            dots = [float(q @ K[b, p, 0]) for p in range(j * blk, (j + 1) * blk)]
            s = T.block_score(q, kmin[b, j, 0], kmax[b, j, 0], kmean[b, j, 0], T.MOBA)
            _close(s, sum(dots) / blk, 1e-12, "moba == mean of per-key dots")
            _close(kmin[b, j, 0], [min(K[b, p, 0, d] for p in range(j * blk, (j + 1) * blk)) for d in range(Dh)],
                   0.0, "block minimum")
            _close(kmax[b, j, 0], [max(K[b, p, 0, d] for p in range(j * blk, (j + 1) * blk)) for d in range(Dh)],
                   0.0, "block maximum")


def tpin_selection_bruteforce(T):
    """The chosen blocks are the subset of candidates with the largest score
    sum (enumerating every subset of size topk); among equal sums, the one
    with the lower block indices."""
    import itertools
    rng = _rng(23)
    blk = 4
    for trial in range(60):
        local = int(rng.integers(1, 9))
        t = local * blk + int(rng.integers(0, blk))
        topk = int(rng.integers(0, 6))
        scores = np.round(rng.normal(size=local), 1) if trial % 3 else rng.normal(size=local)   # ties sometimes
        cand = list(range(1, local))
        if len(cand) <= topk:
            want = cand
        else:
            best = None
            for sub in itertools.combinations(cand, topk):
                key = (-sum(scores[j] for j in sub), sorted(sub))
                if best is None or key < best:
                    best = key
            want = list(best[1])
            # the tie rule: equal-sum subsets resolved towards lower indices only matter when
            # scores tie; the top-k set then prefers lower indices element by element
            ranked = sorted(cand, key=lambda j: (-scores[j], j))[:topk]
            assert sorted(ranked) == want or sum(scores[j] for j in ranked) == -best[0]
        got = T.select_blocks(t, blk, topk, scores)
        assert got == sorted(got)
        if len(cand) > topk:
            _close(sum(scores[j] for j in got), sum(scores[j] for j in want), 1e-12, "top-k score sum")
            # ties: every chosen block scores >= every unchosen candidate, and a
            # tie between a chosen and an unchosen block goes to the lower index
            for u in set(cand) - set(got):
                for c in got:
                    assert scores[c] > scores[u] or (scores[c] == scores[u] and c < u), (got, u, scores)
        else:
            assert got == want


def tpin_ties_prefer_lower_blocks(T):
    """Equal scores: the lowest-indexed candidates are chosen."""
    for local in range(2, 12):
        for topk in range(0, local):
            t = local * 8 + 3
            got = T.select_blocks(t, 8, topk, np.zeros(local))
            assert got == list(range(1, min(local, topk + 1))), (local, topk, got)


def tpin_prefill_selects_by_key_states(T):
    """The selections made inside topk_prefill are the top-k of scores
    recomputed here from the key states (per-key dot products for MoBA,
    per-key corner maxima for Quest)."""
    import oracle.rat_oracle as O
    rng = _rng(26)
    B, L, H, Dh, blk, topk = 1, 48, 2, 4, 4, 3
    q, k, v = (rng.normal(size=(B, L, H, Dh)) for _ in range(3))
    zk, zv = rng.normal(0.5, 1, size=(2, B, L, H, Dh))
    Kt = O.scan(k, zk)
    for meth in (T.QUEST, T.MOBA):
        _, chosen = T.topk_prefill(q, k, v, zk, zv, blk, topk, meth)
        for (b, t, h), sel in chosen.items():
            local = t // blk
            scores = np.full(max(local, 1), -np.inf)
            for j in range(1, local):
                rows = Kt[b, j * blk:(j + 1) * blk, h]
                if meth == T.MOBA:
                    scores[j] = np.mean(rows @ q[b, t, h])
                else:
                    scores[j] = np.sum(np.max(rows * q[b, t, h], axis=0))
            cand = list(range(1, local))
            want = cand if len(cand) <= topk else sorted(sorted(cand, key=lambda j: (-scores[j], j))[:topk])
            assert sel == want, (meth, b, t, h, sel, want)


def tpin_key_positions_bruteforce(T):
    blk = 3
    for t in range(0, 40):
        local = t // blk
        for chosen in ([], [1], [2, 5], list(range(1, local))):
            chosen = [j for j in chosen if 1 <= j < local]
            want = [p for p in range(t + 1) if (p // blk) in ({0, local} | set(chosen))]
            assert list(T.key_positions(t, blk, chosen)) == want, (t, chosen)


def tpin_all_blocks_is_dense(T):
    """With topk at least the number of candidate blocks every position
    0..t is a key: causal attention over the states (rat_oracle with D = 1)."""
    import oracle.rat_oracle as O
    rng = _rng(24)
    B, L, H, Dh = 1, 40, 2, 8
    q, k, v = (rng.normal(size=(B, L, H, Dh)) for _ in range(3))
    zk, zv = rng.normal(1, 1, size=(2, B, L, H, Dh))
    for meth in (T.QUEST, T.MOBA):
        out, _ = T.topk_prefill(q, k, v, zk, zv, 4, 100, meth)
        _close(out, O.prefill(q, k, v, zk, zv, 1, 0), 1e-12, f"{meth} with every block == dense")


def tpin_first_and_local_only(T):
    """topk = 0 keeps the first and the local block: attention over those
    positions by a dense masked softmax (a [T, T] score matrix)."""
    import oracle.rat_oracle as O
    rng = _rng(25)
    B, L, H, Dh, blk = 1, 37, 1, 4, 5
    q, k, v = (rng.normal(size=(B, L, H, Dh)) for _ in range(3))
    zk, zv = rng.normal(1, 1, size=(2, B, L, H, Dh))
    Kt, Vt = O.scan(k, zk), O.scan(v, zv)
    mask = np.zeros((L, L), dtype=bool)
    for t in range(L):
        for p in range(t + 1):
            mask[t, p] = p < blk or p // blk == t // blk
    want = _masked_softmax_attention(q[0, :, 0], Kt[0, :, 0], Vt[0, :, 0], mask, 1.0 / math.sqrt(Dh))
    out, _ = T.topk_prefill(q, k, v, zk, zv, blk, 0, T.QUEST)
    out = out[0, :, 0]
    _close(out, want, 1e-12, "first + local blocks")


TOPK_PINS = [tpin_golden, tpin_quest_is_box_maximum, tpin_moba_is_mean_dot, tpin_selection_bruteforce,
             tpin_ties_prefer_lower_blocks, tpin_prefill_selects_by_key_states, tpin_key_positions_bruteforce,
             tpin_all_blocks_is_dense, tpin_first_and_local_only]


def run_topk(T):
    failed = []
    for p in TOPK_PINS:
        try:
            p(T)
        except Exception as e:  # noqa: BLE001
            failed.append(f"{p.__name__}: {type(e).__name__}: {e}")
    return failed


# ---------------------------------------------------------------------------
# RAT chunk-local variant (oracle.local_oracle)
# ---------------------------------------------------------------------------

def lpin_chunks_are_independent(LO):
    """The chunk-local states are the RAT+ recurrence run on every chunk
    separately from a zero state."""
    import oracle.rat_oracle as O
    rng = _rng(41)
    x = rng.normal(size=(2, 50, 2, 3))
    z = rng.normal(1, 1.5, size=x.shape)
    for L in (1, 4, 7, 50, 64):
        want = np.concatenate([O.scan(x[:, s:s + L], z[:, s:s + L]) for s in range(0, 50, L)], axis=1)
        _close(LO.scan_local(x, z, L), want, 1e-13, f"chunk-local states L={L}")


def lpin_full_chunk_is_ratplus(LO):
    """L = T is the RAT+ recurrence, and the operator equals RAT+ with D = T, W = 1."""
    import oracle.rat_oracle as O
    rng = _rng(42)
    q, k, v = (rng.normal(size=(1, 30, 2, 4)) for _ in range(3))
    zk, zv = rng.normal(1, 1, size=(2, 1, 30, 2, 4))
    _close(LO.scan_local(k, zk, 30), O.scan(k, zk), 1e-14, "L = T states")
    _close(LO.local_prefill(q, k, v, zk, zv, 30), O.prefill(q, k, v, zk, zv, 30, 1), 1e-13, "L = T operator")


def lpin_unit_chunks_are_causal_attention(LO):
    """L = 1 with open gates (z = -inf, so g = 0) leaves the raw keys and
    values as states, every earlier chunk-final state is a key: causal
    softmax attention (torch sdpa on the CPU, fp64)."""
    rng = _rng(43)
    B, T, H, Dh = 1, 24, 2, 8
    q, k, v = (rng.normal(size=(B, T, H, Dh)) for _ in range(3))
    z = np.full((B, T, H, Dh), -np.inf)
    _close(LO.local_prefill(q, k, v, z, z, 1), _sdpa_causal(q, k, v, 1.0 / math.sqrt(Dh)), 1e-12,
           "L = 1, g = 0 == causal attention")


def lpin_key_positions(LO):
    for L in (1, 3, 8):
        for t in range(40):
            want = [p for p in range(t) if (p + 1) % L == 0 and p < (t // L) * L] + [t]
            assert list(LO.key_positions(t, L)) == want, (L, t)


def lpin_decode_continuation(LO):
    """Prefill of T + s positions equals prefill of T, then s decode steps
    from the chunk-local cache (steps cross chunk starts)."""
    rng = _rng(44)
    B, H, Dh, L, T, s = 2, 2, 4, 5, 13, 9
    q, k, v = (rng.normal(size=(B, T + s, H, Dh)) for _ in range(3))
    zk, zv = rng.normal(1, 1, size=(2, B, T + s, H, Dh))
    full = LO.local_prefill(q, k, v, zk, zv, L)
    cap = [(T + s) // L] * H
    cache = LO.local_cache_from_prefill(k[:, :T], v[:, :T], zk[:, :T], zv[:, :T], L, cap)
    for i in range(s):
        t = T + i
        out = LO.local_decode_step(cache, q[:, t], k[:, t], v[:, t], zk[:, t], zv[:, t], [t] * B, L)
        _close(out, full[:, t], 1e-12, f"decode step at {t}")


LOCAL_PINS = [lpin_chunks_are_independent, lpin_full_chunk_is_ratplus, lpin_unit_chunks_are_causal_attention,
              lpin_key_positions, lpin_decode_continuation]


def run_local(LO):
    failed = []
    for p in LOCAL_PINS:
        try:
            p(LO)
        except Exception as e:  # noqa: BLE001
            failed.append(f"{p.__name__}: {type(e).__name__}: {e}")
    return failed
