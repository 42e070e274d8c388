"""Top-k block attention over the memory states (rat_topk_prefill,
rat_topk_decode_step) against the fp64 oracle (oracle.topk_oracle).

The block choice is a floating-point decision: the kernel scores in fp32, the
oracle in fp64, so near-ties may fall either way.  Each test therefore checks
that the kernel's choice is a valid top-k under the oracle's scores (every
chosen block scores at least as high as every unchosen candidate, up to a
bound on the fp32 rounding of the two scores), compares the outputs with the
oracle's attention over the kernel's own choice, and requires the choice to
equal the oracle's own for almost every query.  Caches and block summaries
are compared with the oracle's states and statistics."""
import numpy as np
import pytest
import torch

import oracle
from oracle import topk_oracle as TK
from recurrence_augmented_dilated_amd import inputs
from tests.gpu_util import BF16_TOL, F32_TOL, f64, need_gpu, report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
METHODS = {0: TK.QUEST, 1: TK.MOBA}


def _check_choice(sel_row, q_row, kmin, kmax, kmean, t, block, topk, method):
    """sel_row: the kernel's chosen blocks (-1 padded) for one query; stats
    [nb, Dh] of its (b, h), taken over the states rounded to the cache type
    (the precision the kernel decides in).  Returns (choice, equal to the
    oracle's)."""
    local = t // block
    cand = list(range(1, local))
    sel = [int(x) for x in sel_row if x >= 0]
    assert all(x == -1 for x in sel_row[len(sel):]), sel_row
    assert sel == sorted(set(sel)) and all(1 <= j < local for j in sel), (t, sel)
    assert len(sel) == min(topk, len(cand)), (t, sel, topk, len(cand))
    scores = {j: TK.block_score(q_row, kmin[j], kmax[j], kmean[j], method) for j in cand}
    if method == TK.QUEST:
        bound = {j: float(np.sum(np.abs(q_row) * np.maximum(np.abs(kmin[j]), np.abs(kmax[j])))) for j in cand}
    else:
        bound = {j: float(np.sum(np.abs(q_row) * np.abs(kmean[j]))) + float(np.sum(np.abs(q_row))) * 0.02 for j in cand}
    # fp32 scoring, plus one state element rounded the other way at a
    # rounding boundary (fp32 vs fp64 recurrence)
    flip = {j: float(np.max(np.abs(q_row) * np.maximum(np.abs(kmin[j]), np.abs(kmax[j])))) * 2.0 ** -7 for j in cand}
    eps = {j: 2e-5 * bound[j] + flip[j] + 1e-6 for j in cand}
    for c in sel:
        for u in set(cand) - set(sel):
            assert scores[c] >= scores[u] - (eps[c] + eps[u]), (t, c, u, scores[c], scores[u])
    return sel, sel == TK.select_blocks(t, block, topk, [scores.get(j, -np.inf) for j in range(max(local, 1))])


def _verify(out, chosen, q, Kt, Vt, t_list, block, topk, method, tol, stats, what):
    """out/chosen: GPU results for queries (b, t, h) -> rows; checks choice and output."""
    agree = total = 0
    worst = 0.0
    kmin, kmax, kmean = stats
    scale = oracle.default_scale(q.shape[-1])
    for (b, t, h), (o_row, s_row) in zip(t_list, zip(out, chosen)):
        sel, same = _check_choice(s_row, q[b, t, h], kmin[b, :, h], kmax[b, :, h], kmean[b, :, h], t, block, topk,
                                  method)
        want = TK.attend_selected(q[b, t, h], Kt[b, :, h], Vt[b, :, h], t, block, sel, scale)
        worst = max(worst, float(np.max(np.abs(o_row - want))))
        agree += same
        total += 1
    print(f"[topk] {what}: max_abs={worst:.3e}, choice equal to the oracle's for {agree}/{total}", flush=True)
    assert worst <= tol, what
    assert agree >= 0.97 * total, (agree, total)


def _run(B, H, Dh, block, topk, score, chunks, decode_steps, dtype, seed, mu=1.5):
    R = need_gpu()
    tol = BF16_TOL if dtype == torch.bfloat16 else F32_TOL
    method = METHODS[score]
    L = sum(chunks)
    total = L + decode_steps
    max_pos = (total + block - 1) // block * block + block
    print(f"[topk] B={B} H={H} Dh={Dh} block={block} topk={topk} {method} chunks={chunks} decode={decode_steps} "
          f"{dtype}", flush=True)
    x = inputs.prefill_inputs(B, total, H, Dh, dtype=dtype, mu=mu, seed=seed)
    q = f64(x["q"])
    Kt = oracle.scan(f64(x["k"]), f64(x["zk"]))
    Vt = oracle.scan(f64(x["v"]), f64(x["zv"]))
    Kr = torch.from_numpy(Kt).to(dtype).double().numpy()   # states as the cache stores them
    cache = R.topk_cache(B, H, Dh, max_pos, block, dtype, DEV)
    p0 = 0
    for T in chunks:
        sl = slice(p0, p0 + T)
        d = {n: t[:, sl].contiguous().to(DEV) for n, t in x.items()}
        chosen = torch.full((B, T, H, max(topk, 1)), -7, dtype=torch.int32, device=DEV)
        out = R.rat_topk_prefill(d["q"], d["k"], d["v"], d["zk"], d["zv"], cache, p0, max_pos, block, topk, score,
                                 chosen=chosen if topk > 0 else None)
        torch.cuda.synchronize()
        stats = TK.block_stats(Kr[:, :p0 + T], block)
        keys = [(b, p0 + i, h) for b in range(B) for i in range(T) for h in range(H)]
        o = f64(out).reshape(B * T * H, Dh)
        c = chosen.cpu().numpy().reshape(B * T * H, -1) if topk > 0 else np.full((B * T * H, 1), -1)
        _verify(o, c[:, :topk] if topk > 0 else np.zeros((B * T * H, 0), dtype=int), q, Kt, Vt, keys, block, topk,
                method, tol, stats, f"prefill p0={p0} T={T}")
        p0 += T
    # caches and summaries after the prefix
    ck = f64(cache["cache_k"])            # [H, B, max_pos, Dh]
    for h in range(H):
        assert np.max(np.abs(ck[h, :, :L] - Kt[:, :L, h])) <= tol
        assert np.max(np.abs(f64(cache["cache_v"])[h, :, :L] - Vt[:, :L, h])) <= tol
    smin, smax, smean = TK.block_stats(Kt[:, :L], block)
    summ = f64(cache["summary"])         # [H, B, nb, 3, Dh]
    nb = L // block
    for h in range(H):
        for s_i, ref in enumerate((smin, smax, smean)):
            assert np.max(np.abs(summ[h, :, :nb, s_i] - ref[:, :nb, h]), initial=0.0) <= tol
    assert np.max(np.abs(f64(cache["state_k"]) - Kt[:, L - 1])) <= 1e-4
    # decode on
    pos = torch.full((B,), L, dtype=torch.int32, device=DEV)
    outs, chs, keys = [], [], []
    for i in range(decode_steps):
        t = L + i
        d = {n: x[n][:, t].contiguous().to(DEV) for n in x}
        chosen = torch.full((B, H, max(topk, 1)), -7, dtype=torch.int32, device=DEV)
        o = R.rat_topk_decode_step(d["q"], d["k"], d["v"], d["zk"], d["zv"], cache, pos, max_pos, block, topk,
                                   score, chosen=chosen if topk > 0 else None)
        torch.cuda.synchronize()
        outs.append(f64(o).reshape(B * H, Dh))
        chs.append(chosen.cpu().numpy().reshape(B * H, -1)[:, :topk])
        keys += [(b, t, h) for b in range(B) for h in range(H)]
        pos += 1
    if decode_steps:
        stats = TK.block_stats(Kr, block)
        _verify(np.concatenate(outs), np.concatenate(chs), q, Kt, Vt, keys, block, topk, method, tol, stats, "decode")


@pytest.mark.parametrize("score", [0, 1], ids=["quest", "moba"])
def test_topk_prefill_bf16(score):
    _run(2, 2, 128, 64, 4, score, [1024], 0, torch.bfloat16, seed=31)


@pytest.mark.parametrize("score", [0, 1], ids=["quest", "moba"])
def test_topk_chunks_then_decode(score):
    """Chunks not aligned to blocks, then decode steps that complete blocks."""
    _run(1, 3, 64, 32, 3, score, [300, 200], 70, torch.bfloat16, seed=32)


def test_topk_fp32():
    _run(1, 2, 64, 16, 2, 0, [160, 96], 40, torch.float32, seed=33)


@pytest.mark.parametrize("topk", [0, 100])
def test_topk_degenerate_budgets(topk):
    """topk = 0: first + local block only; topk above the candidate count: every block."""
    _run(1, 2, 128, 32, topk, 1, [256], 20, torch.bfloat16, seed=34)


def test_topk_block_of_one():
    _run(1, 1, 64, 1, 5, 0, [48], 16, torch.bfloat16, seed=35)


def test_topk_decode_bad_position():
    R = need_gpu()
    B, H, Dh, block, max_pos = 2, 2, 64, 16, 128
    cache = R.topk_cache(B, H, Dh, max_pos, block, torch.bfloat16, DEV)
    st = inputs.decode_step_inputs(B, H, Dh, 1, seed=3, device=DEV)
    ws = torch.zeros(R.lib().rat_topk_decode_workspace_size(), dtype=torch.uint8, device=DEV)
    pos = torch.tensor([5, max_pos], dtype=torch.int32, device=DEV)
    out = R.rat_topk_decode_step(st["q"][0], st["k"][0], st["v"][0], st["zk"][0], st["zv"][0], cache, pos, max_pos,
                                 block, 2, 0, ws=ws)
    torch.cuda.synchronize()
    assert R.workspace_error(ws) & 2
    assert torch.all(out[1] == 0)
    assert torch.all(cache["cache_k"][:, 1] == 0)     # the bad sequence's cache is untouched
    assert torch.any(cache["cache_k"][:, 0, 5] != 0)


def test_topk_summarize_matches_block_statistics():
    """rat_topk_summarize over a cache filled by other means equals the
    oracle's block statistics of the same (bf16) values."""
    R = need_gpu()
    B, H, Dh, block, max_pos = 2, 3, 128, 32, 512
    cache = R.topk_cache(B, H, Dh, max_pos, block, torch.bfloat16, DEV)
    g = torch.Generator(device=DEV).manual_seed(7)
    cache["cache_k"].copy_(torch.randn(cache["cache_k"].shape, generator=g, device=DEV).to(torch.bfloat16))
    R.rat_topk_summarize(cache, 2, 12, max_pos, block)
    torch.cuda.synchronize()
    ck = f64(cache["cache_k"])                       # [H, B, max_pos, Dh]
    kmin, kmax, kmean = TK.block_stats(np.transpose(ck, (1, 2, 0, 3)), block)   # [B, nb, H, Dh]
    s = f64(cache["summary"])                        # [H, B, nb, 3, Dh]
    for h in range(H):
        for i, ref in enumerate((kmin, kmax, kmean)):
            assert np.max(np.abs(s[h, :, 2:12, i] - ref[:, 2:12, h])) <= 1e-5
        assert np.all(s[h, :, :2] == 0) and np.all(s[h, :, 12:] == 0)   # other blocks untouched


# bf16, block 64, from position 0: the selection pass plus the MFMA prefill
# attention over the per-query block sets (top-k <= 16); above that top-k the
# same call takes one workgroup per query.
BLOCK64_CASES = [
    (1, 3, 64, 16, 1, 1000),    # ragged T, the largest top-k of the MFMA path
    (2, 2, 128, 0, 0, 640),     # first and own block only; lists kept in the workspace
    (1, 2, 128, 16, 0, 448),    # at most 5 candidates: every one kept
    (1, 2, 64, 20, 1, 512),     # top-k above the MFMA path's limit
]


@pytest.mark.parametrize("case", BLOCK64_CASES, ids=["ragged-k16", "k0", "all-kept", "k20"])
def test_topk_prefill_block64(case):
    B, H, Dh, topk, score, T = case
    _run(B, H, Dh, 64, topk, score, [T], 0, torch.bfloat16, seed=36)


def test_topk_prefill_lists_in_workspace():
    """Without a chosen buffer the selection lists live in the workspace: the
    output is the same as with one."""
    R = need_gpu()
    B, H, Dh, T, block, topk = 1, 2, 128, 768, 64, 8
    max_pos = T + block
    x = inputs.prefill_inputs(B, T, H, Dh, dtype=torch.bfloat16, mu=1.5, seed=37)
    d = {n: t.contiguous().to(DEV) for n, t in x.items()}
    outs = []
    for with_chosen in (True, False):
        cache = R.topk_cache(B, H, Dh, max_pos, block, torch.bfloat16, DEV)
        chosen = torch.full((B, T, H, topk), -7, dtype=torch.int32, device=DEV) if with_chosen else None
        outs.append(R.rat_topk_prefill(d["q"], d["k"], d["v"], d["zk"], d["zv"], cache, 0, max_pos, block, topk, 1,
                                       chosen=chosen).clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def _sampled_prefill(B, H, Dh, T, block, topk, score, seed, rows, what, mu=2.0):
    """One rat_topk_prefill call from position 0 over T rows; the chosen
    lists and outputs of the sampled (b, t, h) rows are checked against the
    oracle (validated choice, attention over it)."""
    R = need_gpu()
    max_pos = T + block
    x = inputs.prefill_inputs(B, T, H, Dh, dtype=torch.bfloat16, mu=mu, seed=seed)
    q = f64(x["q"])
    Kt = oracle.scan(f64(x["k"]), f64(x["zk"]))
    Vt = oracle.scan(f64(x["v"]), f64(x["zv"]))
    Kr = torch.from_numpy(Kt).to(torch.bfloat16).double().numpy()
    cache = R.topk_cache(B, H, Dh, max_pos, block, torch.bfloat16, DEV)
    d = {n: t.contiguous().to(DEV) for n, t in x.items()}
    chosen = torch.full((B, T, H, topk), -7, dtype=torch.int32, device=DEV)
    out = R.rat_topk_prefill(d["q"], d["k"], d["v"], d["zk"], d["zv"], cache, 0, max_pos, block, topk, score,
                             chosen=chosen)
    torch.cuda.synchronize()
    o = f64(out)
    c = chosen.cpu().numpy()
    _verify([o[b, t, h] for b, t, h in rows], [c[b, t, h] for b, t, h in rows], q, Kt, Vt, rows, block, topk,
            METHODS[score], BF16_TOL, TK.block_stats(Kr, block), what)


def test_topk_prefill_full_size_sampled():
    """T = 4096, 16 x 128, block 64, top-16 MoBA (the top-k prefill workload):
    sampled rows against the oracle's attention over the kernel's (validated)
    choice."""
    T, H = 4096, 16
    rng = np.random.default_rng(39)
    rows = [(0, int(t), int(h)) for t, h in zip(rng.integers(0, T, 256), rng.integers(0, H, 256))]
    rows += [(0, T - 1, 0), (0, 0, 1), (0, 63, 2), (0, 64, 3)]
    _sampled_prefill(1, H, 128, T, 64, 16, 1, 38, rows, "prefill T=4096 sampled")


def _long_rows(T, H, seed):
    """The last rows (the most candidates), rows at block edges and random rows."""
    rng = np.random.default_rng(seed)
    ts = {T - 1, T - 2, T - 63, T - 64, T - 65, 0, 63, 64, 127, 128, 4095, 4096}
    ts.update(int(t) for t in rng.integers(T // 2, T, 96))
    ts.update(int(t) for t in rng.integers(0, T, 32))
    return [(0, t, h) for t in sorted(ts) for h in range(H)]


@pytest.mark.parametrize("score", [0, 1], ids=["quest", "moba"])
def test_topk_prefill_tile_select_at_its_limit(score):
    """T = 64 * 257, the longest sequence the per-tile selection kernel takes
    (its candidate summaries fill the most LDS: 255 candidates per query)."""
    T, H = 64 * 257, 2
    _sampled_prefill(1, H, 128, T, 64, 16, score, 51 + score, _long_rows(T, H, 52), f"prefill T={T} tile select")


@pytest.mark.parametrize("score", [0, 1], ids=["quest", "moba"])
def test_topk_prefill_per_query_select_branch(score):
    """T = 64 * 258, one block past the per-tile selection's limit: the lists
    come from the per-query selection pass (written, attention skipped), then
    the MFMA attention walks them."""
    T, H = 64 * 258, 2
    _sampled_prefill(1, H, 128, T, 64, 16, score, 53 + score, _long_rows(T, H, 54), f"prefill T={T} per-query select")


def test_topk_prefill_many_candidates_sampled():
    """More than 1024 candidate blocks (block 4, T = 4200): the selection by
    repeated argmax; sampled rows among the last queries and a few early
    ones against the oracle."""
    R = need_gpu()
    B, H, Dh, T, block, topk, score = 1, 2, 64, 4200, 4, 3, 0
    max_pos = T + block
    x = inputs.prefill_inputs(B, T, H, Dh, dtype=torch.bfloat16, mu=1.5, seed=40)
    q = f64(x["q"])
    Kt = oracle.scan(f64(x["k"]), f64(x["zk"]))
    Vt = oracle.scan(f64(x["v"]), f64(x["zv"]))
    Kr = torch.from_numpy(Kt).to(torch.bfloat16).double().numpy()
    cache = R.topk_cache(B, H, Dh, max_pos, block, torch.bfloat16, DEV)
    d = {n: t.contiguous().to(DEV) for n, t in x.items()}
    chosen = torch.full((B, T, H, topk), -7, dtype=torch.int32, device=DEV)
    out = R.rat_topk_prefill(d["q"], d["k"], d["v"], d["zk"], d["zv"], cache, 0, max_pos, block, topk, score,
                             chosen=chosen)
    torch.cuda.synchronize()
    o = f64(out)
    c = chosen.cpu().numpy()
    rows = [(0, t, h) for t in (T - 1, T - 2, T - 37, 4105, 4101) for h in range(H)] + [(0, 200, 0), (0, 9, 1)]
    _verify([o[b, t, h] for b, t, h in rows], [c[b, t, h] for b, t, h in rows], q, Kt, Vt, rows, block, topk,
            TK.QUEST, BF16_TOL, TK.block_stats(Kr, block), "prefill T=4200 block=4")


def _random_case(seed):
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 4))
    Dh = int(rng.choice([64, 128]))
    block = int(rng.choice([16, 32, 64]))
    topk = int(rng.choice([0, 1, 4, 16, 20]))
    score = int(rng.integers(0, 2))
    n = int(rng.integers(1, 3))
    chunks = [int(rng.integers(1, 700)) for _ in range(n)]
    steps = int(rng.integers(0, 20))
    dtype = torch.float32 if rng.random() < 0.25 else torch.bfloat16
    return B, H, Dh, block, topk, score, chunks, steps, dtype


@pytest.mark.parametrize("seed", range(8))
def test_topk_random(seed):
    """Seeded random block sizes, budgets, scores, chunkings and dtypes
    (including the block-64 MFMA path when the draw allows it)."""
    B, H, Dh, block, topk, score, chunks, steps, dtype = _random_case(seed)
    _run(B, H, Dh, block, topk, score, chunks, steps, dtype, seed=6000 + seed)


@pytest.mark.parametrize("score", [0, 1], ids=["quest", "moba"])
def test_topk_prefill_tied_scores(score):
    """A zero query (+0 in head 0, -0 in head 1) scores every candidate block
    exactly 0 (as +0 or -0): ties go to the lower index, so each query keeps
    blocks 1 .. min(k, candidates), in order.  T spans fewer and more than 64
    candidates per query."""
    R = need_gpu()
    B, H, Dh, block, topk, T = 1, 2, 128, 64, 16, 64 * 72
    max_pos = T + block
    x = inputs.prefill_inputs(B, T, H, Dh, dtype=torch.bfloat16, mu=2.0, seed=41)
    d = {n: t.contiguous().to(DEV) for n, t in x.items()}
    d["q"] = torch.zeros_like(d["q"])
    d["q"][:, :, 1] = -0.0
    cache = R.topk_cache(B, H, Dh, max_pos, block, torch.bfloat16, DEV)
    chosen = torch.full((B, T, H, topk), -7, dtype=torch.int32, device=DEV)
    R.rat_topk_prefill(d["q"], d["k"], d["v"], d["zk"], d["zv"], cache, 0, max_pos, block, topk, score, chosen=chosen)
    torch.cuda.synchronize()
    got = chosen.cpu().numpy()
    assert np.signbit(d["q"][0, 0, 1, 0].cpu().float().numpy())
    for t in range(T):
        nsel = min(topk, max(t // block - 1, 0))
        want = list(range(1, nsel + 1)) + [-1] * (topk - nsel)
        for h in range(H):
            assert got[0, t, h].tolist() == want, (t, h, got[0, t, h].tolist())
