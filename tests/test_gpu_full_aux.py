"""Parity at the auxiliary workloads' full sizes -- chunked prefill into a
decode cache, RAT chunk-local prefill, top-k block decode -- built and
launched as the benchmark builds and launches them, on sampled outputs that
the fp64 oracle computes one by one.  Inputs come from the seeded generators
of recurrence_augmented_dilated_amd.inputs and are copied to the host for the
oracle; nothing the oracle sees comes from librat.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import local_oracle as LO
from oracle import topk_oracle as TK
from recurrence_augmented_dilated_amd import inputs
from tests.gpu_util import BF16_TOL, f64, need_gpu, report
from tests.test_gpu_full_configs import _sample_rows
from tests.test_gpu_topk import _check_choice

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]
DEV = "cuda:0"


def _compare_rows(out, x, rows, head_group, ref_fn, what):
    """out [B, T, H, Dh] on the GPU; ref_fn(q, k, v, zk, zv, rows) gives the
    oracle's [B, T, h, Dh] for a group of heads (only `rows` filled)."""
    B, T, H, Dh = out.shape
    ridx = torch.tensor(rows, device=DEV)
    got = f64(out[:, ridx])
    worst = 0.0
    for h0 in range(0, H, head_group):
        hs = slice(h0, h0 + head_group)
        print(f"[full-aux] {what}: oracle heads {h0}..{h0 + head_group - 1}", flush=True)
        q = np.zeros((B, T, head_group, Dh))
        q[:, rows] = f64(x["q"][:, ridx][:, :, hs])
        ref = ref_fn(q, *(f64(x[n][:, :, hs]) for n in ("k", "v", "zk", "zv")), rows)
        worst = max(worst, report(f"{what} heads {h0}+", got[:, :, hs], ref[:, rows]))
    return worst


def test_chunked_prefill_full_size():
    """T = 16384, 16 x 128, D = 16, W = 128 in four chunks of 4096 continuing
    a decode cache: the chunk outputs equal the one-sequence oracle rows
    (sampled, plus the rows around every chunk start), and the final
    recurrent states equal the oracle's."""
    R = need_gpu()
    B, H, Dh, T, D, W, ch = 1, 16, 128, 16384, 16, 128, 4096
    print(f"[full-aux] chunked prefill T={T} chunks of {ch} D={D} W={W}", flush=True)
    x = inputs.prefill_inputs(B, T, H, Dh, dtype=torch.bfloat16, mu=2.0, seed=2, device=DEV)
    max_pos = T + 1024
    off, cap, nrows = R.rat_grid_layout(H, [D] * H, max_pos)
    gk = torch.zeros(B * nrows * Dh, dtype=torch.bfloat16, device=DEV)
    gv = torch.zeros_like(gk)
    rk = torch.zeros((B, H, W, Dh), dtype=torch.bfloat16, device=DEV)
    rv = torch.zeros_like(rk)
    sk = torch.zeros((B, H, Dh), dtype=torch.float32, device=DEV)
    sv = torch.zeros_like(sk)
    outs = []
    for p0 in range(0, T, ch):
        d = {n: t[:, p0:p0 + ch].contiguous() for n, t in x.items()}
        outs.append(R.rat_prefill_chunk(d["q"], d["k"], d["v"], d["zk"], d["zv"], sk, sv, gk, gv, off, cap, rk, rv,
                                        p0, max_pos, [D] * H, W))
    torch.cuda.synchronize()
    out = torch.cat(outs, dim=1)
    rows = set(_sample_rows(T, D, 6))
    for p0 in range(ch, T, ch):
        rows.update(range(p0 - 2, p0 + W + 2))
    rows = sorted(rows)

    def ref(q, k, v, zk, zv, r):
        return oracle.prefill(q, k, v, zk, zv, D, W, rows=r)

    assert _compare_rows(out, x, rows, 8, ref, "chunked prefill") <= BF16_TOL
    Kl = oracle.scan(f64(x["k"]), f64(x["zk"]))[:, -1]
    Vl = oracle.scan(f64(x["v"]), f64(x["zv"]))[:, -1]
    assert np.max(np.abs(f64(sk) - Kl)) <= 1e-4
    assert np.max(np.abs(f64(sv) - Vl)) <= 1e-4


def test_local_prefill_full_size():
    """RAT chunk-local prefill, T = 16384, 16 x 128, L = 16: sampled rows
    (chunk starts included) equal the oracle's."""
    R = need_gpu()
    B, H, Dh, T, L = 1, 16, 128, 16384, 16
    print(f"[full-aux] chunk-local prefill T={T} L={L}", flush=True)
    x = inputs.prefill_inputs(B, T, H, Dh, dtype=torch.bfloat16, mu=2.0, seed=2, device=DEV)
    max_pos = T + 64
    off, cap, nrows = R.rat_grid_layout(H, [L] * H, max_pos)
    gk = torch.zeros(B * nrows * Dh, dtype=torch.bfloat16, device=DEV)
    gv = torch.zeros_like(gk)
    rk = torch.zeros((B, H, 1, Dh), dtype=torch.bfloat16, device=DEV)
    rv = torch.zeros_like(rk)
    sk = torch.zeros((B, H, Dh), dtype=torch.float32, device=DEV)
    sv = torch.zeros_like(sk)
    out = R.rat_local_prefill_chunk(x["q"], x["k"], x["v"], x["zk"], x["zv"], sk, sv, gk, gv, off, cap, rk, rv, 0,
                                    max_pos, L)
    torch.cuda.synchronize()
    rows = _sample_rows(T, L, 9)

    def ref(q, k, v, zk, zv, r):
        return LO.local_prefill(q, k, v, zk, zv, L, rows=r)

    assert _compare_rows(out, x, rows, 8, ref, "chunk-local prefill") <= BF16_TOL


def test_topk_decode_full_size():
    """Top-k decode (Quest), batch 128, context 32768, block 64, top-16, on the
    benchmark's random state cache: 64 steps; for 3 sequences and every head,
    the choice at steps 0, 1, 2 and 63 is a valid top-k under the oracle's
    scores (and almost always the oracle's own), the outputs equal the
    oracle's attention over it, the summary of the block the steps complete
    equals the oracle's statistics, and the final states the oracle's."""
    R = need_gpu()
    B, H, Dh, ctx, blk, k, steps = 128, 16, 128, 32768, 64, 16, 64
    max_pos = (ctx + steps + blk + blk - 1) // blk * blk
    print(f"[full-aux] top-k decode B={B} ctx={ctx} block={blk} k={k} steps={steps}", flush=True)
    cache = R.topk_cache(B, H, Dh, max_pos, blk, torch.bfloat16, DEV)
    inputs.fill_topk_cache(cache, seed=7)
    R.rat_topk_summarize(cache, 0, ctx // blk, max_pos, blk)
    st = inputs.decode_step_inputs(B, H, Dh, steps, mu=2.0, seed=5, device=DEV)
    bs = [0, 77, 127]
    # host copies of the sampled sequences before decoding: [b, position, h, Dh]
    ck0 = f64(cache["cache_k"][:, bs, :ctx]).transpose(1, 2, 0, 3)
    cv0 = f64(cache["cache_v"][:, bs, :ctx]).transpose(1, 2, 0, 3)
    sk0, sv0 = f64(cache["state_k"][bs]), f64(cache["state_v"][bs])
    check = (0, 1, 2, steps - 1)
    pos = torch.full((B,), ctx, dtype=torch.int32, device=DEV)
    outs, chs = {}, {}
    for i in range(steps):
        chosen = torch.full((B, H, k), -7, dtype=torch.int32, device=DEV)
        o = R.rat_topk_decode_step(st["q"][i], st["k"][i], st["v"][i], st["zk"][i], st["zv"][i], cache, pos,
                                   max_pos, blk, k, 0, chosen=chosen)
        if i in check:
            outs[i], chs[i] = f64(o[bs]), chosen[bs].cpu().numpy()
        pos += 1
    torch.cuda.synchronize()

    xs = {n: f64(st[n][:, bs]).transpose(1, 0, 2, 3) for n in st}   # [b, step, h, Dh]
    Kn = oracle.scan(xs["k"], xs["zk"], h0=sk0)
    Vn = oracle.scan(xs["v"], xs["zv"], h0=sv0)
    Kt = np.concatenate([ck0, Kn], axis=1)
    Vt = np.concatenate([cv0, Vn], axis=1)
    del ck0, cv0
    Kr = torch.from_numpy(Kt).to(torch.bfloat16).double().numpy()   # rows as the cache stores them
    kmin, kmax, kmean = TK.block_stats(Kr, blk)
    scale = oracle.default_scale(Dh)
    worst, agree, total = 0.0, 0, 0
    for i in check:
        t = ctx + i
        for bi in range(len(bs)):
            for h in range(H):
                q = xs["q"][bi, i, h]
                sel, same = _check_choice(chs[i][bi, h], q, kmin[bi, :, h], kmax[bi, :, h], kmean[bi, :, h], t, blk,
                                          k, TK.QUEST)
                want = TK.attend_selected(q, Kt[bi, :, h], Vt[bi, :, h], t, blk, sel, scale)
                worst = max(worst, float(np.max(np.abs(outs[i][bi, h] - want))))
                agree += same
                total += 1
    print(f"[full-aux] top-k decode: max_abs={worst:.3e}, choice equal to the oracle's for {agree}/{total}",
          flush=True)
    assert worst <= BF16_TOL
    assert agree >= 0.97 * total
    jb = ctx // blk                         # the block the 64 steps complete
    summ = f64(cache["summary"][:, bs, jb])  # [h, b, 3, Dh]
    for s_i, ref in enumerate((kmin, kmax, kmean)):
        assert np.max(np.abs(summ[:, :, s_i] - ref[:, jb].transpose(1, 0, 2))) <= BF16_TOL
    assert np.max(np.abs(f64(cache["state_k"][bs]) - Kn[:, -1])) <= 1e-4
    assert np.max(np.abs(f64(cache["state_v"][bs]) - Vn[:, -1])) <= 1e-4
