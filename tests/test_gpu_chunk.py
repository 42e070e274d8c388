"""Prefill continuing a decode cache (rat_prefill_chunk) against the fp64
oracle.  A sequence prefilled in chunks must give the rows of one prefill
over the whole sequence, leave behind the cache the oracle builds for that
prefix (state, grid entries, ring slots), and decoding on from that cache
must give the rows of the longer prefill (continuation pin P8 on the GPU).
Inputs are seeded (recurrence_augmented_dilated_amd.inputs); every expected
value comes from the oracle."""
import numpy as np
import pytest
import torch

import oracle
from recurrence_augmented_dilated_amd import inputs
from tests.gpu_util import BF16_TOL, F32_TOL, f64, need_gpu, report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(B, H, Dh, dil, W, chunks, dtype, decode_steps, seed, mu=2.0):
    R = need_gpu()
    tol = BF16_TOL if dtype == torch.bfloat16 else F32_TOL
    L = sum(chunks)
    total = L + decode_steps
    print(f"[chunk] B={B} H={H} Dh={Dh} D={dil} W={W} chunks={chunks} {dtype} decode={decode_steps}", flush=True)
    x = inputs.prefill_inputs(B, total, H, Dh, dtype=dtype, mu=mu, seed=seed)
    ref = oracle.prefill(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["zk"]), f64(x["zv"]), dil, W)
    max_pos = total + 64
    off, cap, rows = R.rat_grid_layout(H, dil, max_pos)
    grid_k = torch.zeros(B * rows * Dh, dtype=dtype, device=DEV)
    grid_v = torch.zeros(B * rows * Dh, dtype=dtype, device=DEV)
    ring_k = torch.zeros((B, H, W, Dh), dtype=dtype, device=DEV) if W > 0 else None
    ring_v = torch.zeros((B, H, W, Dh), dtype=dtype, device=DEV) if W > 0 else None
    state_k = torch.zeros((B, H, Dh), dtype=torch.float32, device=DEV)
    state_v = torch.zeros((B, H, Dh), dtype=torch.float32, device=DEV)

    worst = 0.0
    p0 = 0
    for T in chunks:
        sl = slice(p0, p0 + T)
        d = {n: t[:, sl].contiguous().to(DEV) for n, t in x.items()}
        out = R.rat_prefill_chunk(d["q"], d["k"], d["v"], d["zk"], d["zv"], state_k, state_v, grid_k, grid_v,
                                  off, cap, ring_k, ring_v, p0, max_pos, dil, W)
        torch.cuda.synchronize()
        worst = max(worst, report(f"chunk p0={p0} T={T}", f64(out), ref[:, sl]))
        p0 += T

    # the cache after the prefix equals the oracle's
    cache = oracle.DecodeCache.from_prefill(f64(x["k"][:, :L]), f64(x["v"][:, :L]), f64(x["zk"][:, :L]),
                                            f64(x["zv"][:, :L]), dil, W, cap=cap)
    st_tol = 1e-4
    assert np.max(np.abs(f64(state_k) - cache.state_k)) <= st_tol
    assert np.max(np.abs(f64(state_v) - cache.state_v)) <= st_tol
    for h in range(H):
        n = L // dil[h]
        gk = f64(grid_k[B * off[h] * Dh: B * (off[h] + cap[h]) * Dh].view(B, cap[h], Dh))
        gv = f64(grid_v[B * off[h] * Dh: B * (off[h] + cap[h]) * Dh].view(B, cap[h], Dh))
        assert np.max(np.abs(gk[:, :n] - cache.grid_k[h][:, :n]), initial=0.0) <= tol, h
        assert np.max(np.abs(gv[:, :n] - cache.grid_v[h][:, :n]), initial=0.0) <= tol, h
    if W > 0:
        for p in range(max(0, L - W), L):
            assert np.max(np.abs(f64(ring_k[:, :, p % W]) - cache.ring_k[:, :, p % W])) <= tol, p
            assert np.max(np.abs(f64(ring_v[:, :, p % W]) - cache.ring_v[:, :, p % W])) <= tol, p

    # decoding on from the cache gives the rows of the longer prefill
    pos = torch.full((B,), L, dtype=torch.int32, device=DEV)
    for i in range(decode_steps):
        t = L + i
        d = {n: x[n][:, t].contiguous().to(DEV) for n in x}
        o = R.rat_decode_step(d["q"], d["k"], d["v"], d["zk"], d["zv"], state_k, state_v, grid_k, grid_v,
                              off, cap, ring_k, ring_v, pos, max_pos, dil, W)
        torch.cuda.synchronize()
        worst = max(worst, report(f"decode t={t}", f64(o), ref[:, t]))
        pos += 1
    return worst, tol


@pytest.mark.parametrize("case", [
    # B, H, Dh, dilation, W, chunks, dtype, decode steps
    (2, 4, 128, [4, 16, 1, 64], 96, [256, 384, 360], torch.bfloat16, 8),
    (1, 2, 64, [8, 3], 0, [64, 64, 192, 100], torch.bfloat16, 4),
    (1, 3, 128, [2, 5, 32], 200, [64, 64, 64, 130], torch.bfloat16, 6),   # chunks shorter than W
    (1, 2, 128, [16, 4], 300, [100], torch.bfloat16, 40),                # one chunk: prefill -> decode handoff
    (2, 2, 64, [4, 16], 1, [128, 320, 77], torch.bfloat16, 3),
    (1, 2, 64, [4, 16], 40, [128, 200], torch.float32, 4),
    (1, 2, 128, [1, 7], 0, [192, 64, 5], torch.float32, 3),
])
def test_chunked_prefill_then_decode(case):
    B, H, Dh, dil, W, chunks, dtype, steps = case
    worst, tol = _run(B, H, Dh, dil, W, chunks, dtype, steps, seed=11)
    assert worst <= tol


def test_chunk_equals_one_shot_prefill():
    """Chunks of a sequence and one rat_dilated_prefill over it agree (both
    compared with each other directly, to the bf16 tolerance)."""
    R = need_gpu()
    B, H, Dh, dil, W, L = 1, 4, 128, [16, 16, 64, 4], 128, 2048
    x = {n: t.to(DEV) for n, t in inputs.prefill_inputs(B, L, H, Dh, dtype=torch.bfloat16, seed=5).items()}
    one = R.rat_dilated_prefill(x["q"], x["k"], x["v"], x["zk"], x["zv"], dil, W)
    off, cap, rows = R.rat_grid_layout(H, dil, L)
    gk = torch.zeros(B * rows * Dh, dtype=torch.bfloat16, device=DEV)
    gv = torch.zeros_like(gk)
    rk = torch.zeros((B, H, W, Dh), dtype=torch.bfloat16, device=DEV)
    rv = torch.zeros_like(rk)
    sk = torch.zeros((B, H, Dh), dtype=torch.float32, device=DEV)
    sv = torch.zeros_like(sk)
    outs = []
    for p0, T in ((0, 512), (512, 1024), (1536, 512)):
        sl = slice(p0, p0 + T)
        d = {n: t[:, sl].contiguous() for n, t in x.items()}
        outs.append(R.rat_prefill_chunk(d["q"], d["k"], d["v"], d["zk"], d["zv"], sk, sv, gk, gv, off, cap,
                                        rk, rv, p0, L, dil, W))
    torch.cuda.synchronize()
    err = report("chunks vs one call", f64(torch.cat(outs, dim=1)), f64(one))
    assert err <= BF16_TOL


def _random_case(seed):
    rng = np.random.default_rng(3000 + seed)
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 5))
    Dh = int(rng.choice([64, 128]))
    dil = [int(rng.choice([1, 2, 3, 4, 16, 33, 64, 100])) for _ in range(H)]
    W = int(rng.choice([0, 1, 7, 64, 130]))
    n = int(rng.integers(1, 4))
    chunks = [64 * int(rng.integers(1, 6)) for _ in range(n - 1)] + [int(rng.integers(1, 400))]
    dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    steps = int(rng.integers(1, 40))
    return B, H, Dh, dil, W, chunks, dtype, steps


@pytest.mark.parametrize("seed", range(12))
def test_chunked_prefill_random(seed):
    """Seeded random chunk splits, head mixes, windows and dtypes: chunk
    outputs, caches and the decode steps that follow against the oracle."""
    B, H, Dh, dil, W, chunks, dtype, steps = _random_case(seed)
    print(f"[chunk-random] seed={seed} B={B} H={H} Dh={Dh} D={dil} W={W} chunks={chunks} {dtype} decode={steps}",
          flush=True)
    worst, tol = _run(B, H, Dh, dil, W, chunks, dtype, steps, seed=4000 + seed)
    assert worst <= tol
