"""rat_decode_step on the GPU against the fp64 oracle's cache semantics."""
import numpy as np
import pytest
import torch

import oracle
from recurrence_augmented_dilated_amd import inputs
from tests.gpu_util import BF16_TOL, F32_TOL, f64, need_gpu, report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _oracle_cache(c, B, H, Dh, dil, W, off, cap):
    gk = f64(c["grid_k"]).reshape(-1)
    gv = f64(c["grid_v"]).reshape(-1)
    grids_k = [gk[B * off[h] * Dh: B * (off[h] + cap[h]) * Dh].reshape(B, cap[h], Dh) for h in range(H)]
    grids_v = [gv[B * off[h] * Dh: B * (off[h] + cap[h]) * Dh].reshape(B, cap[h], Dh) for h in range(H)]
    return oracle.DecodeCache(f64(c["state_k"]), f64(c["state_v"]), f64(c["ring_k"]), f64(c["ring_v"]),
                              grids_k, grids_v, dil, W)


def _decode_run(B, H, Dh, dil, W, pos0, steps, dtype, seed, check_every=1):
    R = need_gpu()
    max_pos = max(pos0) + steps
    off, cap, rows = R.rat_grid_layout(H, dil, max_pos)
    c = inputs.decode_cache(B, H, Dh, dil, W, context=0, steps=0, dtype=dtype, seed=seed)
    # random-fill a cache with the layout for max_pos
    g = torch.Generator().manual_seed(seed)
    c["grid_k"] = torch.randn(B * rows * Dh, generator=g).to(dtype)
    c["grid_v"] = torch.randn(B * rows * Dh, generator=g).to(dtype)
    ref = _oracle_cache(c, B, H, Dh, dil, W, off, cap)
    st = inputs.decode_step_inputs(B, H, Dh, steps, dtype=dtype, seed=seed + 1)
    d = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in c.items()}
    pos = torch.tensor(pos0, dtype=torch.int32, device=DEV)
    worst = 0.0
    for i in range(steps):
        out = R.rat_decode_step(st["q"][i].to(DEV), st["k"][i].to(DEV), st["v"][i].to(DEV),
                                st["zk"][i].to(DEV), st["zv"][i].to(DEV), d["state_k"], d["state_v"],
                                d["grid_k"], d["grid_v"], off, cap, d["ring_k"] if W else None,
                                d["ring_v"] if W else None, pos, max_pos, dil, W)
        want = ref.step(f64(st["q"][i]), f64(st["k"][i]), f64(st["v"][i]), f64(st["zk"][i]),
                        f64(st["zv"][i]), [p + i for p in pos0])
        if i % check_every == 0 or i == steps - 1:
            worst = max(worst, report(f"decode step {i}", f64(out), want))
        pos += 1
    torch.cuda.synchronize()
    return worst, d, ref, off, cap


@pytest.mark.parametrize("W", [8, 0])
def test_decode_bf16_mixed_heads(W):
    dil = [1, 3, 16, 5]
    worst, d, ref, off, cap = _decode_run(3, 4, 128, dil, W, [100, 57, 130], 40, torch.bfloat16, seed=W + 1)
    assert worst <= BF16_TOL
    # final caches
    assert np.max(np.abs(f64(d["state_k"]) - ref.state_k)) <= 1e-4
    assert np.max(np.abs(f64(d["state_v"]) - ref.state_v)) <= 1e-4
    if W:
        assert np.max(np.abs(f64(d["ring_k"]) - ref.ring_k)) <= 2e-2
    gk = f64(d["grid_k"]).reshape(-1)
    B, H, Dh = 3, 4, 128
    for h in range(H):
        blk = gk[B * off[h] * Dh: B * (off[h] + cap[h]) * Dh].reshape(B, cap[h], Dh)
        assert np.max(np.abs(blk - ref.grid_k[h])) <= 2e-2


def test_decode_fp32_dh64():
    worst, *_ = _decode_run(2, 3, 64, [2, 1, 7], 4, [10, 33], 30, torch.float32, seed=7)
    assert worst <= F32_TOL


def test_decode_many_splits():
    """Long D=1 heads with a small batch: several splits per (b, h) and the
    combine kernel."""
    worst, *_ = _decode_run(2, 2, 128, [1, 4], 16, [3000, 2500], 6, torch.bfloat16, seed=11)
    assert worst <= BF16_TOL


def test_decode_from_position_zero():
    """Empty key sets (t < D - 1, W = 0) give zeros; the first steps fill the grid."""
    worst, *_ = _decode_run(2, 2, 128, [4, 1], 0, [0, 0], 12, torch.bfloat16, seed=13)
    assert worst <= BF16_TOL


def test_decode_continues_prefill():
    """Prefill T0 + s tokens equals caches built from the first T0 tokens plus
    s decode steps (both on the GPU), and both match the oracle."""
    R = need_gpu()
    B, H, Dh, T0, s, W = 2, 2, 128, 333, 20, 8
    dil = [4, 1]
    x = inputs.prefill_inputs(B, T0 + s, H, Dh, dtype=torch.float32, seed=31, device=DEV)
    full = R.rat_dilated_prefill(x["q"], x["k"], x["v"], x["zk"], x["zv"], dil, W)
    max_pos = T0 + s
    off, cap, rows = R.rat_grid_layout(H, dil, max_pos)
    grid_k = torch.zeros(B * rows * Dh, device=DEV)
    grid_v = torch.zeros(B * rows * Dh, device=DEV)
    ring_k = torch.zeros((B, H, W, Dh), device=DEV)
    ring_v = torch.zeros((B, H, W, Dh), device=DEV)
    state_k = torch.zeros((B, H, Dh), device=DEV)
    state_v = torch.zeros((B, H, Dh), device=DEV)
    for h, D in enumerate(dil):
        for name, zname, grid, ring, state in (("k", "zk", grid_k, ring_k, state_k),
                                               ("v", "zv", grid_v, ring_v, state_v)):
            xs = x[name][:, :T0, h:h + 1].contiguous()
            zs = x[zname][:, :T0, h:h + 1].contiguous()
            allst, hl = R.rat_scan(xs, zs, store_every=1, want_h_last=True)
            gst, _ = R.rat_scan(xs, zs, store_every=D)
            n = T0 // D
            blk = grid[B * off[h] * Dh: B * (off[h] + cap[h]) * Dh].view(B, cap[h], Dh)
            blk[:, :n] = gst[:, :, 0]
            for p in range(T0 - W, T0):
                ring[:, h, p % W] = allst[:, p, 0]
            state[:, h] = hl[:, 0]
    pos = torch.full((B,), T0, dtype=torch.int32, device=DEV)
    outs = []
    for i in range(s):
        t = T0 + i
        o = R.rat_decode_step(x["q"][:, t].contiguous(), x["k"][:, t].contiguous(), x["v"][:, t].contiguous(),
                              x["zk"][:, t].contiguous(), x["zv"][:, t].contiguous(), state_k, state_v,
                              grid_k, grid_v, off, cap, ring_k, ring_v, pos, max_pos, dil, W)
        outs.append(o.clone())
        pos += 1
    dec = torch.stack(outs, dim=1)
    torch.cuda.synchronize()
    err = report("decode vs prefill (gpu)", f64(dec), f64(full[:, T0:]))
    assert err <= 1e-5
    ref = oracle.prefill(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["zk"]), f64(x["zv"]), dil, W,
                         rows=range(T0, T0 + s))
    assert report("decode vs oracle", f64(dec), ref[:, T0:]) <= F32_TOL


def test_decode_bad_position_flags_error():
    R = need_gpu()
    B, H, Dh, W = 2, 2, 128, 4
    dil = [2, 2]
    max_pos = 50
    off, cap, rows = R.rat_grid_layout(H, dil, max_pos)
    c = inputs.decode_cache(B, H, Dh, dil, W, 0, 0, seed=3, device=DEV)
    gk = torch.randn(B * rows * Dh, device=DEV).to(torch.bfloat16)
    gv = torch.randn(B * rows * Dh, device=DEV).to(torch.bfloat16)
    st = inputs.decode_step_inputs(B, H, Dh, 1, seed=4, device=DEV)
    pos = torch.tensor([10, 50], dtype=torch.int32, device=DEV)   # 50 is out of range
    ws = torch.zeros(R.rat_decode_workspace_size(B, H, Dh, dil, W, max_pos), dtype=torch.uint8, device=DEV)
    sk0 = c["state_k"].clone()
    out = R.rat_decode_step(st["q"][0], st["k"][0], st["v"][0], st["zk"][0], st["zv"][0], c["state_k"],
                            c["state_v"], gk, gv, off, cap, c["ring_k"], c["ring_v"], pos, max_pos, dil, W, ws=ws)
    torch.cuda.synchronize()
    assert R.workspace_error(ws) & 2
    assert torch.all(out[1] == 0)
    assert torch.equal(c["state_k"][1], sk0[1])
    assert not torch.equal(c["state_k"][0], sk0[0])


@pytest.mark.parametrize("seed", range(10))
def test_decode_random(seed):
    """Seeded random batch, heads, head size, dilation mix, window, per-sequence
    start positions (so the sequences of one step sit at different positions)
    and dtype: every step against the oracle's replay."""
    rng = np.random.default_rng(7000 + seed)
    B = int(rng.integers(1, 5))
    H = int(rng.integers(1, 5))
    Dh = int(rng.choice([64, 128]))
    dil = [int(rng.choice([1, 2, 3, 4, 16, 33, 64, 100])) for _ in range(H)]
    W = int(rng.choice([0, 1, 7, 64]))
    pos0 = [int(rng.integers(0, 1500)) for _ in range(B)]
    steps = int(rng.integers(1, 30))
    dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    print(f"[decode-random] seed={seed} B={B} H={H} Dh={Dh} D={dil} W={W} pos0={pos0} steps={steps} {dtype}",
          flush=True)
    worst, *_ = _decode_run(B, H, Dh, dil, W, pos0, steps, dtype, seed=8000 + seed)
    assert worst <= (F32_TOL if dtype == torch.float32 else BF16_TOL)
