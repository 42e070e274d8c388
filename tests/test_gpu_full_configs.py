"""Parity at the benchmark workloads' full sizes, in the launch configuration
the benchmark times, on sampled outputs that the fp64 oracle computes one by
one.  Inputs are generated on the GPU with torch's seeded generator and
copied to the host for the oracle; nothing the oracle sees comes from librat.

Samples: the T=16384 prefill is compared on its full output; the longer and
hybrid prefills on rows at the start (t < 2D), around grid boundaries in eight
regions, the last 256 rows and seeded random rows, every head; decode: 8 or 4
sequences, all heads, the outputs at steps {0, 1, 2, 15, 16, 63, 64, 65, 511,
1023} and the final recurrent states, ring and grid rows.

With N(0, 1) inputs attention is nearly uniform, so a key-set slip of one
position moves an output by ~1/|S_t|, far below the bf16 tolerance.  The
planted-key tests below therefore run the same launch shapes on inputs where
one key decides each boundary row (see _planted_inputs).
"""
import numpy as np
import pytest
import torch

import oracle
from recurrence_augmented_dilated_amd import inputs
from tests.gpu_util import BF16_TOL, RMS_TOL, f64, need_gpu, report

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]
DEV = "cuda:0"


def _sample_rows(T, D, seed, n_random=256):
    rows = set(range(min(T, 2 * D)))
    for k in range(8):
        c = (T // 8) * k + D * 7
        c = (c // D) * D
        rows.update(t for t in range(c - 2, c + 1) if 0 <= t < T)
    rows.update(range(max(0, T - 256), T))
    rng = np.random.default_rng(seed)
    rows.update(int(x) for x in rng.integers(0, T, n_random))
    return sorted(rows)


def _prefill_check(B, T, H, Dh, D, W, mu, seed, head_group, all_rows=False, x=None, rows=None,
                   rms_max=RMS_TOL):
    R = need_gpu()
    print(f"[full] prefill B={B} T={T} H={H} D={D} W={W}: generating inputs", flush=True)
    if x is None:
        x = inputs.prefill_inputs(B, T, H, Dh, dtype=torch.bfloat16, mu=mu, seed=seed, device=DEV)
    out = R.rat_dilated_prefill(x["q"], x["k"], x["v"], x["zk"], x["zv"], D, W)
    torch.cuda.synchronize()
    Ds = D if isinstance(D, list) else [D] * H
    if all_rows:
        rows = list(range(T))
    elif rows is None:
        rows = sorted(set().union(*(_sample_rows(T, d, seed) for d in sorted(set(Ds)))))
    ridx = torch.tensor(rows, device=DEV)
    got = f64(out[:, ridx])
    worst = 0.0
    for h0 in range(0, H, head_group):
        hs = slice(h0, h0 + head_group)
        print(f"[full]   oracle heads {h0}..{h0 + head_group - 1}", flush=True)
        Kt = oracle.scan(f64(x["k"][:, :, hs]), f64(x["zk"][:, :, hs]))
        Vt = oracle.scan(f64(x["v"][:, :, hs]), f64(x["zv"][:, :, hs]))
        q = np.zeros((B, T, head_group, Dh))
        q[:, rows] = f64(x["q"][:, ridx][:, :, hs])
        ref = oracle.prefill(q, None, None, None, None, Ds[hs], W, rows=rows, states=(Kt, Vt))
        worst = max(worst, report(f"prefill T={T} heads {h0}+", got[:, :, hs], ref[:, rows], rms_max=rms_max))
        del Kt, Vt, q, ref
    return worst


def test_config2_prefill_full_size():
    """B=1, 16 x 128, T=16384, D=16, W=128, bf16, z ~ N(2,1): every output
    row of every head against the oracle."""
    assert _prefill_check(1, 16384, 16, 128, 16, 128, 2.0, 2, head_group=16, all_rows=True) <= BF16_TOL


def test_hybrid_head_prefill_full_size():
    """B=1, 32 x 128, T=16384, W=64, per-head dilation 8 x D=1, 12 x 16,
    12 x 64 (the hybrid-head mix), bf16, z ~ N(2,1)."""
    D = [1] * 8 + [16] * 12 + [64] * 12
    assert _prefill_check(1, 16384, 32, 128, D, 64, 2.0, 10, head_group=8) <= BF16_TOL


def test_config3_long_prefill_full_size():
    """B=1, 16 x 128, T=262144, D=64, W=0, bf16, z ~ N(3,1)."""
    assert _prefill_check(1, 262144, 16, 128, 64, 0, 3.0, 3, head_group=4) <= BF16_TOL


def _planted_inputs(T, H, Dh, Ds, W, n_plant, seed):
    """Inputs on which every sampled boundary row is decided by one key.

    Gate logits are -inf, so every state equals its input (g = 0) and the key
    set alone decides each output.  Every query has q[0] = 16; n_plant
    "planted" positions p carry k[p, 0] = 4 (12 + r) for the r-th of them in
    position order (an integer multiple of 4 below 1024, exact in bf16), all
    other keys and every other channel stay N(0, 1).  A planted key then
    scores ~34 nats above the unplanted ones at the default scale and 5.7
    nats above the previous planted key, so each row's output is essentially
    the value (N(0, 1/4)) of the latest planted key in its key set.  Planted positions
    are spread over the sequence at least W + 2 apart and sit, per a random
    draw, on the grid of every head (p = D_max - 1 mod D_max), on the grid of
    the denser heads only, next to the grid (p = 0 or D - 2 mod D: never a
    key without a window) or anywhere.  Returns (inputs, sampled rows, p)."""
    rng = np.random.default_rng(seed)
    Dset = sorted(set(Ds))
    span = T // n_plant
    assert span >= W + 4 and n_plant <= 244
    plant = []
    for i in range(n_plant):
        lo = i * span + 1
        p = int(rng.integers(lo, lo + span - W - 3))
        D = int(rng.choice(Dset))
        kind = int(rng.integers(0, 4))
        if kind == 0:
            D = Dset[-1]
        if D > 1 and kind < 3:
            base = p - p % D
            p = base + (D - 1 if kind < 2 else int(rng.choice([0, D - 2])))
        plant.append(min(max(p, 0), T - 1))
    plant = sorted(set(plant))
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn((1, T, H, Dh), generator=g, device=DEV)
    k = torch.randn((1, T, H, Dh), generator=g, device=DEV)
    v = 0.5 * torch.randn((1, T, H, Dh), generator=g, device=DEV)   # outputs ~v: bf16 half-ulps below 1e-2
    q[..., 0] = 16.0
    pidx = torch.tensor(plant, device=DEV)
    k[0, pidx, :, 0] = (4.0 * (12 + torch.arange(len(plant), device=DEV, dtype=torch.float32)))[:, None]
    zinf = torch.full((1, T, H, Dh), float("-inf"), device=DEV)
    x = dict(q=q.to(torch.bfloat16), k=k.to(torch.bfloat16), v=v.to(torch.bfloat16), zk=zinf, zv=zinf.clone())
    rows = {0, 1, T - 1}
    for D in Dset:
        rows.update(r for r in (D - 2, D - 1, D) if 0 <= r < T)
    for p in plant:
        rows.update(r for r in (p - 1, p, p + 1, p + W - 1, p + W, p + W + 1) if 0 <= r < T)
    rows.update(int(r) for r in rng.integers(0, T, 64))
    return x, sorted(rows), plant


def _planted_check(T, H, Dh, D, W, n_plant, seed, head_group):
    Ds = D if isinstance(D, list) else [D] * H
    x, rows, plant = _planted_inputs(T, H, Dh, Ds, W, n_plant, seed)
    # the inputs do decide the boundary rows: the oracle's output moves by
    # O(1) from row p - 1 to row p at most planted positions, so a key-set
    # slip of one position at such a row fails the bf16 tolerance
    Kt = oracle.scan(f64(x["k"][:, :, :1]), f64(x["zk"][:, :, :1]))
    Vt = oracle.scan(f64(x["v"][:, :, :1]), f64(x["zv"][:, :, :1]))
    qq = f64(x["q"][:, :, :1])
    # (only planted positions that are keys of head 0 at all: without a
    # window the off-grid ones are decoys that must never enter a key set)
    keyed = [p for p in plant[1:] if p in oracle.key_set(p, Ds[0], W)]
    moved = 0
    for p in keyed:
        o = oracle.prefill(qq, None, None, None, None, [Ds[0]], W, rows=[p - 1, p], states=(Kt, Vt))
        moved += float(np.max(np.abs(o[0, p] - o[0, p - 1]))) > 0.25
    print(f"[full] planted: {len(plant)} keys ({len(keyed)} keyed in head 0), {len(rows)} rows; row p-1 -> p "
          f"moves by > 0.25 at {moved}/{len(keyed)}", flush=True)
    assert len(keyed) >= 0.25 * len(plant) and moved >= 0.8 * len(keyed)
    del Kt, Vt
    return _prefill_check(1, T, H, Dh, D, W, None, seed, head_group, x=x, rows=rows, rms_max=None)


def test_config2_planted_keys_full_size():
    """Index-sensitive check at the T=16384, D=16, W=128 launch shape."""
    assert _planted_check(16384, 16, 128, 16, 128, 100, 21, head_group=16) <= BF16_TOL


def test_config3_planted_keys_full_size():
    """Index-sensitive check at the T=262144, D=64, W=0 launch shape (4096
    grid entries per head, 1024 q-tiles per head)."""
    assert _planted_check(262144, 16, 128, 64, 0, 240, 22, head_group=4) <= BF16_TOL


def test_hybrid_planted_keys_full_size():
    """Index-sensitive check at the hybrid-head shape: 32 heads (8 x D=1,
    12 x 16, 12 x 64; eight-class block order with padding), W=64."""
    D = [1] * 8 + [16] * 12 + [64] * 12
    assert _planted_check(16384, 32, 128, D, 64, 150, 23, head_group=8) <= BF16_TOL


STEPS_CHECKED = [0, 1, 2, 15, 16, 63, 64, 65, 511, 1023]


def _decode_check(B, H, Dh, ctx, dil, W, steps, n_seq, seed):
    R = need_gpu()
    max_pos = ctx + steps
    off, cap, rows = R.rat_grid_layout(H, dil, max_pos)
    print(f"[full] decode B={B} H={H} ctx={ctx}: cache {2 * B * rows * Dh * 2 / 1e9:.1f} GB", flush=True)
    c = inputs.decode_cache(B, H, Dh, dil, W, ctx, steps, seed=seed, device=DEV)
    st = inputs.decode_step_inputs(B, H, Dh, steps, seed=seed + 1, device=DEV)
    rng = np.random.default_rng(seed)
    seqs = sorted(rng.choice(B, n_seq, replace=False).tolist())
    sidx = torch.tensor(seqs, device=DEV)

    # host copies of the sampled sequences' caches, before any step
    def grids(buf):
        return [f64(buf[B * off[h] * Dh: B * (off[h] + cap[h]) * Dh].view(B, cap[h], Dh)[sidx])
                for h in range(H)]
    ref = oracle.DecodeCache(f64(c["state_k"][sidx]), f64(c["state_v"][sidx]), f64(c["ring_k"][sidx]),
                             f64(c["ring_v"][sidx]), grids(c["grid_k"]), grids(c["grid_v"]), dil, W)
    pos = torch.full((B,), ctx, dtype=torch.int32, device=DEV)
    out = torch.empty((B, H, Dh), dtype=torch.bfloat16, device=DEV)
    saved = {}
    print(f"[full]   {steps} GPU steps", flush=True)
    for i in range(steps):
        R.rat_decode_step(st["q"][i], st["k"][i], st["v"][i], st["zk"][i], st["zv"][i], c["state_k"],
                          c["state_v"], c["grid_k"], c["grid_v"], off, cap, c["ring_k"], c["ring_v"], pos,
                          max_pos, dil, W, out=out)
        if i in STEPS_CHECKED:
            saved[i] = out[sidx].clone()
        pos += 1
    torch.cuda.synchronize()
    print("[full]   oracle replay", flush=True)
    worst = 0.0
    for i in range(steps):
        compute = i in STEPS_CHECKED
        want = ref.step(f64(st["q"][i][sidx]), f64(st["k"][i][sidx]), f64(st["v"][i][sidx]),
                        f64(st["zk"][i][sidx]), f64(st["zv"][i][sidx]), [ctx + i] * n_seq, compute=compute)
        if compute:
            worst = max(worst, report(f"decode step {i}", f64(saved[i]), want, rms_max=RMS_TOL))
    # final caches of the sampled sequences
    assert np.max(np.abs(f64(c["state_k"][sidx]) - ref.state_k)) <= 1e-4
    assert np.max(np.abs(f64(c["state_v"][sidx]) - ref.state_v)) <= 1e-4
    assert np.max(np.abs(f64(c["ring_v"][sidx]) - ref.ring_v)) <= 2e-2
    for h in range(H):
        g = grids(c["grid_k"])[h]
        assert np.max(np.abs(g - ref.grid_k[h])) <= 2e-2, h
    return worst


def test_config4_batched_decode_full_size():
    """Batch 256, 16 x 128, context 32768, D=16, W=64, 1024 steps."""
    assert _decode_check(256, 16, 128, 32768, [16] * 16, 64, 1024, 8, 4) <= BF16_TOL


def test_config5_hybrid_decode_full_size():
    """Batch 128, 32 x 128, context 131072, 8 heads D=1, 12 D=16, 12 D=64, W=64."""
    dil = [1] * 8 + [16] * 12 + [64] * 12
    assert _decode_check(128, 32, 128, 131072, dil, 64, 1024, 4, 5) <= BF16_TOL
