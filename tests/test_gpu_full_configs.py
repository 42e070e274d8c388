"""Parity at the benchmark workloads' full sizes, in the launch configuration
the benchmark times, on sampled outputs that the fp64 oracle computes one by
one.  Inputs are generated on the GPU with torch's seeded generator and
copied to the host for the oracle; nothing the oracle sees comes from librat.

Samples: prefill rows at the start (t < 2D), around grid boundaries in eight
regions, the last 256 rows and seeded random rows, every head; decode: 8 or 4
sequences, all heads, the outputs at steps {0, 1, 2, 15, 16, 63, 64, 65, 511,
1023} and the final recurrent states, ring and grid rows.
"""
import numpy as np
import pytest
import torch

import oracle
from recurrence_augmented_dilated_amd import inputs
from tests.gpu_util import BF16_TOL, f64, need_gpu, report

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


def _prefill_check(B, T, H, Dh, D, W, mu, seed, head_group):
    R = need_gpu()
    print(f"[full] prefill B={B} T={T} H={H} D={D} W={W}: generating inputs", flush=True)
    x = inputs.prefill_inputs(B, T, H, Dh, dtype=torch.bfloat16, mu=mu, seed=seed, device=DEV)
    out = R.rat_dilated_prefill(x["q"], x["k"], x["v"], x["zk"], x["zv"], D, W)
    torch.cuda.synchronize()
    Ds = D if isinstance(D, list) else [D] * H
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
        worst = max(worst, report(f"prefill T={T} heads {h0}+", got[:, :, hs], ref[:, rows]))
        del Kt, Vt, q, ref
    return worst


def test_config2_prefill_full_size():
    """B=1, 16 x 128, T=16384, D=16, W=128, bf16, z ~ N(2,1)."""
    assert _prefill_check(1, 16384, 16, 128, 16, 128, 2.0, 2, head_group=16) <= BF16_TOL


def test_hybrid_head_prefill_full_size():
    """B=1, 32 x 128, T=16384, W=64, per-head dilation 8 x D=1, 12 x 16,
    12 x 64 (the hybrid-head mix), bf16, z ~ N(2,1)."""
    D = [1] * 8 + [16] * 12 + [64] * 12
    assert _prefill_check(1, 16384, 32, 128, D, 64, 2.0, 10, head_group=8) <= BF16_TOL


def test_config3_long_prefill_full_size():
    """B=1, 16 x 128, T=262144, D=64, W=0, bf16, z ~ N(3,1)."""
    assert _prefill_check(1, 262144, 16, 128, 64, 0, 3.0, 3, head_group=4) <= BF16_TOL


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
            worst = max(worst, report(f"decode step {i}", f64(saved[i]), want))
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
