"""bf16 prefill without a local window on launches with more q-tiles than
compute units, so that every persistent attention block walks several
q-tiles (256 query rows each) in turn: the next q-tile's Q rows and first
key tiles load while the current one finishes, the output rows go out one
step late, q-tiles without any key get zero rows on the way, and the blocks'
q-tile lists are dealt per XCD in alternating directions.  Against the fp64
oracle on sampled rows: one row of every wave (32 rows) of every q-tile
("RAT+: Train Dense, Infer Sparse", abstract and Fig. 1c: the dilated key
set)."""
import numpy as np
import pytest
import torch

import oracle
from recurrence_augmented_dilated_amd import inputs
from tests.gpu_util import BF16_TOL, RMS_TOL, f64, need_gpu, report
from tests.test_gpu_full_configs import _planted_check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _wave_rows(T, seed):
    """One seeded row in every 32-row wave slice of the sequence."""
    rng = np.random.default_rng(seed)
    rows = [w + int(rng.integers(0, 32)) for w in range(0, T, 32)]
    return sorted({min(r, T - 1) for r in rows} | {0, T - 1})


@pytest.mark.parametrize("B,H,Dh,T,dil", [
    # 512 q-tiles: two per block, one from each dealing direction
    (1, 8, 128, 16384, [16] * 8),
    # keyless q-tiles (D above a q-tile's reach, D above T) and one-tile
    # q-tiles between full ones; a dense head
    (2, 8, 128, 8192, [16, 300, 700, 5000, 9000, 64, 1, 3000]),
    # 15 (b, h) pairs, not a multiple of 8 (no XCD pinning); head size 64;
    # three rounds of q-tiles per block
    (3, 5, 64, 9000, [1, 17, 256, 4096, 9001]),
], ids=["two-rounds", "keyless-mix", "odd-pairs-dh64"])
def test_grid_only_qtile_stream(B, H, Dh, T, dil):
    R = need_gpu()
    print(f"[stream] B={B} H={H} Dh={Dh} T={T} D={dil}", flush=True)
    x = inputs.prefill_inputs(B, T, H, Dh, dtype=torch.bfloat16, seed=31 + T)
    d = {k: v.to(DEV) for k, v in x.items()}
    out = R.rat_dilated_prefill(d["q"], d["k"], d["v"], d["zk"], d["zv"], dil, 0)
    torch.cuda.synchronize()
    rows = _wave_rows(T, seed=T)
    ref = oracle.prefill(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["zk"]), f64(x["zv"]), dil, 0, rows=rows)
    err = report(f"stream B={B} H={H} T={T}", f64(out)[:, rows], ref[:, rows], rms_max=RMS_TOL)
    assert err <= BF16_TOL
    # rows whose key set is empty are exactly zero
    empty = [t for t in rows if any(len(oracle.key_set(t, D, 0)) == 0 for D in dil)]
    for t in empty:
        for h, D in enumerate(dil):
            if len(oracle.key_set(t, D, 0)) == 0:
                assert torch.count_nonzero(out[:, t, h]).item() == 0, (t, h)


@pytest.mark.parametrize("Dh,seed", [(128, 23), (64, 24)])
def test_grid_only_qtile_stream_planted_keys(Dh, seed):
    """Index-sensitive check at a many-q-tile grid-only shape with mixed
    dilations (1024 q-tiles: four per block), both head sizes."""
    assert _planted_check(16384, 16, Dh, [16] * 8 + [64] * 4 + [4] * 4, 0, 100, seed, head_group=16) <= BF16_TOL


def test_grid_only_chunk_at_offset():
    """rat_prefill_chunk without a window: a 4096-row chunk, then an
    8192-row chunk at position 4096 (16 heads: 512 q-tiles, two per block,
    key positions offset from the query rows) against the oracle's prefill
    of the whole sequence on sampled rows of the second chunk."""
    R = need_gpu()
    B, H, Dh = 1, 16, 128
    dil = [16] * 8 + [64] * 4 + [4] * 4
    chunks = [4096, 8192]
    L = sum(chunks)
    x = inputs.prefill_inputs(B, L, H, Dh, dtype=torch.bfloat16, seed=77)
    max_pos = L + 64
    off, cap, nrows = R.rat_grid_layout(H, dil, max_pos)
    grid_k = torch.zeros(B * nrows * Dh, dtype=torch.bfloat16, device=DEV)
    grid_v = torch.zeros(B * nrows * Dh, dtype=torch.bfloat16, device=DEV)
    state_k = torch.zeros((B, H, Dh), dtype=torch.float32, device=DEV)
    state_v = torch.zeros((B, H, Dh), dtype=torch.float32, device=DEV)
    p0 = 0
    outs = []
    for T in chunks:
        d = {n: t[:, p0:p0 + T].contiguous().to(DEV) for n, t in x.items()}
        outs.append(R.rat_prefill_chunk(d["q"], d["k"], d["v"], d["zk"], d["zv"], state_k, state_v, grid_k, grid_v,
                                        off, cap, None, None, p0, max_pos, dil, 0))
        p0 += T
    torch.cuda.synchronize()
    rows = _wave_rows(chunks[1], seed=5)
    ref = oracle.prefill(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["zk"]), f64(x["zv"]), dil, 0,
                         rows=[chunks[0] + r for r in rows])
    err = report("chunk p0=4096", f64(outs[1])[:, rows], ref[:, [chunks[0] + r for r in rows]], rms_max=RMS_TOL)
    assert err <= BF16_TOL
