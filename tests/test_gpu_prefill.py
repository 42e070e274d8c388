"""rat_dilated_prefill on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from recurrence_augmented_dilated_amd import inputs
from tests.gpu_util import BF16_TOL, F32_TOL, RMS_TOL, f64, need_gpu, report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _ref(x, dil, W, scale=None, rows=None):
    return oracle.prefill(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["zk"]), f64(x["zv"]),
                          dil, W, scale=scale, rows=rows)


def _gpu(x, dil, W, scale=None):
    R = need_gpu()
    d = {k: v.to(DEV) for k, v in x.items()}
    out = R.rat_dilated_prefill(d["q"], d["k"], d["v"], d["zk"], d["zv"], dil, W, scale=scale)
    torch.cuda.synchronize()
    return out


def test_config1_tiny_fp32():
    """B=1, 2 heads x 64, T=1024, D=4, W=0, fp32, z ~ N(2,1): full output."""
    x = inputs.prefill_inputs(1, 1024, 2, 64, dtype=torch.float32, mu=2.0, seed=1)
    out = _gpu(x, 4, 0)
    err = report("config1 fp32", f64(out), _ref(x, 4, 0))
    assert err <= F32_TOL


@pytest.mark.parametrize("D,W", [(1, 0), (3, 0), (16, 0), (64, 0), (5, 3), (16, 128), (1, 7), (700, 0), (4, 1000)])
def test_bf16_small(D, W):
    """Ragged T (several q-tiles and key tiles plus a tail), 2 heads x 128."""
    x = inputs.prefill_inputs(1, 700, 2, 128, dtype=torch.bfloat16, seed=D * 31 + W)
    out = _gpu(x, D, W)
    err = report(f"bf16 D={D} W={W}", f64(out), _ref(x, D, W))
    assert err <= BF16_TOL


@pytest.mark.parametrize("D,W", [(2, 0), (8, 4), (1, 0), (16, 0), (40, 0)])
def test_fp32_small(D, W):
    x = inputs.prefill_inputs(2, 333, 2, 128, dtype=torch.float32, seed=D * 7 + W)
    out = _gpu(x, D, W)
    err = report(f"fp32 D={D} W={W}", f64(out), _ref(x, D, W))
    assert err <= F32_TOL


@pytest.mark.parametrize("Dh", [64, 128])
def test_fp32_64query_blocks(Dh):
    """fp32 with at least as many 64-query blocks as compute units (2 x 8
    heads x 18 q-tiles = 288), so the exact-fp32 kernel runs with 64-query
    blocks (smaller launches use 16-query blocks); ragged T, a window."""
    x = inputs.prefill_inputs(2, 1100, 8, Dh, dtype=torch.float32, seed=40 + Dh)
    out = _gpu(x, 4, 16)
    err = report(f"fp32 64-query blocks Dh={Dh}", f64(out), _ref(x, 4, 16))
    assert err <= F32_TOL


def test_bf16_dh64_batch():
    x = inputs.prefill_inputs(3, 257, 4, 64, dtype=torch.bfloat16, seed=11)
    out = _gpu(x, 4, 16)
    err = report("bf16 Dh=64 B=3", f64(out), _ref(x, 4, 16))
    assert err <= BF16_TOL


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("T", [64, 3000])
def test_segmented_scan_prefill(dtype, T):
    """No window and every D >= 16: the recurrence runs as the segmented
    scan (grid states from per-segment (A, B) pairs).  Per-head D (16, 17,
    64, 100, 1000), Dh = 64 (64-channel slabs), B = 2, ragged T."""
    dil = [16, 17, 64, 100, 1000]
    x = inputs.prefill_inputs(2, T, 5, 64, dtype=dtype, seed=T + 5)
    out = _gpu(x, dil, 0)
    err = report(f"segmented scan {dtype} T={T}", f64(out), _ref(x, dil, 0))
    assert err <= (F32_TOL if dtype == torch.float32 else BF16_TOL)


@pytest.mark.parametrize("B,H,dtype,mu", [(1, 16, torch.bfloat16, 2.0), (1, 16, torch.bfloat16, 9.0),
                                           (2, 8, torch.bfloat16, 9.0), (2, 8, torch.float32, 9.0)],
                         ids=["bf16-mu2", "bf16-slow-decay", "bf16-B2-slow-decay", "f32-B2-slow-decay"])
def test_segmented_scan_multichunk_segments(B, H, dtype, mu):
    """The segmented scan with 32 slabs of 128 channels (B x H = 16 heads of
    128, keys and values): on 256 compute units each slab gets 8 segments, so
    T = 6221 (25 chunks of 256 steps, the last one partial) gives segments of
    4 chunks and a last segment of one.  With mean logit 9 (g ~ 0.9999) the
    carry across every segment boundary moves the grid states; D = 16 and 64
    heads mixed."""
    dil = [16, 64] * (H // 2)
    x = inputs.prefill_inputs(B, 6221, H, 128, dtype=dtype, seed=77 + B, mu=mu)
    out = _gpu(x, dil, 0)
    ref = _ref(x, dil, 0)
    if dtype == torch.float32:
        err = report(f"segmented scan multi-chunk f32 B={B} mu={mu}", f64(out), ref)
        assert err <= F32_TOL
    else:
        # rel_rms bound too: with mu = 9 the outputs are ~0.04, below any
        # meaningful max-abs tolerance
        err = report(f"segmented scan multi-chunk B={B} mu={mu}", f64(out), ref, rms_max=RMS_TOL)
        assert err <= BF16_TOL


def test_per_head_dilation():
    """Hybrid heads: D = 1, 16, 64, 3 on one call equals the oracle head by head."""
    dil = [1, 16, 64, 3]
    x = inputs.prefill_inputs(2, 400, 4, 128, dtype=torch.bfloat16, seed=12)
    out = _gpu(x, dil, 8)
    err = report("per-head D", f64(out), _ref(x, dil, 8))
    assert err <= BF16_TOL


@pytest.mark.parametrize("W", [12, 0])
def test_many_dilation_classes(W):
    """24 heads over 13 distinct dilations: the launch orders blocks by class
    (at most 8 classes, the last one merges the sparsest), pads classes to 8
    blocks and keeps the 16 dense (b, h) pairs XCD-pinned.  With a window the
    dense heads read their grid from the all-state arrays; without one the
    scan writes their transposed grid through LDS, next to a sparser head in
    the same 128-channel slab (Dh = 64)."""
    dil = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 1, 1, 16, 2, 64, 3, 1, 5, 9, 700, 1, 1, 1, 1]
    x = inputs.prefill_inputs(2, 600, 24, 64, dtype=torch.bfloat16, seed=31 + W)
    out = _gpu(x, dil, W)
    err = report(f"13 dilation classes W={W}", f64(out), _ref(x, dil, W))
    assert err <= BF16_TOL


def _onehot_inputs(T, H, Dh, dtype, hot, seed):
    """Gates closed (z = -inf: states equal raw k, v) and one key per head made
    dominant: queries that see position `hot` return v[hot] almost exactly,
    others do not.  Exposes any off-by-one in the key-set boundaries."""
    x = inputs.prefill_inputs(1, T, H, Dh, dtype=torch.float32, seed=seed)
    x["zk"].fill_(float("-inf"))
    x["zv"].fill_(float("-inf"))
    x["q"] = x["q"] / 8
    x["q"][..., 0] += 2.0          # every query shares a direction e0 ...
    x["k"] = x["k"] / 8
    x["k"][:, hot] = 0.0
    x["k"][:, hot, :, 0] = 60.0    # ... that only the hot key carries
    x["v"][:, hot] = 10.0
    for key in ("q", "k", "v"):
        x[key] = x[key].to(dtype)
    return x


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("D,W,hot", [(4, 0, 63), (4, 0, 64), (4, 0, 67), (16, 8, 47), (16, 8, 95),
                                     (16, 8, 96), (3, 5, 100), (8, 0, 7), (1, 0, 128), (1, 8, 100),
                                     (1, 8, 200), (1, 70, 130), (16, 0, 47), (16, 0, 48), (64, 0, 127),
                                     (64, 0, 191)])
def test_key_set_boundaries_onehot(dtype, D, W, hot):
    T, H, Dh = 256, 2, 128
    x = _onehot_inputs(T, H, Dh, dtype, hot, seed=hot)
    out = _gpu(x, D, W)
    ref = _ref(x, D, W)
    err = report(f"onehot {dtype} D={D} W={W} hot={hot}", f64(out), ref)
    tol = F32_TOL if dtype == torch.float32 else BF16_TOL * 5   # outputs here reach 10
    assert err <= tol
    # the rows that see the hot key are ~10, the rows that do not are small
    sees = [t for t in range(T) if hot in set(oracle.key_set(t, D, W).tolist())]
    blind = [t for t in range(T) if t not in set(sees)]
    assert np.all(f64(out)[0, sees, :, 0] > 5.0)
    assert np.all(np.abs(f64(out)[0, blind, :, 0]) < 5.0)


def test_sharpened_scores():
    """Scale x8 makes the softmax peaky, so masks and tile merges matter."""
    x = inputs.prefill_inputs(1, 600, 2, 128, dtype=torch.float32, seed=21)
    s = 8.0 / np.sqrt(128)
    out = _gpu(x, 16, 32, scale=s)
    err = report("sharp fp32", f64(out), _ref(x, 16, 32, scale=s))
    assert err <= F32_TOL


def test_prefill_deterministic_and_stage_split():
    R = need_gpu()
    x = inputs.prefill_inputs(1, 2048, 4, 128, dtype=torch.bfloat16, seed=22, device=DEV)
    a = R.rat_dilated_prefill(x["q"], x["k"], x["v"], x["zk"], x["zv"], 16, 64)
    b = R.rat_dilated_prefill(x["q"], x["k"], x["v"], x["zk"], x["zv"], 16, 64)
    c = torch.empty_like(a)
    R.rat_dilated_prefill_stage(1, x["q"], x["k"], x["v"], x["zk"], x["zv"], 16, 64)
    R.rat_dilated_prefill_stage(2, x["q"], x["k"], x["v"], x["zk"], x["zv"], 16, 64, out=c)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_empty_rows_are_zero():
    """D = T, W = 0: only the last row has a key."""
    x = inputs.prefill_inputs(1, 300, 2, 128, dtype=torch.bfloat16, seed=23)
    out = f64(_gpu(x, 300, 0))
    assert np.all(out[:, :299] == 0.0)
    ref = _ref(x, 300, 0, rows=[299])
    assert report("D=T last row", out[:, 299], ref[:, 299]) <= BF16_TOL


def test_t_zero_and_one():
    R = need_gpu()
    z = torch.zeros((1, 0, 2, 128), dtype=torch.bfloat16, device=DEV)
    zf = torch.zeros((1, 0, 2, 128), dtype=torch.float32, device=DEV)
    o = R.rat_dilated_prefill(z, z, z, zf, zf, 4, 0)
    assert o.shape[1] == 0
    x = inputs.prefill_inputs(1, 1, 2, 128, dtype=torch.bfloat16, seed=24)
    for D, W in [(1, 0), (2, 0), (1, 1)]:
        out = _gpu(x, D, W)
        assert report(f"T=1 D={D} W={W}", f64(out), _ref(x, D, W)) <= BF16_TOL
