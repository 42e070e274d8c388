"""rat_scan on the GPU against the fp64 oracle scan."""
import numpy as np
import pytest
import torch

import oracle
from recurrence_augmented_dilated_amd import inputs
from tests.gpu_util import F32_TOL, f64, need_gpu, report

pytestmark = pytest.mark.gpu


def _run(B, T, H, Dh, dtype, E, mu=2.0, seed=0, h0=True, z_override=None):
    R = need_gpu()
    x = inputs.prefill_inputs(B, T, H, Dh, dtype=dtype, mu=mu, seed=seed)
    xk, zk = x["k"], x["zk"]
    if z_override is not None:
        zk = z_override(zk)
    g = torch.Generator().manual_seed(seed + 100)
    h0t = torch.randn((B, H, Dh), generator=g) if h0 else None
    dev = "cuda:0"
    states, h_last = R.rat_scan(xk.to(dev), zk.to(dev), None if h0t is None else h0t.to(dev),
                                store_every=E, want_h_last=True)
    torch.cuda.synchronize()
    ref = oracle.scan(f64(xk), f64(zk), None if h0t is None else f64(h0t))
    return states, h_last, ref


def _check_states(states, ref, E, dtype, name):
    G = ref.shape[1] // E
    want = ref[:, E - 1::E][:, :G]
    got = f64(states)
    err = report(name, got, want)
    if dtype == torch.float32:
        assert err <= 1e-5, err
    else:
        # one bf16 rounding of the fp32 state: half an ulp plus fp32 noise
        lim = np.abs(want) * 2.0 ** -8 + 1e-6
        assert np.all(np.abs(got - want) <= lim), err


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("H,Dh", [(1, 64), (2, 64), (2, 128), (4, 128)])
@pytest.mark.parametrize("E", [1, 4, 7])
def test_scan_shapes(dtype, H, Dh, E):
    B, T = 2, 300   # ragged: 300 = 4 chunks of 64 + 44
    states, h_last, ref = _run(B, T, H, Dh, dtype, E, seed=H * 10 + E)
    _check_states(states, ref, E, dtype, f"scan {dtype} H={H} Dh={Dh} E={E}")
    assert np.max(np.abs(f64(h_last) - ref[:, -1])) <= 1e-5


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_scan_long_lookback(dtype):
    """Thousands of chunks: the carry crosses many look-back hops."""
    R = need_gpu()
    B, T, H, Dh = 1, 40000, 2, 128
    states, h_last, ref = _run(B, T, H, Dh, dtype, 1, mu=4.0, seed=3)
    _check_states(states, ref, 1, dtype, f"scan long {dtype}")
    assert np.max(np.abs(f64(h_last) - ref[:, -1])) <= 1e-5
    ws = R.workspace(0, "cuda:0", "scan")
    assert R.workspace_error(ws) == 0


def test_scan_extreme_gates():
    """Gate logits of +-inf: g = 1 holds the state, g = 0 copies the input."""
    def poke(z):
        z = z.clone()
        z[:, ::5] = float("inf")
        z[:, 1::7] = float("-inf")
        z[:, 2::11] = 40.0
        z[:, 3::13] = -40.0
        return z
    states, h_last, ref = _run(1, 500, 2, 64, torch.float32, 1, seed=5, z_override=poke)
    _check_states(states, ref, 1, torch.float32, "scan extreme gates")


def test_scan_long_memory_carries_across_chunks():
    """g ~ 1 everywhere: the initial state survives thousands of steps, so a
    wrong carry anywhere in the chain shows (as an O(0.1) error).

    Tolerance: with a constant logit the fp32 gate g differs from the exact
    sigmoid by a fixed ~1 ulp (6e-8 relative), so after n = 9000 steps the
    fp32 product of gates drifts by up to n * 6e-8 ~ 5.4e-4 relative from the
    fp64 one; |h0| * g^n is ~0.3 here, so errors near 2e-4 are inherent to
    fp32 state and the check allows 1e-3."""
    def slow(z):
        return torch.full_like(z, 9.0)
    states, h_last, ref = _run(1, 9000, 2, 64, torch.float32, 1, seed=6, z_override=slow)
    err = report("scan slow decay", f64(states), ref)
    assert err <= 1e-3


def test_scan_deterministic():
    R = need_gpu()
    x = inputs.prefill_inputs(1, 5000, 4, 128, dtype=torch.bfloat16, seed=9, device="cuda:0")
    a, _ = R.rat_scan(x["k"], x["zk"])
    b, _ = R.rat_scan(x["k"], x["zk"])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_scan_empty_and_tiny():
    R = need_gpu()
    x = torch.zeros((1, 0, 2, 64), device="cuda:0")
    s, _ = R.rat_scan(x, x.clone())
    assert s.shape[1] == 0
    states, h_last, ref = _run(1, 1, 2, 64, torch.float32, 1, seed=7)
    _check_states(states, ref, 1, torch.float32, "scan T=1")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_scan_lookback_recompute_path(dtype, monkeypatch):
    """Force the look-back's fallback (a block that sees no published
    predecessor folds that chunk in from its inputs) on every wait."""
    monkeypatch.setenv("RAT_SCAN_FALLBACK_SPINS", "0")
    states, h_last, ref = _run(2, 3000, 2, 128, dtype, 1, seed=41)
    _check_states(states, ref, 1, dtype, f"scan fallback {dtype}")
    assert np.max(np.abs(f64(h_last) - ref[:, -1])) <= 1e-5


@pytest.mark.parametrize("dil,W", [(16, 32), (16, 0), ([1, 3, 32, 33], 0), ([2, 16, 1, 64], 8)],
                         ids=["D16-W32", "D16-W0", "mixed-W0", "mixed-W8"])
def test_prefill_with_lookback_recompute_path(dil, W, monkeypatch):
    """The recompute fallback on every wait, with the grid layouts the scan
    writes from its LDS staging (dense heads, 2 <= D <= 32) and directly
    (D > 32), with and without a window."""
    R = need_gpu()
    monkeypatch.setenv("RAT_SCAN_FALLBACK_SPINS", "0")
    H = len(dil) if isinstance(dil, list) else 2
    x = inputs.prefill_inputs(1, 2000, H, 128, dtype=torch.bfloat16, seed=42)
    d = {k: v.to("cuda:0") for k, v in x.items()}
    out = R.rat_dilated_prefill(d["q"], d["k"], d["v"], d["zk"], d["zv"], dil, W)
    torch.cuda.synchronize()
    ref = oracle.prefill(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["zk"]), f64(x["zv"]), dil, W)
    assert report(f"prefill fallback D={dil} W={W}", f64(out), ref) <= 2e-2
