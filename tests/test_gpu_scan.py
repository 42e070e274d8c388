"""rat_scan on the GPU against the fp64 oracle scan."""
import numpy as np
import pytest
import torch

import oracle
from recurrence_augmented_dilated_amd import inputs
from tests.gpu_util import F32_TOL, f64, need_gpu, report

pytestmark = pytest.mark.gpu


def _run(B, T, H, Dh, dtype, E, mu=2.0, seed=0, h0=True, z_override=None, polls=None, want_inputs=False):
    R = need_gpu()
    x = inputs.prefill_inputs(B, T, H, Dh, dtype=dtype, mu=mu, seed=seed)
    xk, zk = x["k"], x["zk"]
    if z_override is not None:
        zk = z_override(zk)
    g = torch.Generator().manual_seed(seed + 100)
    h0t = torch.randn((B, H, Dh), generator=g) if h0 else None
    dev = "cuda:0"
    ws = None
    if polls is not None:
        # a workspace of its own whose header caps the look-back polls
        ws = torch.zeros(R.rat_scan_workspace_size(B, T, H, Dh), dtype=torch.uint8, device=dev)
        R.workspace_set_poll_limit(ws, polls)
    states, h_last = R.rat_scan(xk.to(dev), zk.to(dev), None if h0t is None else h0t.to(dev),
                                store_every=E, want_h_last=True, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.scan(f64(xk), f64(zk), None if h0t is None else f64(h0t))
    if want_inputs:
        return states, h_last, ref, (f64(xk), f64(zk), None if h0t is None else f64(h0t))
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
@pytest.mark.parametrize("H,Dh", [(1, 64), (3, 64), (2, 128)])
@pytest.mark.parametrize("E", [16, 37, 64])
def test_scan_grid_only_shapes(dtype, H, Dh, E):
    """Grid states only, every E >= 16 (the persistent grid-only scan): at
    most one stored state per 16 steps, taken from a partial aggregate;
    ragged T, an initial state and the final state."""
    B, T = 2, 1000
    states, h_last, ref = _run(B, T, H, Dh, dtype, E, seed=H * 100 + E)
    _check_states(states, ref, E, dtype, f"grid-only scan {dtype} H={H} Dh={Dh} E={E}")
    assert np.max(np.abs(f64(h_last) - ref[:, -1])) <= 1e-5


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_scan_grid_only_long(dtype):
    """Thousands of chunks per slab on persistent blocks (several items per
    block), grid states every 64 steps."""
    B, T, H, Dh = 1, 70000, 4, 128
    states, h_last, ref = _run(B, T, H, Dh, dtype, 64, mu=4.0, seed=12)
    _check_states(states, ref, 64, dtype, f"grid-only scan long {dtype}")
    assert np.max(np.abs(f64(h_last) - ref[:, -1])) <= 1e-5


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_scan_grid_only_recompute_path(dtype):
    """The grid-only scan with the look-back's local recompute on every wait."""
    states, h_last, ref = _run(2, 5000, 2, 128, dtype, 32, seed=43, polls=0)
    _check_states(states, ref, 32, dtype, f"grid-only scan fallback {dtype}")
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


def _fp32_recurrence_bound(x, z, h0, ref):
    """Per-element bound on |fp32 scan - exact scan| for one carry chain.

    One fused fp32 step h_t = g h_{t-1} + (1 - g) x_t is off by at most half
    an ulp of g (2^-25 absolute for g in [1/2, 1)) times |h_{t-1}|, plus the
    roundings of (1 - g) x_t and of the result (2^-24 relative each), plus a
    few ulps of the complement 1 - g (from exp2 and a reciprocal): 1.5 u |h|
    + ~4 u (1 - g) |x| with u = 2^-24.  The chunked scan carries a state
    across chunks as A h + B, where A is a product of the chunk's gates: one
    more rounding per step in A, and the unfused multiply-add of the carry,
    so k_h = 4 and k_x = 8 here.  An earlier error decays with the same gate:
        E_t = g_t E_{t-1} + u (k_h |h_{t-1}| + k_x (1 - g_t) |x_t|),
    which for a constant gate and x ~ 0 is the k_h u t g^t |h0| growth of a
    decayed initial state (a relative error of at most k_h u t)."""
    u = 2.0 ** -24
    g, c = oracle.gates(z)
    B, T, H, Dh = x.shape
    E = np.zeros((B, T, H, Dh))
    e = np.zeros((B, H, Dh))
    prev = np.zeros((B, H, Dh)) if h0 is None else np.abs(h0)
    for t in range(T):
        e = g[:, t] * e + u * (4.0 * prev + 8.0 * c[:, t] * np.abs(x[:, t]))
        E[:, t] = e
        prev = np.abs(ref[:, t])
    return E


def test_scan_long_memory_carries_across_chunks():
    """g ~ 1 everywhere: the initial state survives thousands of steps, so a
    wrong carry anywhere in the chain shows.  With a constant logit the fp32
    gate is off by a fixed fraction of an ulp, which compounds over the
    steps; every element is held to the bound that this rounding allows
    (_fp32_recurrence_bound), not to a blanket tolerance."""
    def slow(z):
        return torch.full_like(z, 9.0)
    states, h_last, ref, (x, z, h0) = _run(1, 9000, 2, 64, torch.float32, 1, seed=6, z_override=slow,
                                           want_inputs=True)
    got = f64(states)
    report("scan slow decay", got, ref)
    bound = _fp32_recurrence_bound(x, z, h0, ref)
    excess = np.abs(got - ref) - bound
    i = np.unravel_index(np.argmax(excess), excess.shape)
    print(f"[parity] scan slow decay: worst err/bound = {np.max(np.abs(got - ref) / (bound + 1e-30)):.3f} "
          f"(bound there {bound[i]:.3e})", flush=True)
    assert np.all(excess <= 0), (i, float(np.abs(got - ref)[i]), float(bound[i]))
    # the bound stays far below what a wrong carry would do: one chunk of
    # decay too many or too few (g^128 ~ 0.984) moves h by 1.6e-2 |h|
    big = np.abs(ref) >= 1e-2
    assert float(np.max(bound[big] / np.abs(ref[big]))) < 5e-3


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
def test_scan_lookback_recompute_path(dtype):
    """Force the look-back's fallback (a block that sees no published
    predecessor folds that chunk in from its inputs) on every wait, through
    the workspace header's poll limit."""
    states, h_last, ref = _run(2, 3000, 2, 128, dtype, 1, seed=41, polls=0)
    _check_states(states, ref, 1, dtype, f"scan fallback {dtype}")
    assert np.max(np.abs(f64(h_last) - ref[:, -1])) <= 1e-5


@pytest.mark.parametrize("dil,W", [(16, 32), (16, 0), ([1, 3, 32, 33], 0), ([2, 16, 1, 64], 8),
                                   ([16, 33, 64, 100], 0)],
                         ids=["D16-W32", "D16-W0", "mixed-W0", "mixed-W8", "grid-only-W0"])
def test_prefill_with_lookback_recompute_path(dil, W):
    """The recompute fallback on every wait, with the grid layouts the scan
    writes from its LDS staging (dense heads, 2 <= D <= 32) and directly
    (D > 32), with and without a window."""
    R = need_gpu()
    H = len(dil) if isinstance(dil, list) else 2
    x = inputs.prefill_inputs(1, 2000, H, 128, dtype=torch.bfloat16, seed=42)
    d = {k: v.to("cuda:0") for k, v in x.items()}
    ws = torch.zeros(R.rat_dilated_prefill_workspace_size(1, 2000, H, 128, dil, W), dtype=torch.uint8,
                     device="cuda:0")
    R.workspace_set_poll_limit(ws, 0)
    out = R.rat_dilated_prefill(d["q"], d["k"], d["v"], d["zk"], d["zv"], dil, W, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.prefill(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["zk"]), f64(x["zv"]), dil, W)
    assert report(f"prefill fallback D={dil} W={W}", f64(out), ref) <= 2e-2
