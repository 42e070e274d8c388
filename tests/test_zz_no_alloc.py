"""rat_decode_step_noalloc (the decode step with the library's built-in
scratch instead of a workspace) against rat_decode_step on identical cache
copies: two steps on a batch with split-K partials, then a smaller batch
right after it (the scratch keeps the last call's contents), outputs and
every cache buffer bit for bit; and the size limit, checked on the host."""
import ctypes

import pytest
import torch

from recurrence_augmented_dilated_amd import inputs

DEV = "cuda:0"


def _case(R, B, H, Dh, dil, W, pos0, seed):
    max_pos = max(pos0) + 4
    off, cap, rows = R.rat_grid_layout(H, dil, max_pos)
    c = inputs.decode_cache(B, H, Dh, dil, W, context=0, steps=0, seed=seed)
    g = torch.Generator().manual_seed(seed)
    c["grid_k"] = torch.randn(B * rows * Dh, generator=g).to(torch.bfloat16)
    c["grid_v"] = torch.randn(B * rows * Dh, generator=g).to(torch.bfloat16)
    names = ("state_k", "state_v", "grid_k", "grid_v", "ring_k", "ring_v")
    a = {n: c[n].to(DEV) for n in names}
    b = {n: t.clone() for n, t in a.items()}
    st = inputs.decode_step_inputs(B, H, Dh, 2, seed=seed + 1, device=DEV)
    return max_pos, off, cap, a, b, st, names


def _compare(R, B, H, Dh, dil, W, pos0, seed):
    max_pos, off, cap, a, b, st, names = _case(R, B, H, Dh, dil, W, pos0, seed)
    n_items_split = R.rat_decode_workspace_size(B, H, Dh, dil, W, max_pos)
    print(f"[noalloc] B={B} H={H} D={dil} W={W} pos0={pos0}: workspace {n_items_split} bytes", flush=True)
    pos = torch.tensor(pos0, dtype=torch.int32, device=DEV)
    for i in range(2):
        args = (st["q"][i], st["k"][i], st["v"][i], st["zk"][i], st["zv"][i])
        o_ws = R.rat_decode_step(*args, a["state_k"], a["state_v"], a["grid_k"], a["grid_v"], off, cap,
                                 a["ring_k"], a["ring_v"], pos, max_pos, dil, W)
        o_na = R.rat_decode_step_noalloc(*args, b["state_k"], b["state_v"], b["grid_k"], b["grid_v"], off, cap,
                                         b["ring_k"], b["ring_v"], pos, max_pos, dil, W)
        torch.cuda.synchronize()
        assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16)), (B, i)
        pos += 1
    for n in names:
        assert torch.equal(a[n].view(torch.uint8), b[n].view(torch.uint8)), n
    return n_items_split


@pytest.mark.gpu
def test_decode_noalloc_matches_workspace_entry():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import recurrence_augmented_dilated_amd as R
    R.lib()
    # long dense heads with a small batch: several splits per (b, h), so the
    # partials in the scratch and the combine kernel are in use
    big = _compare(R, 6, 4, 128, [1, 4, 16, 64], 16, [5000, 4100, 4500, 3999, 4096, 4800], seed=3)
    # then a smaller call on the same scratch
    small = _compare(R, 2, 3, 64, [1, 2, 5], 8, [700, 1500], seed=4)
    assert small < big <= R.DECODE_SCRATCH_BYTES


def test_decode_noalloc_rejects_steps_beyond_its_scratch():
    """Host-side validation: a step whose workspace exceeds the built-in
    scratch returns RAT_ERR_WORKSPACE before any HIP call (no GPU needed:
    the pointers are placeholders that nothing dereferences)."""
    import recurrence_augmented_dilated_amd as R
    L = R.lib()
    B, H, Dh, W = 128, 32, 128, 64
    dil = [1] * 8 + [16] * 12 + [64] * 12
    max_pos = 1 << 24
    need = R.rat_decode_workspace_size(B, H, Dh, dil, W, max_pos)
    assert need > R.DECODE_SCRATCH_BYTES
    off, cap, _ = R.rat_grid_layout(H, dil, max_pos)
    p = ctypes.c_void_p(1 << 20)
    offs = (ctypes.c_int64 * H)(*off)
    caps = (ctypes.c_int32 * H)(*cap)
    dl = (ctypes.c_int32 * H)(*dil)
    st = L.rat_decode_step_noalloc(p, p, p, p, p, p, p, p, p, offs, caps, p, p, p, max_pos, p, B, H, Dh, dl, W,
                                   -1.0, 1, None)
    assert st == -3, st   # RAT_ERR_WORKSPACE
    assert b"scratch" in L.rat_last_error()
