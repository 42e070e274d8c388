"""Python binding of librat, the RAT+ temporal-mixing operator on MI355X.

A thin ctypes layer over the C ABI in include/rat.h: it checks tensor
devices, dtypes and contiguity, allocates outputs and zero-initialised
workspaces with torch, and passes raw pointers and torch's current HIP
stream.  Every step of the operator runs in librat's HIP kernels; there is no
CPU or PyTorch fallback.  If librat.so is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

__all__ = [
    "RatError", "lib", "rat_scan", "rat_scan_workspace_size", "rat_dilated_prefill",
    "rat_dilated_prefill_stage",
    "rat_dilated_prefill_workspace_size", "rat_grid_layout", "rat_decode_step",
    "rat_decode_workspace_size", "rat_decode_step_noalloc", "DECODE_SCRATCH_BYTES", "workspace",
    "workspace_error", "workspace_set_poll_limit", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librat.so")

RAT_F32, RAT_BF16 = 0, 1
_STATUS = {0: "RAT_OK", -1: "RAT_ERR_INVALID_ARG", -2: "RAT_ERR_UNSUPPORTED",
           -3: "RAT_ERR_WORKSPACE", -4: "RAT_ERR_HIP"}

_lib = None
_lock = threading.Lock()


class RatError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status


def lib():
    """The loaded librat (ctypes.CDLL).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"librat.so not found at {LIB_PATH}: build it with "
                    "`python -m recurrence_augmented_dilated_amd.build_lib`")
            L = ctypes.CDLL(LIB_PATH)
            c_int, c_i64, c_sz, vp, c_f = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                          ctypes.c_void_p, ctypes.c_float)
            L.rat_status_string.restype = ctypes.c_char_p
            L.rat_status_string.argtypes = [c_int]
            L.rat_last_error.restype = ctypes.c_char_p
            L.rat_last_error.argtypes = []
            L.rat_scan_workspace_size.restype = c_sz
            L.rat_scan_workspace_size.argtypes = [c_int, c_int, c_int, c_int]
            L.rat_scan.restype = c_int
            L.rat_scan.argtypes = [vp, vp, vp, vp, c_int, vp, c_int, c_int, c_int, c_int, c_int,
                                   vp, c_sz, vp]
            L.rat_dilated_prefill_workspace_size.restype = c_sz
            L.rat_dilated_prefill_workspace_size.argtypes = [c_int, c_int, c_int, c_int, vp, c_int, c_int]
            L.rat_dilated_prefill.restype = c_int
            L.rat_dilated_prefill.argtypes = [vp, vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, vp,
                                              c_int, c_f, c_int, vp, c_sz, vp]
            L.rat_dilated_prefill_stage.restype = c_int
            L.rat_dilated_prefill_stage.argtypes = [c_int, vp, vp, vp, vp, vp, vp, c_int, c_int, c_int,
                                                    c_int, vp, c_int, c_f, c_int, vp, c_sz, vp]
            L.rat_grid_layout.restype = c_int
            L.rat_grid_layout.argtypes = [c_int, vp, c_i64, vp, vp, vp]
            L.rat_decode_workspace_size.restype = c_sz
            L.rat_decode_workspace_size.argtypes = [c_int, c_int, c_int, vp, c_int, c_i64]
            L.rat_decode_step.restype = c_int
            L.rat_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                          c_i64, vp, c_int, c_int, c_int, vp, c_int, c_f, c_int,
                                          vp, c_sz, vp]
            L.rat_decode_step_noalloc.restype = c_int
            L.rat_decode_step_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                  c_i64, vp, c_int, c_int, c_int, vp, c_int, c_f, c_int, vp]
            L.rat_prefill_chunk_workspace_size.restype = c_sz
            L.rat_prefill_chunk_workspace_size.argtypes = [c_int, c_int, c_int, c_int, vp, c_int, c_i64, c_int]
            L.rat_prefill_chunk.restype = c_int
            L.rat_prefill_chunk.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, c_i64,
                                            c_i64, c_int, c_int, c_int, c_int, vp, c_int, c_f, c_int, vp,
                                            c_sz, vp]
            L.rat_topk_prefill_workspace_size.restype = c_sz
            L.rat_topk_prefill_workspace_size.argtypes = [c_int, c_int, c_int, c_int]
            L.rat_topk_prefill.restype = c_int
            L.rat_topk_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, c_i64, c_i64, c_int,
                                           c_int, c_int, c_int, c_int, c_int, c_int, c_f, c_int, vp, c_sz, vp]
            L.rat_topk_decode_workspace_size.restype = c_sz
            L.rat_topk_decode_workspace_size.argtypes = []
            L.rat_topk_decode_step.restype = c_int
            L.rat_topk_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, c_i64, vp, vp, c_int,
                                               c_int, c_int, c_int, c_int, c_int, c_f, c_int, vp, c_sz, vp]
            L.rat_local_prefill_chunk_workspace_size.restype = c_sz
            L.rat_local_prefill_chunk_workspace_size.argtypes = [c_int, c_int, c_int, c_int, c_int, c_i64, c_int]
            L.rat_local_prefill_chunk.restype = c_int
            L.rat_local_prefill_chunk.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, c_i64,
                                                  c_i64, c_int, c_int, c_int, c_int, c_int, c_f, c_int, vp, c_sz,
                                                  vp]
            L.rat_local_decode_workspace_size.restype = c_sz
            L.rat_local_decode_workspace_size.argtypes = [c_int, c_int, c_int, c_int, c_i64]
            L.rat_local_decode_step.restype = c_int
            L.rat_local_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, c_i64, vp,
                                                c_int, c_int, c_int, c_int, c_f, c_int, vp, c_sz, vp]
            L.rat_topk_summarize.restype = c_int
            L.rat_topk_summarize.argtypes = [vp, vp, c_i64, c_i64, c_i64, c_int, c_int, c_int, c_int, c_int, vp]
            _lib = L
    return _lib


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def _check(status: int):
    if status != 0:
        raise RatError(status, lib().rat_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RAT_BF16
    if t.dtype == torch.float32:
        return RAT_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _i32_array(vals):
    arr = (ctypes.c_int32 * len(vals))(*[int(v) for v in vals])
    return arr


_ws_cache: dict = {}


def workspace(nbytes: int, device, key="default") -> torch.Tensor:
    """A zero-initialised workspace of at least nbytes, cached per (device, key).

    Workspaces are reused by calls in stream order; they are zero-filled once
    when allocated.
    """
    dev = torch.device(device)
    k = (dev, key)
    ws = _ws_cache.get(k)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=dev)
        _ws_cache[k] = ws
    return ws


def workspace_error(ws: torch.Tensor) -> int:
    """The sticky device error word of a workspace (synchronises)."""
    return int(ws[8:12].view(torch.int32).item())


def workspace_set_poll_limit(ws: torch.Tensor, polls=None) -> None:
    """Set the workspace header's look-back poll limit (byte offset 12):
    None restores the library default; polls = n makes a scan block wait for
    at most n polls of an unpublished predecessor before it computes that
    predecessor's chunk itself (0: on every wait)."""
    ws[12:16].view(torch.int32).fill_(0 if polls is None else int(polls) + 1)


def _per_head(dilation, H):
    if isinstance(dilation, int):
        return [dilation] * H
    d = [int(x) for x in dilation]
    if len(d) != H:
        raise ValueError("dilation must be an int or one value per head")
    return d


# ---------------------------------------------------------------------------
# rat_scan
# ---------------------------------------------------------------------------

def rat_scan_workspace_size(B, T, H, Dh) -> int:
    return int(lib().rat_scan_workspace_size(B, T, H, Dh))


def rat_scan(x, z, h0=None, store_every=1, states=None, h_last=None, ws=None, want_h_last=False):
    """Gated recurrence h_t = g_t h_{t-1} + (1 - g_t) x_t over [B, T, H, Dh].

    Returns (states [B, T // store_every, H, Dh] in x's dtype, h_last or None).
    """
    B, T, H, Dh = x.shape
    if states is None:
        states = torch.empty((B, T // store_every, H, Dh), dtype=x.dtype, device=x.device)
    if want_h_last and h_last is None:
        h_last = torch.empty((B, H, Dh), dtype=torch.float32, device=x.device)
    if z.dtype != torch.float32:
        raise TypeError("gate logits must be fp32")
    if ws is None:
        ws = workspace(rat_scan_workspace_size(B, T, H, Dh), x.device, "scan")
    _check(lib().rat_scan(_ptr(x), _ptr(z), _ptr(h0), _ptr(states), int(store_every), _ptr(h_last),
                          B, T, H, Dh, _dtype_code(x), _ptr(ws), ws.numel(), _stream(x.device)))
    return states, h_last


# ---------------------------------------------------------------------------
# rat_dilated_prefill
# ---------------------------------------------------------------------------

def rat_dilated_prefill_workspace_size(B, T, H, Dh, dilation, W, dtype=torch.bfloat16) -> int:
    d = _i32_array(_per_head(dilation, H))
    code = RAT_BF16 if dtype == torch.bfloat16 else RAT_F32
    return int(lib().rat_dilated_prefill_workspace_size(B, T, H, Dh, d, W, code))


STAGE_ALL, STAGE_RECURRENCE, STAGE_ATTENTION = 0, 1, 2


def rat_dilated_prefill(q, k, v, zk, zv, dilation, W=0, scale=None, out=None, ws=None):
    """Dilated attention over recurrent states; returns out [B, T, H, Dh]."""
    return rat_dilated_prefill_stage(STAGE_ALL, q, k, v, zk, zv, dilation, W, scale, out, ws)


def rat_dilated_prefill_stage(stage, q, k, v, zk, zv, dilation, W=0, scale=None, out=None, ws=None):
    """One stage (0 all, 1 recurrence, 2 attention) of rat_dilated_prefill."""
    B, T, H, Dh = q.shape
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v must share shape and dtype")
    for t in (zk, zv):
        if t.shape != q.shape or t.dtype != torch.float32:
            raise ValueError("zk, zv must be fp32 with q's shape")
    dil = _per_head(dilation, H)
    if out is None:
        out = torch.empty_like(q)
    if ws is None:
        ws = workspace(rat_dilated_prefill_workspace_size(B, T, H, Dh, dil, W, q.dtype), q.device, "prefill")
    s = -1.0 if scale is None else float(scale)
    _check(lib().rat_dilated_prefill_stage(int(stage), _ptr(q), _ptr(k), _ptr(v), _ptr(zk), _ptr(zv),
                                           _ptr(out), B, T, H, Dh, _i32_array(dil), int(W), s,
                                           _dtype_code(q), _ptr(ws), ws.numel(), _stream(q.device)))
    return out


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def rat_grid_layout(H, dilation, max_pos):
    """(grid_off list, grid_cap list, rows per sequence) of the ragged grid cache."""
    dil = _per_head(dilation, H)
    off = (ctypes.c_int64 * H)()
    cap = (ctypes.c_int32 * H)()
    rows = ctypes.c_int64()
    _check(lib().rat_grid_layout(H, _i32_array(dil), int(max_pos), off, cap, ctypes.byref(rows)))
    return list(off), list(cap), int(rows.value)


def rat_decode_workspace_size(B, H, Dh, dilation, W, max_pos) -> int:
    return int(lib().rat_decode_workspace_size(B, H, Dh, _i32_array(_per_head(dilation, H)), W, int(max_pos)))


def rat_decode_step(q, k, v, zk, zv, state_k, state_v, grid_k, grid_v, grid_off, grid_cap,
                    ring_k, ring_v, pos, max_pos, dilation, W, scale=None, out=None, ws=None):
    """One decode step (mutates state, ring and grid caches); returns out [B, H, Dh]."""
    B, H, Dh = q.shape
    dil = _per_head(dilation, H)
    if pos.dtype != torch.int32:
        raise TypeError("pos must be int32")
    if out is None:
        out = torch.empty_like(q)
    if ws is None:
        ws = workspace(rat_decode_workspace_size(B, H, Dh, dil, W, max_pos), q.device, "decode")
    off = (ctypes.c_int64 * H)(*[int(x) for x in grid_off])
    cap = _i32_array(grid_cap)
    s = -1.0 if scale is None else float(scale)
    _check(lib().rat_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(zk), _ptr(zv), _ptr(state_k), _ptr(state_v), _ptr(grid_k),
        _ptr(grid_v), off, cap, _ptr(ring_k), _ptr(ring_v), _ptr(pos), int(max_pos), _ptr(out), B, H,
        Dh, _i32_array(dil), int(W), s, _dtype_code(q), _ptr(ws), ws.numel(), _stream(q.device)))
    return out


DECODE_SCRATCH_BYTES = 32 << 20   # RAT_DECODE_SCRATCH_BYTES in include/rat.h


def rat_decode_step_noalloc(q, k, v, zk, zv, state_k, state_v, grid_k, grid_v, grid_off, grid_cap,
                            ring_k, ring_v, pos, max_pos, dilation, W, scale=None, out=None):
    """rat_decode_step without a workspace: the library's built-in scratch
    (DECODE_SCRATCH_BYTES per GPU) holds the split partials.  Calls that
    overlap on one GPU race; `out` must be given by callers that cannot
    allocate (else it is allocated here)."""
    B, H, Dh = q.shape
    dil = _per_head(dilation, H)
    if pos.dtype != torch.int32:
        raise TypeError("pos must be int32")
    if out is None:
        out = torch.empty_like(q)
    off = (ctypes.c_int64 * H)(*[int(x) for x in grid_off])
    cap = _i32_array(grid_cap)
    s = -1.0 if scale is None else float(scale)
    _check(lib().rat_decode_step_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(zk), _ptr(zv), _ptr(state_k), _ptr(state_v), _ptr(grid_k),
        _ptr(grid_v), off, cap, _ptr(ring_k), _ptr(ring_v), _ptr(pos), int(max_pos), _ptr(out), B, H,
        Dh, _i32_array(dil), int(W), s, _dtype_code(q), _stream(q.device)))
    return out


def rat_prefill_chunk_workspace_size(B, T, H, Dh, dilation, W, p0, dtype=torch.bfloat16) -> int:
    d = _i32_array(_per_head(dilation, H))
    code = RAT_BF16 if dtype == torch.bfloat16 else RAT_F32
    return int(lib().rat_prefill_chunk_workspace_size(B, T, H, Dh, d, W, int(p0), code))


def rat_prefill_chunk(q, k, v, zk, zv, state_k, state_v, grid_k, grid_v, grid_off, grid_cap,
                      ring_k, ring_v, p0, max_pos, dilation, W, scale=None, out=None, ws=None):
    """Prefill positions p0 .. p0+T-1 continuing a decode cache (mutates the
    states, grid and ring caches); returns out [B, T, H, Dh]."""
    B, T, H, Dh = q.shape
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v must share shape and dtype")
    for t in (zk, zv):
        if t.shape != q.shape or t.dtype != torch.float32:
            raise ValueError("zk, zv must be fp32 with q's shape")
    dil = _per_head(dilation, H)
    if out is None:
        out = torch.empty_like(q)
    if ws is None:
        ws = workspace(rat_prefill_chunk_workspace_size(B, T, H, Dh, dil, W, p0, q.dtype), q.device, "chunk")
    off = (ctypes.c_int64 * H)(*[int(x) for x in grid_off])
    cap = _i32_array(grid_cap)
    s = -1.0 if scale is None else float(scale)
    _check(lib().rat_prefill_chunk(
        _ptr(q), _ptr(k), _ptr(v), _ptr(zk), _ptr(zv), _ptr(out), _ptr(state_k), _ptr(state_v),
        _ptr(grid_k), _ptr(grid_v), off, cap, _ptr(ring_k), _ptr(ring_v), int(p0), int(max_pos), B, T, H,
        Dh, _i32_array(dil), int(W), s, _dtype_code(q), _ptr(ws), ws.numel(), _stream(q.device)))
    return out


# ---------------------------------------------------------------------------
# RAT chunk-local variant (restart every L positions, D = L, W = 1)
# ---------------------------------------------------------------------------

def rat_local_prefill_chunk(q, k, v, zk, zv, state_k, state_v, grid_k, grid_v, grid_off, grid_cap, ring_k,
                            ring_v, p0, max_pos, L, scale=None, out=None, ws=None):
    """Chunk-local prefill of positions p0 .. p0+T-1 continuing a decode
    cache (grid layout rat_grid_layout(H, L, max_pos), ring [B, H, 1, Dh])."""
    B, T, H, Dh = q.shape
    if out is None:
        out = torch.empty_like(q)
    if ws is None:
        n = int(lib().rat_local_prefill_chunk_workspace_size(B, T, H, Dh, int(L), int(p0), _dtype_code(q)))
        ws = workspace(n, q.device, "local_chunk")
    off = (ctypes.c_int64 * H)(*[int(x) for x in grid_off])
    cap = _i32_array(grid_cap)
    s = -1.0 if scale is None else float(scale)
    _check(lib().rat_local_prefill_chunk(
        _ptr(q), _ptr(k), _ptr(v), _ptr(zk), _ptr(zv), _ptr(out), _ptr(state_k), _ptr(state_v), _ptr(grid_k),
        _ptr(grid_v), off, cap, _ptr(ring_k), _ptr(ring_v), int(p0), int(max_pos), B, T, H, Dh, int(L), s,
        _dtype_code(q), _ptr(ws), ws.numel(), _stream(q.device)))
    return out


def rat_local_decode_step(q, k, v, zk, zv, state_k, state_v, grid_k, grid_v, grid_off, grid_cap, ring_k, ring_v,
                          pos, max_pos, L, scale=None, out=None, ws=None):
    """One chunk-local decode step at positions pos (int32 [B])."""
    B, H, Dh = q.shape
    if pos.dtype != torch.int32:
        raise TypeError("pos must be int32")
    if out is None:
        out = torch.empty_like(q)
    if ws is None:
        ws = workspace(int(lib().rat_local_decode_workspace_size(B, H, Dh, int(L), int(max_pos))), q.device,
                       "local_decode")
    off = (ctypes.c_int64 * H)(*[int(x) for x in grid_off])
    cap = _i32_array(grid_cap)
    s = -1.0 if scale is None else float(scale)
    _check(lib().rat_local_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(zk), _ptr(zv), _ptr(state_k), _ptr(state_v), _ptr(grid_k), _ptr(grid_v),
        off, cap, _ptr(ring_k), _ptr(ring_v), _ptr(pos), int(max_pos), _ptr(out), B, H, Dh, int(L), s,
        _dtype_code(q), _ptr(ws), ws.numel(), _stream(q.device)))
    return out


# ---------------------------------------------------------------------------
# top-k block attention over the memory states
# ---------------------------------------------------------------------------

TOPK_QUEST, TOPK_MOBA = 0, 1


def topk_cache(B, H, Dh, max_pos, block, dtype=torch.bfloat16, device="cuda:0"):
    """Zeroed state caches for top-k block attention: dict(state_k, state_v
    fp32 [B, H, Dh]; cache_k, cache_v [H, B, max_pos, Dh]; summary fp32
    [H, B, max_pos // block, 3, Dh])."""
    return dict(state_k=torch.zeros((B, H, Dh), dtype=torch.float32, device=device),
                state_v=torch.zeros((B, H, Dh), dtype=torch.float32, device=device),
                cache_k=torch.zeros((H, B, max_pos, Dh), dtype=dtype, device=device),
                cache_v=torch.zeros((H, B, max_pos, Dh), dtype=dtype, device=device),
                summary=torch.zeros((H, B, max_pos // block, 3, Dh), dtype=torch.float32, device=device))


def rat_topk_prefill(q, k, v, zk, zv, cache, p0, max_pos, block, topk, score=TOPK_QUEST, scale=None,
                     out=None, chosen=None, ws=None):
    """Top-k block attention prefill of positions p0 .. p0+T-1 (extends the
    caches in `cache`, see topk_cache); returns out [B, T, H, Dh] (and fills
    `chosen` [B, T, H, topk] int32 if given)."""
    B, T, H, Dh = q.shape
    if out is None:
        out = torch.empty_like(q)
    if ws is None:
        ws = workspace(int(lib().rat_topk_prefill_workspace_size(B, T, H, Dh)), q.device, "topk_prefill")
    s = -1.0 if scale is None else float(scale)
    _check(lib().rat_topk_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(zk), _ptr(zv), _ptr(out), _ptr(chosen), _ptr(cache["state_k"]),
        _ptr(cache["state_v"]), _ptr(cache["cache_k"]), _ptr(cache["cache_v"]), _ptr(cache["summary"]), int(p0),
        int(max_pos), B, T, H, Dh, int(block), int(topk), int(score), s, _dtype_code(q), _ptr(ws), ws.numel(),
        _stream(q.device)))
    return out


def rat_topk_summarize(cache, j_lo, j_hi, max_pos, block):
    """Block summaries j_lo .. j_hi-1 of cache["cache_k"] into cache["summary"]."""
    H, B, _, Dh = cache["cache_k"].shape
    _check(lib().rat_topk_summarize(_ptr(cache["cache_k"]), _ptr(cache["summary"]), int(j_lo), int(j_hi),
                                    int(max_pos), B, H, Dh, int(block), _dtype_code(cache["cache_k"]),
                                    _stream(cache["cache_k"].device)))


def rat_topk_decode_step(q, k, v, zk, zv, cache, pos, max_pos, block, topk, score=TOPK_QUEST, scale=None,
                         out=None, chosen=None, ws=None):
    """One top-k block attention decode step at positions pos (int32 [B]);
    returns out [B, H, Dh] (and fills `chosen` [B, H, topk] if given)."""
    B, H, Dh = q.shape
    if pos.dtype != torch.int32:
        raise TypeError("pos must be int32")
    if out is None:
        out = torch.empty_like(q)
    if ws is None:
        ws = workspace(int(lib().rat_topk_decode_workspace_size()), q.device, "topk_decode")
    s = -1.0 if scale is None else float(scale)
    _check(lib().rat_topk_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(zk), _ptr(zv), _ptr(cache["state_k"]), _ptr(cache["state_v"]),
        _ptr(cache["cache_k"]), _ptr(cache["cache_v"]), _ptr(cache["summary"]), _ptr(pos), int(max_pos), _ptr(out),
        _ptr(chosen), B, H, Dh, int(block), int(topk), int(score), s, _dtype_code(q), _ptr(ws), ws.numel(),
        _stream(q.device)))
    return out


def default_scale(Dh: int) -> float:
    return 1.0 / math.sqrt(Dh)
