"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import recurrence_augmented_dilated_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "rat.h")).read()
    return sorted(set(re.findall(r"\b(rat_[a-z_]+)\s*\(", src)))


def test_header_symbols_exported():
    L = R.lib()
    names = _declared()
    assert "rat_scan" in names and "rat_dilated_prefill" in names and "rat_decode_step" in names
    for n in names:
        assert hasattr(L, n), f"librat.so does not export {n}"


def test_status_strings():
    L = R.lib()
    assert L.rat_status_string(0) == b"RAT_OK"
    assert L.rat_status_string(-3) == b"RAT_ERR_WORKSPACE"


FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced: validation fails first
MIS = ctypes.c_void_p(0x10004)       # misaligned


def _scan(**kw):
    a = dict(x=FAKE, z=FAKE, h0=None, states=FAKE, E=1, hl=None, B=1, T=16, H=2, Dh=64, dt=0,
             ws=FAKE, wsb=0)
    a.update(kw)
    return R.lib().rat_scan(a["x"], a["z"], a["h0"], a["states"], a["E"], a["hl"], a["B"], a["T"],
                            a["H"], a["Dh"], a["dt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), -1), (dict(z=None), -1), (dict(x=MIS), -1), (dict(Dh=96), -2),
    (dict(B=0), -1), (dict(T=-1), -1), (dict(H=0), -1), (dict(H=129), -1), (dict(E=0), -1),
    (dict(dt=7), -1), (dict(ws=None), -1), (dict(wsb=16), -3),
])
def test_scan_validation(kw, code):
    assert _scan(**kw) == code
    assert R.lib().rat_last_error() != b""


def _prefill(dil=(4, 4), W=0, wsb=0, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, zk=FAKE, zv=FAKE, out=FAKE, B=1, T=64, H=2, Dh=128, dt=1,
             ws=FAKE)
    a.update(kw)
    d = (ctypes.c_int32 * len(dil))(*dil) if dil is not None else None
    return R.lib().rat_dilated_prefill(a["q"], a["k"], a["v"], a["zk"], a["zv"], a["out"], a["B"],
                                       a["T"], a["H"], a["Dh"], d, W, -1.0, a["dt"], a["ws"], wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dil=(0, 4)), -1), (dict(dil=None), -1), (dict(W=-1), -1), (dict(q=None), -1),
    (dict(out=MIS), -1), (dict(Dh=32), -2), (dict(wsb=100), -3),
])
def test_prefill_validation(kw, code):
    assert _prefill(**kw) == code


def test_prefill_length_limit():
    """bf16 attention addresses value rows with 32-bit offsets: at most
    2^31 / Dh positions (rejected before anything is launched; at the limit
    the call gets as far as the workspace check).  fp32 has no such limit."""
    assert _prefill(T=1 << 24) == -3
    assert _prefill(T=(1 << 24) + 1) == -2
    assert b"2^31" in R.lib().rat_last_error()
    assert _prefill(T=1 << 25, Dh=64) == -3
    assert _prefill(T=(1 << 25) + 1, Dh=64) == -2
    assert _prefill(T=(1 << 24) + 1, dt=0) == -3


def test_stage_validation():
    d = (ctypes.c_int32 * 2)(4, 4)
    st = R.lib().rat_dilated_prefill_stage(9, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 2, 128, d, 0,
                                           -1.0, 1, FAKE, 1 << 30, None)
    assert st == -1


def test_decode_validation():
    L = R.lib()
    H = 2
    d = (ctypes.c_int32 * H)(4, 4)
    off = (ctypes.c_int64 * H)(0, 25)
    cap_ok = (ctypes.c_int32 * H)(25, 25)
    cap_bad = (ctypes.c_int32 * H)(24, 25)

    def call(cap=cap_ok, W=4, ring=FAKE, max_pos=100, wsb=0, pos=FAKE):
        return L.rat_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, off, cap, ring, ring,
                                 pos, max_pos, FAKE, 1, H, 128, d, W, -1.0, 1, FAKE, wsb, None)

    assert call(cap=cap_bad) == -1          # grid capacity below max_pos / D
    assert call(ring=None) == -1            # W > 0 needs ring buffers
    assert call(max_pos=0) == -1
    assert call(pos=None) == -1
    assert call() == -3                     # workspace too small
    assert call(W=-2) == -1


def test_workspace_sizes():
    assert R.rat_scan_workspace_size(1, 1024, 2, 64) > 256
    a = R.rat_dilated_prefill_workspace_size(1, 16384, 16, 128, 16, 0)
    b = R.rat_dilated_prefill_workspace_size(1, 16384, 16, 128, 16, 128)
    assert b > a > 0
    assert R.rat_decode_workspace_size(256, 16, 128, 16, 64, 32768 + 1024) > 256


def test_grid_layout():
    off, cap, rows = R.rat_grid_layout(3, [1, 16, 64], 131072 + 1024)
    assert cap == [132096, 8256, 2064]
    assert off == [0, 132096, 132096 + 8256]
    assert rows == sum(cap)


def test_prefill_chunk_validation():
    L = R.lib()
    H = 2
    d = (ctypes.c_int32 * H)(4, 16)
    off = (ctypes.c_int64 * H)(0, 64)
    cap_ok = (ctypes.c_int32 * H)(64, 16)
    cap_bad = (ctypes.c_int32 * H)(63, 16)

    def call(p0=64, T=128, max_pos=256, cap=cap_ok, W=8, ring=FAKE, wsb=0, q=FAKE, dil=d):
        return L.rat_prefill_chunk(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, off, cap, ring,
                                   ring, p0, max_pos, 1, T, H, 128, dil, W, -1.0, 1, FAKE, wsb, None)

    assert call(p0=32) == -2                 # chunk start must be a multiple of 64
    assert call(p0=-64) == -1
    assert call(T=193) == -1                 # p0 + T > max_pos
    assert call(max_pos=1 << 31) == -1       # positions must fit in 31 bits
    assert call(cap=cap_bad) == -1           # grid capacity below max_pos / D
    assert call(ring=None) == -1             # W > 0 needs ring buffers
    assert call(q=None) == -1
    assert call(q=MIS) == -1
    assert call(dil=None) == -1
    assert call(W=-1) == -1
    assert call() == -3                      # workspace too small
    assert call(T=0, q=None, ring=None) == 0  # empty chunk: no-op, NULL buffers allowed
    big_cap = (ctypes.c_int32 * H)(1 << 23, 1 << 21)
    assert call(p0=0, T=(1 << 24) + 1, max_pos=1 << 25, cap=big_cap, wsb=1 << 62) == -2   # bf16 length limit


def test_prefill_chunk_workspace_size():
    a = R.rat_prefill_chunk_workspace_size(1, 1024, 16, 128, 16, 0, 0)
    b = R.rat_prefill_chunk_workspace_size(1, 1024, 16, 128, 16, 128, 0)
    c = R.rat_prefill_chunk_workspace_size(1, 1024, 16, 128, 16, 128, 4096)
    assert 0 < a < b < c          # window buffers; later chunks also hold the ring prefix and more grid
    assert R.rat_prefill_chunk_workspace_size(1, 1024, 16, 128, 16, 0, -64) == 0


def test_topk_validation():
    L = R.lib()

    def pre(block=64, topk=8, score=0, p0=0, T=256, max_pos=1024, chosen=None, q=FAKE, wsb=0):
        return L.rat_topk_prefill(q, FAKE, FAKE, FAKE, FAKE, FAKE, chosen, FAKE, FAKE, FAKE, FAKE, FAKE, p0,
                                  max_pos, 1, T, 2, 128, block, topk, score, -1.0, 1, FAKE, wsb, None)

    assert pre(block=0) == -1
    assert pre(block=2048) == -1
    assert pre(topk=-1) == -1
    assert pre(topk=129) == -1
    assert pre(score=5) == -1
    assert pre(p0=-1) == -1
    assert pre(T=1025) == -1                  # p0 + T > max_pos
    assert pre(block=1, max_pos=8193) == -2   # more blocks than a workgroup can score
    assert pre(q=None) == -1
    assert pre(chosen=MIS) == -1
    assert pre() == -3                        # workspace too small
    assert pre(T=0, q=None) == 0

    def dec(block=64, topk=8, pos=FAKE, wsb=0, max_pos=1024):
        return L.rat_topk_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, pos, max_pos, FAKE,
                                      None, 2, 2, 64, block, topk, 1, -1.0, 1, FAKE, wsb, None)

    assert dec(block=0) == -1
    assert dec(pos=None) == -1
    assert dec(max_pos=0) == -1
    assert dec() == -3
    assert L.rat_topk_decode_workspace_size() == 256
    assert R.lib().rat_topk_prefill_workspace_size(1, 4096, 16, 128) > 256


def test_local_validation():
    L = R.lib()
    H = 2
    off = (ctypes.c_int64 * H)(0, 16)
    cap = (ctypes.c_int32 * H)(16, 16)

    def pre(Lc=16, p0=0, T=128, wsb=0, H=H):
        return L.rat_local_prefill_chunk(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, off, cap, FAKE,
                                         FAKE, p0, 256, 1, T, H, 128, Lc, -1.0, 1, FAKE, wsb, None)

    assert pre(Lc=0) == -1
    assert pre(H=0) == -1
    assert pre(p0=32) == -2                  # chunk start must be a multiple of 64
    assert pre() == -3
    assert L.rat_local_prefill_chunk_workspace_size(1, 128, 2, 128, 16, 0, 1) > 0
    assert L.rat_local_prefill_chunk_workspace_size(1, 128, 2, 128, 0, 0, 1) == 0

    def dec(Lc=16, wsb=0, pos=FAKE):
        return L.rat_local_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, off, cap, FAKE, FAKE,
                                       pos, 256, FAKE, 1, H, 128, Lc, -1.0, 1, FAKE, wsb, None)

    assert dec(Lc=0) == -1
    assert dec(pos=None) == -1
    assert dec() == -3
    assert L.rat_local_decode_workspace_size(1, H, 128, 16, 256) > 256


def test_topk_summarize_validation():
    L = R.lib()
    assert L.rat_topk_summarize(FAKE, FAKE, 0, 17, 1024, 1, 2, 128, 64, 1, None) == -1   # j_hi > max_pos / block
    assert L.rat_topk_summarize(FAKE, FAKE, 5, 4, 1024, 1, 2, 128, 64, 1, None) == -1
    assert L.rat_topk_summarize(None, FAKE, 0, 4, 1024, 1, 2, 128, 64, 1, None) == -1
    assert L.rat_topk_summarize(None, None, 3, 3, 1024, 1, 2, 128, 64, 1, None) == 0      # empty range: no-op
