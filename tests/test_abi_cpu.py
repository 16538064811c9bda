"""The C ABI without a GPU: the library loads, exports what include/sdpa.h
declares, and rejects invalid calls on the host before any HIP call.

Pointers passed here are fake addresses; every call below is one the library
must refuse (or treat as empty) before touching the device.
"""
import ctypes
import os
import re

import pytest

import head_attention_fwd_amd as sdpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdpa.h")

FAKE_Q, FAKE_K, FAKE_V, FAKE_O = 0x1000000, 0x2000000, 0x3000000, 0x4000000


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdpa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(sdpa.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(sdpa.LIBRARY)
    for name in declared_functions():
        assert hasattr(lib, name), name


TIMELINE_READERS = ("sdpa_timeline_fwd", "sdpa_timeline_wide", "sdpa_timeline_row")


def test_timeline_build_exports_the_abi_and_its_readers():
    """libsdpa_timeline.so (the same sources with per-workgroup stamps) has the
    whole C ABI plus one record reader per instrumented source; the normal
    library compiles the stamps out and has no reader."""
    tl = ctypes.CDLL(os.path.join(os.path.dirname(sdpa.LIBRARY), "libsdpa_timeline.so"))
    for name in declared_functions() + list(TIMELINE_READERS):
        assert hasattr(tl, name), name
    lib = ctypes.CDLL(sdpa.LIBRARY)
    for name in TIMELINE_READERS:
        assert not hasattr(lib, name), name


def test_status_strings():
    for st in range(8):
        s = sdpa.sdpa_status_str(st)
        assert isinstance(s, str) and s
    assert sdpa.sdpa_status_str(0) == "success"
    assert "unknown" in sdpa.sdpa_status_str(99)
    assert sdpa.sdpa_last_hip_error() == 0


def call(Q=FAKE_Q, K=FAKE_K, V=FAKE_V, kl=0, causal=0, O=FAKE_O, B=2, H=2, Lq=16, Lk=16,
         dk=64, dv=64, dtype=sdpa.SDPA_BF16):
    return sdpa.sdpa_forward(Q, K, V, kl, causal, O, B, H, Lq, Lk, dk, dv, dtype, 0)


@pytest.mark.parametrize("kw,expected", [
    (dict(Q=0), sdpa.SDPA_ERR_NULL_POINTER),
    (dict(K=0), sdpa.SDPA_ERR_NULL_POINTER),
    (dict(V=0), sdpa.SDPA_ERR_NULL_POINTER),
    (dict(O=0), sdpa.SDPA_ERR_NULL_POINTER),
    (dict(B=-1), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(H=-3), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(Lq=-1), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(Lk=-1), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(dk=0), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(dv=0), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(Lq=2**31), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(B=2**20, H=2**20), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(B=2**16, H=2**10, Lq=2**20, Lk=1, dk=1, dv=1), sdpa.SDPA_ERR_BAD_SHAPE),
    # the wide kernel (d > 256) uses ceil(Lq / 16) workgroups per head: 2^24 + 1 is too many
    (dict(B=1, H=1, Lq=2**28 + 1, Lk=1, dk=512, dv=512), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(dk=513), sdpa.SDPA_ERR_UNSUPPORTED),
    (dict(dv=513), sdpa.SDPA_ERR_UNSUPPORTED),
    (dict(dk=513, dtype=sdpa.SDPA_F32), sdpa.SDPA_ERR_UNSUPPORTED),
    (dict(dtype=7), sdpa.SDPA_ERR_UNSUPPORTED),
    # out overlapping an input (byte ranges computed on the host)
    (dict(O=FAKE_Q), sdpa.SDPA_ERR_ALIAS),
    (dict(O=FAKE_Q + 2 * 2 * 16 * 64 * 2 - 2), sdpa.SDPA_ERR_ALIAS),
    (dict(O=FAKE_K - 2), sdpa.SDPA_ERR_ALIAS),
    (dict(O=FAKE_V + 64), sdpa.SDPA_ERR_ALIAS),
    (dict(kl=FAKE_O + 8), sdpa.SDPA_ERR_ALIAS),
])
def test_prelaunch_validation(kw, expected):
    assert call(**kw) == expected


def test_adjacent_buffers_are_not_aliases_but_empty_calls_launch_nothing():
    # B == 0, H == 0 or Lq == 0: nothing to compute, success without any HIP call.
    assert call(B=0) == sdpa.SDPA_OK
    assert call(H=0) == sdpa.SDPA_OK
    assert call(Lq=0) == sdpa.SDPA_OK
    # empty call with NULL pointers is still fine
    assert call(Q=0, K=0, V=0, O=0, Lq=0) == sdpa.SDPA_OK
    # out exactly one past the end of Q is not an overlap (checked on an empty-free
    # shape only through the alias helper's arithmetic: Q occupies [Q, Q + 8192)).
    assert call(O=FAKE_Q + 2 * 2 * 16 * 64 * 2, B=0) == sdpa.SDPA_OK


def test_python_forward_rejects_bad_arguments_without_gpu():
    import torch
    q = torch.zeros(1, 1, 4, 8)
    with pytest.raises(ValueError):
        sdpa.forward(q, q, q)          # CPU tensors are refused, never computed
    with pytest.raises(ValueError):
        sdpa.forward(q[0], q, q)
    with pytest.raises(TypeError):
        sdpa.forward(q.half(), q.half(), q.half())


def test_python_multihead_rejects_bad_arguments_without_gpu():
    import torch
    x = torch.zeros(1, 4, 64, dtype=torch.bfloat16)
    w = torch.zeros(64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sdpa.multihead(x, x, w, w, w, w, 0)       # no heads
    with pytest.raises(ValueError):
        sdpa.multihead(x, x, w, w, w, w, 2)       # CPU tensors are refused, never computed


# ---- sdpa_decode: the same host-side checks, plus the workspace

# Default shape: keys split over two chunks (a workspace is needed), every
# buffer inside its 16 MiB slot of fake addresses.
def dcall(Q=FAKE_Q, K=FAKE_K, V=FAKE_V, kl=0, O=FAKE_O, B=1, H=1, Lq=1, Lk=600,
          dk=64, dv=64, dtype=sdpa.SDPA_BF16, ws=0x8000000, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = sdpa.sdpa_decode_workspace_bytes(B, H, Lq, Lk, dk, dv, dtype)
    return sdpa.sdpa_decode(Q, K, V, kl, O, B, H, Lq, Lk, dk, dv, dtype, ws, ws_bytes, 0)


def test_decode_workspace_bytes():
    ws = sdpa.sdpa_decode_workspace_bytes
    bf, f32 = sdpa.SDPA_BF16, sdpa.SDPA_F32
    # one query row: the vector-unit kernel, steps of 4096 / d keys, chunks of
    # four waves with at least two steps per wave and about 2048 waves in all;
    # 4 * (d_v + 2) bytes per head and chunk
    assert ws(4, 16, 1, 8192, 64, 64, bf) == 4 * 66 * 64 * 8       # 128 steps, 8 chunks of 16
    assert ws(4, 8, 1, 8192, 128, 128, bf) == 4 * 130 * 32 * 16    # 256 steps of 32 keys, 16 chunks
    assert ws(1, 1, 1, 600, 64, 64, bf) == 4 * 66 * 2              # 10 steps: two chunks of 8
    assert ws(2, 100, 1, 1025, 64, 64, bf) == 4 * 66 * 200 * 3     # 17 steps: three chunks of 8
    assert ws(1, 1, 1, 512, 64, 64, bf) == 0                       # 8 steps: one chunk, no merge
    assert ws(1, 1, 1, 100, 64, 64, bf) == 0
    assert ws(64, 8, 1, 256, 64, 64, bf) == 0                      # at least 256 heads: one chunk
    assert ws(64, 8, 1, 100000, 128, 128, bf) == 0
    assert ws(4, 16, 1, 0, 64, 64, bf) == 0                        # no keys: one (empty) chunk
    # 2 to 32 query rows: the matrix-core kernels, linear in Lq for a fixed plan
    five = ws(4, 16, 5, 8192, 64, 64, bf)
    assert five > 0 and five % (4 * 66 * 64 * 5) == 0              # 4 * (d_v + 2) * B * H * Lq * chunks
    assert ws(4, 16, 32, 8192, 64, 64, bf) * 5 == five * 32
    assert ws(4, 8, 2, 8192, 128, 128, bf) % (4 * 130 * 32 * 2) == 0
    assert ws(64, 8, 32, 1024, 128, 128, bf) == 0                  # at least 256 heads: merged in LDS
    # the dedicated paths are bf16, d in {64, 128}, Lq <= 32 only; otherwise no workspace
    assert ws(4, 16, 33, 8192, 64, 64, bf) == 0
    assert ws(4, 16, 1, 8192, 64, 64, f32) == 0
    assert ws(4, 16, 1, 8192, 32, 32, bf) == 0
    assert ws(4, 16, 1, 8192, 256, 256, bf) == 0
    assert ws(0, 16, 1, 8192, 64, 64, bf) == 0                     # empty call
    # sizes the entry point rejects
    assert ws(-1, 16, 1, 8192, 64, 64, bf) == -1
    assert ws(4, 16, 1, 8192, 513, 64, bf) == -1
    assert ws(4, 16, 1, 8192, 64, 64, 9) == -1


@pytest.mark.parametrize("kw,expected", [
    (dict(Q=0), sdpa.SDPA_ERR_NULL_POINTER),
    (dict(O=0), sdpa.SDPA_ERR_NULL_POINTER),
    (dict(B=-1), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(dk=513), sdpa.SDPA_ERR_UNSUPPORTED),
    (dict(O=FAKE_Q), sdpa.SDPA_ERR_ALIAS),
    (dict(ws=0), sdpa.SDPA_ERR_WORKSPACE),
    (dict(ws_bytes=100), sdpa.SDPA_ERR_WORKSPACE),        # the plan needs 528 bytes
    (dict(ws=FAKE_V + 64), sdpa.SDPA_ERR_WORKSPACE),     # overlaps V
    (dict(ws=FAKE_O - 64), sdpa.SDPA_ERR_WORKSPACE),     # overlaps out
])
def test_decode_prelaunch_validation(kw, expected):
    assert dcall(**kw) == expected


def test_decode_empty_calls():
    assert dcall(B=0) == sdpa.SDPA_OK
    assert dcall(Lq=0, ws=0) == sdpa.SDPA_OK
    assert dcall(Q=0, K=0, V=0, O=0, H=0, ws=0) == sdpa.SDPA_OK
    assert sdpa.sdpa_status_str(sdpa.SDPA_ERR_WORKSPACE).startswith("the workspace")


# ---- sdpa_decode_noalloc: sdpa_decode's checks, the static scratch's limit

def ncall(Q=FAKE_Q, K=FAKE_K, V=FAKE_V, kl=0, O=FAKE_O, B=4, H=16, Lq=1, Lk=8192, dk=64, dv=64,
          dtype=sdpa.SDPA_BF16):
    return sdpa.sdpa_decode_noalloc(Q, K, V, kl, O, B, H, Lq, Lk, dk, dv, dtype, 0)


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER, encoding="utf-8").read()
    m = re.search(r"#define SDPA_DECODE_NOALLOC_SCRATCH_BYTES \((\d+) \* (\d+) \* (\d+)\)", text)
    assert m, "SDPA_DECODE_NOALLOC_SCRATCH_BYTES not found"
    assert int(m.group(1)) * int(m.group(2)) * int(m.group(3)) == sdpa.DECODE_NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("kw,expected", [
    (dict(Q=0), sdpa.SDPA_ERR_NULL_POINTER),
    (dict(O=0), sdpa.SDPA_ERR_NULL_POINTER),
    (dict(B=-1), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(dk=513), sdpa.SDPA_ERR_UNSUPPORTED),
    (dict(O=FAKE_K + 64), sdpa.SDPA_ERR_ALIAS),
    # 255 heads x 32 rows in seven chunks each, d = 128: 29.7 MB of partial results
    (dict(Q=1 << 32, K=2 << 32, V=3 << 32, O=4 << 32, B=1, H=255, Lq=32, Lk=8192, dk=128, dv=128),
     sdpa.SDPA_ERR_SCRATCH_LIMIT),
])
def test_noalloc_prelaunch_validation(kw, expected):
    assert ncall(**kw) == expected


def test_noalloc_limit_is_the_workspace_size():
    ws = sdpa.sdpa_decode_workspace_bytes
    assert ws(1, 255, 32, 8192, 128, 128, sdpa.SDPA_BF16) > sdpa.DECODE_NOALLOC_SCRATCH_BYTES
    assert ws(4, 16, 1, 8192, 64, 64, sdpa.SDPA_BF16) <= sdpa.DECODE_NOALLOC_SCRATCH_BYTES
    assert "static device scratch" in sdpa.sdpa_status_str(sdpa.SDPA_ERR_SCRATCH_LIMIT)


def test_noalloc_empty_calls():
    assert ncall(B=0) == sdpa.SDPA_OK
    assert ncall(Q=0, K=0, V=0, O=0, Lq=0) == sdpa.SDPA_OK


# ---- sdpa_forward_restricted: sdpa_forward's checks plus the radius

def rcall(radius=3, **kw):
    a = dict(Q=FAKE_Q, K=FAKE_K, V=FAKE_V, kl=0, causal=0, O=FAKE_O, B=2, H=2, Lq=16, Lk=16,
             dk=64, dv=64, dtype=sdpa.SDPA_BF16)
    a.update(kw)
    return sdpa.sdpa_forward_restricted(a["Q"], a["K"], a["V"], a["kl"], a["causal"], radius,
                                        a["O"], a["B"], a["H"], a["Lq"], a["Lk"], a["dk"], a["dv"],
                                        a["dtype"], 0)


@pytest.mark.parametrize("kw,expected", [
    (dict(radius=-1), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(radius=-2**40), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(radius=-1, B=0), sdpa.SDPA_ERR_BAD_SHAPE),     # checked before the empty-call shortcut
    (dict(Q=0), sdpa.SDPA_ERR_NULL_POINTER),
    (dict(O=0, radius=0), sdpa.SDPA_ERR_NULL_POINTER),
    (dict(Lk=-1), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(dk=513), sdpa.SDPA_ERR_UNSUPPORTED),
    (dict(dtype=7), sdpa.SDPA_ERR_UNSUPPORTED),
    (dict(O=FAKE_V + 64), sdpa.SDPA_ERR_ALIAS),
])
def test_restricted_prelaunch_validation(kw, expected):
    assert rcall(**kw) == expected


def test_restricted_empty_calls():
    assert rcall(B=0) == sdpa.SDPA_OK
    assert rcall(Lq=0, radius=2**40) == sdpa.SDPA_OK
    assert rcall(Q=0, K=0, V=0, O=0, H=0, radius=0) == sdpa.SDPA_OK


# ---- sdpa_multihead_forward: host-side checks

FAKE_X, FAKE_WQ, FAKE_WK, FAKE_WV, FAKE_WO, FAKE_WS = (0x100000, 0x200000, 0x300000, 0x400000,
                                                       0x500000, 0x1000000)
FAKE_OUT = 0x600000


def mcall(**kw):
    a = dict(Xq=FAKE_X, Xkv=FAKE_X, Wq=FAKE_WQ, Wk=FAKE_WK, Wv=FAKE_WV, Wo=FAKE_WO, kl=0,
             causal=0, out=FAKE_OUT, B=2, Lq=16, Lk=16, dm=64, h=2, dk=32, dv=32,
             dtype=sdpa.SDPA_BF16, ws=FAKE_WS, ws_bytes=1 << 20)
    a.update(kw)
    return sdpa.sdpa_multihead_forward(a["Xq"], a["Xkv"], a["Wq"], a["Wk"], a["Wv"], a["Wo"],
                                       a["kl"], a["causal"], a["out"], a["B"], a["Lq"], a["Lk"],
                                       a["dm"], a["h"], a["dk"], a["dv"], a["dtype"], a["ws"],
                                       a["ws_bytes"], 0)


def test_multihead_workspace_bytes():
    f = sdpa.sdpa_multihead_workspace_bytes
    # Q, K, V heads and the attention output, bf16, each 256-byte aligned
    assert f(2, 16, 16, 64, 2, 32, 32, sdpa.SDPA_BF16) == 4 * (2 * 2 * 16 * 32 * 2)
    n = f(3, 7, 9, 64, 2, 8, 32, sdpa.SDPA_BF16)
    sizes = [3 * 2 * 7 * 8 * 2, 3 * 2 * 9 * 8 * 2, 3 * 2 * 9 * 32 * 2, 3 * 2 * 7 * 32 * 2]
    off = 0
    for s in sizes:
        off = (off + s + 255) // 256 * 256
    assert n == off
    assert f(2, 16, 16, 64, 2, 32, 32, sdpa.SDPA_F32) == -1      # bf16 only
    assert f(2, 16, 16, 48, 2, 32, 32, sdpa.SDPA_BF16) == -1     # d_model % 32
    assert f(2, 16, 16, 64, 2, 12, 32, sdpa.SDPA_BF16) == -1     # d_k % 8
    assert f(2, 16, 16, 64, 2, 32, 16, sdpa.SDPA_BF16) == -1     # d_v % 32
    assert f(2, 16, 16, 64, 2, 520, 32, sdpa.SDPA_BF16) == -1    # d_k > 512
    assert f(-1, 16, 16, 64, 2, 32, 32, sdpa.SDPA_BF16) == -1
    assert f(1, 2**21, 2**21, 1024, 16, 64, 64, sdpa.SDPA_BF16) == -1   # tensors past 2 GiB
    assert f(0, 16, 16, 64, 2, 32, 32, sdpa.SDPA_BF16) == 0


@pytest.mark.parametrize("kw,expected", [
    (dict(Xq=0), sdpa.SDPA_ERR_NULL_POINTER),
    (dict(Wk=0), sdpa.SDPA_ERR_NULL_POINTER),
    (dict(Wo=0), sdpa.SDPA_ERR_NULL_POINTER),
    (dict(out=0), sdpa.SDPA_ERR_NULL_POINTER),
    (dict(Xkv=0, Lk=4), sdpa.SDPA_ERR_NULL_POINTER),
    (dict(dtype=sdpa.SDPA_F32), sdpa.SDPA_ERR_UNSUPPORTED),
    (dict(dm=40), sdpa.SDPA_ERR_UNSUPPORTED),
    (dict(dv=40), sdpa.SDPA_ERR_UNSUPPORTED),
    (dict(h=0), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(Lk=-3), sdpa.SDPA_ERR_BAD_SHAPE),
    (dict(ws=0), sdpa.SDPA_ERR_WORKSPACE),
    (dict(ws_bytes=100), sdpa.SDPA_ERR_WORKSPACE),
    (dict(ws=FAKE_X), sdpa.SDPA_ERR_WORKSPACE),          # workspace over an input
    (dict(ws=FAKE_OUT - 64), sdpa.SDPA_ERR_WORKSPACE),   # workspace over out
    (dict(out=FAKE_WQ + 64), sdpa.SDPA_ERR_ALIAS),
    (dict(out=FAKE_X), sdpa.SDPA_ERR_ALIAS),
])
def test_multihead_prelaunch_validation(kw, expected):
    assert mcall(**kw) == expected


def test_multihead_empty_calls():
    assert mcall(B=0) == sdpa.SDPA_OK
    assert mcall(Lq=0, Lk=3) == sdpa.SDPA_OK
    assert mcall(B=0, Xq=0, Xkv=0, Wq=0, Wk=0, Wv=0, Wo=0, out=0, ws=0) == sdpa.SDPA_OK
