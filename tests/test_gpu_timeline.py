"""The timestamped build of the library (libsdpa_timeline.so: the same sources
compiled with SDPA_TIMELINE, loaded only by bench.py --timeline): the stamps
must not change a result, and every workgroup's four stamps (entry, first key
tile in, last tile done, stores issued; csrc/sdpa_timeline.h) must be in order.
Checked for the three instrumented kernel files: the matrix-core forward
kernel, the wide-head kernel and the single-row decode kernel."""
import ctypes
import os

import numpy as np
import pytest
import torch

import head_attention_fwd_amd as sdpa
import workloads
from gpu_helpers import announce, require_gpu, to_dev

pytestmark = pytest.mark.gpu

TIMELINE_LIBRARY = os.path.join(os.path.dirname(sdpa.LIBRARY), "libsdpa_timeline.so")
N_WG, N_EV = 1 << 16, 4


def _timeline_lib():
    lib = ctypes.CDLL(TIMELINE_LIBRARY)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.sdpa_forward.restype = ci
    lib.sdpa_forward.argtypes = [vp, vp, vp, vp, ci, vp, i64, i64, i64, i64, i64, i64, ci, vp]
    lib.sdpa_decode.restype = ci
    lib.sdpa_decode.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, vp, i64, vp]
    for name in ("fwd", "wide", "row"):
        fn = getattr(lib, "sdpa_timeline_" + name)
        fn.restype = ci
        fn.argtypes = [vp, i64, ci]
    return lib


# (kind, B, H, Lq, Lk, d, causal, lengths, reader, workgroups)
CASES = [
    ("forward", 2, 2, 300, 300, 64, True, None, "fwd", 2 * 2 * 3),        # 128-row query tiles
    ("forward", 2, 1, 100, 130, 512, False, [130, 17], "wide", 2 * 1 * 2),  # 64-row query tiles
    ("decode", 4, 16, 1, 3000, 64, False, [3000, 1, 0, 2999], "row", None),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-d%d" % (c[0], c[5]))
def test_timeline_build_matches_and_stamps_are_ordered(case):
    kind, B, H, Lq, Lk, d, causal, lengths, reader, n_wg = case
    dev = require_gpu()
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, d, d, dtype="bf16", seed=900 + d)
    dq, dk, dv = (to_dev(a, torch.bfloat16) for a in (q, k, v))
    kl = None if lengths is None else torch.as_tensor(np.asarray(lengths, np.int32)).to(dev)
    tl = _timeline_lib()
    rd = getattr(tl, "sdpa_timeline_" + reader)
    stream = torch.cuda.current_stream(dev).cuda_stream
    out = torch.full((B, H, Lq, d), float("nan"), dtype=torch.bfloat16, device=dev)
    announce("timeline build %s d=%d" % (kind, d))
    torch.cuda.synchronize()
    assert rd(None, 0, 1) == 0
    klp = None if kl is None else kl.data_ptr()
    if kind == "forward":
        ref = sdpa.forward(dq, dk, dv, key_lengths=kl, causal=causal)
        st = tl.sdpa_forward(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), klp, int(causal),
                             out.data_ptr(), B, H, Lq, Lk, d, d, sdpa.SDPA_BF16, stream)
    else:
        ref = sdpa.decode(dq, dk, dv, key_lengths=kl)
        need = sdpa.sdpa_decode_workspace_bytes(B, H, Lq, Lk, d, d, sdpa.SDPA_BF16)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        st = tl.sdpa_decode(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), klp, out.data_ptr(),
                            B, H, Lq, Lk, d, d, sdpa.SDPA_BF16, ws.data_ptr(), need, stream)
        # one workgroup per (head, chunk of keys)
        n_wg = None
    assert st == 0, sdpa.sdpa_status_str(st)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "stamps changed the result"

    buf = np.zeros(N_WG * N_EV, dtype=np.uint64)
    assert rd(buf.ctypes.data, buf.nbytes, 0) == 0
    t = buf.reshape(N_WG, N_EV).astype(np.int64)
    used = np.nonzero(t[:, 0])[0]
    assert len(used) > 0
    if n_wg is not None:
        assert list(used) == list(range(n_wg)), "every workgroup stamps its entry, no other does"
    else:
        assert used[0] == 0 and list(used) == list(range(len(used)))
    t = t[used]
    assert np.all(t[:, 3] >= t[:, 0]) and np.all(t[:, 3] > 0)
    tiles = t[:, 1] > 0          # workgroups that had a key tile (others skip stamps 1 and 2)
    assert tiles.any()
    x = t[tiles]
    assert np.all(x[:, 0] <= x[:, 1]) and np.all(x[:, 1] <= x[:, 2]) and np.all(x[:, 2] <= x[:, 3])
