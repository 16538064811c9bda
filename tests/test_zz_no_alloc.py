"""sdpa_decode_noalloc (decode step with the partial results in the library's
static device scratch, no allocation) against sdpa_decode, through the C ABI.

Two calls in a row, the second smaller than the first, each compared with
sdpa_decode on the same inputs (same kernels and chunking: the bf16 bars of
the parity tests, and bit-identical output), and the oracle; the binding
allocates nothing through torch around the call.
"""
import numpy as np
import pytest
import torch

import head_attention_fwd_amd as sdpa
import oracle
import workloads
from gpu_helpers import announce, assert_parity, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _inputs(B, H, Lq, Lk, d, lengths, seed):
    dev = require_gpu()
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, d, d, dtype="bf16", seed=seed)
    dq, dk, dv = (to_dev(a, torch.bfloat16) for a in (q, k, v))
    kl = None if lengths is None else torch.as_tensor(np.asarray(lengths, np.int32)).to(dev)
    return (q, k, v), (dq, dk, dv), kl


# (B, H, Lq, Lk, d, lengths): the long decode step, then smaller ones with
# padding (on the key-split paths: one query row at d = 128, several at d = 64
# and 128), then a head size outside them
CALLS = [
    (4, 16, 1, 8192, 64, None),
    (1, 2, 1, 2000, 128, [1999]),
    (2, 4, 5, 3000, 64, [3000, 1234]),
    (1, 2, 3, 700, 128, [650]),
    (1, 2, 3, 300, 256, [250]),
]


def test_noalloc_matches_decode_two_calls():
    for B, H, Lq, Lk, d, lengths in CALLS:
        host, (dq, dk, dv), kl = _inputs(B, H, Lq, Lk, d, lengths, seed=40 + Lk)
        need = sdpa.sdpa_decode_workspace_bytes(B, H, Lq, Lk, d, d, sdpa.SDPA_BF16)
        assert need <= sdpa.DECODE_NOALLOC_SCRATCH_BYTES
        out = torch.full((B, H, Lq, d), float("nan"), dtype=torch.bfloat16, device=dq.device)
        announce("decode_noalloc %s" % ((B, H, Lq, Lk, d),))
        torch.cuda.synchronize()
        n_alloc = torch.cuda.memory_stats()["allocation.all.allocated"]
        sdpa.decode_noalloc(dq, dk, dv, out, key_lengths=kl)
        assert torch.cuda.memory_stats()["allocation.all.allocated"] == n_alloc
        torch.cuda.synchronize()
        ref_dev = sdpa.decode(dq, dk, dv, key_lengths=kl)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        want = ref_dev.float().cpu().numpy().astype(np.float64)
        q, k, v = host
        assert_parity(got, want, v, "bf16", "noalloc vs decode %s" % ((B, H, Lq, Lk),))
        assert np.array_equal(got, want)
        ref = oracle.attention(q, k, v, key_lengths=lengths)
        assert_parity(got, ref, v, "bf16", "noalloc vs oracle %s" % ((B, H, Lq, Lk),))


def test_noalloc_scratch_limit():
    """A split plan larger than the static scratch is refused before any launch,
    and the output is left untouched."""
    dev = require_gpu()
    B, H, Lq, Lk, d = 1, 255, 32, 8192, 128
    need = sdpa.sdpa_decode_workspace_bytes(B, H, Lq, Lk, d, d, sdpa.SDPA_BF16)
    assert need > sdpa.DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, Lq, d), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((B, H, Lk, d), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    out = torch.full((B, H, Lq, d), 7.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(sdpa.SdpaError) as e:
        sdpa.decode_noalloc(q, k, v, out)
    assert e.value.status == sdpa.SDPA_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
