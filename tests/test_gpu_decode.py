"""GPU parity of sdpa_decode (decode-step attention over a long key/value cache)
against the fp64 oracle with causal = 0, through the C ABI.

The dedicated decode paths (bf16, d_k = d_v in {64, 128}, Lq <= 32: the
vector-unit kernel for one query row, the matrix-core kernels for more) are
checked on cache lengths that cross the key tiles or steps and the chunk
boundaries, with key lengths that end inside a chunk, at a chunk boundary, at
0 and past Lk, both with keys split over workgroups (log-sum-exp merge) and
with one workgroup per head (many heads, short caches: no merge); the other
shapes must run the forward kernels and give exactly sdpa_forward's result.
"""
import numpy as np
import pytest
import torch

import head_attention_fwd_amd as sdpa
import oracle
import workloads
from gpu_helpers import announce, assert_parity, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def decode(q, k, v, lengths=None, dtype="bf16", workspace=None):
    dev = require_gpu()
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    dq, dk, dv = (to_dev(a, td) for a in (q, k, v))
    kl = None if lengths is None else torch.as_tensor(np.asarray(lengths, np.int32)).to(dev)
    out = sdpa.decode(dq, dk, dv, key_lengths=kl, workspace=workspace)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


# (B, H, Lq, Lk, lengths or None)
SPLIT_CASES = [
    (4, 16, 1, 8192, None),                      # long cache, one new position
    (2, 8, 1, 4096 + 17, [4096 + 17, 1000]),     # ragged cache, lengths inside a chunk
    (1, 2, 4, 3000, [64 * 7]),                   # a length on a tile boundary
    (3, 4, 7, 700, [0, 1, 5000]),                # no key, one key, past Lk (clamped)
    (2, 2, 32, 2048, [2048, 129]),               # a full wave of query rows
    (1, 1, 1, 1, None),                          # one key
    (1, 1, 3, 63, None),                         # less than one tile
    (1, 1, 1, 32768 + 5, None),                  # one head: many chunks
]
# at least 256 heads: each head's keys split over the four waves of one
# workgroup and merged in LDS, no workspace; lengths that leave some waves
# without keys (1..96 keys) or all of them (0)
DIRECT_CASES = [
    (64, 8, 1, 256, "uniform"),                  # base model decode step
    (64, 8, 7, 1000, [1000, 0, 33, 999] * 16),   # several rows, lengths 0 and in the tail
    (128, 4, 32, 1024, "uniform"),
    (512, 1, 1, 65, None),
    (256, 1, 3, 100, [5, 96, 97, 1] * 64),
    (4, 64, 1, 8192 + 3, [8192 + 3, 4000, 31, 8192]),   # long caches, 256 heads
]


def _split_ids(cases, d):
    return ["d%d-%s" % (d, c[:4]) for c in cases]


@pytest.mark.parametrize("case,d", [(c, d) for d in (64, 128) for c in SPLIT_CASES + DIRECT_CASES],
                         ids=_split_ids(SPLIT_CASES + DIRECT_CASES, 64) +
                         _split_ids(SPLIT_CASES + DIRECT_CASES, 128))
def test_split_path_parity(case, d):
    B, H, Lq, Lk, lengths = case
    seed = 1000 + B * 7 + Lq * 13 + Lk + d
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, d, d, dtype="bf16", seed=seed)
    if lengths == "uniform":
        lengths = list(np.random.default_rng(seed).integers(1, Lk, size=B, endpoint=True))
    need = sdpa.sdpa_decode_workspace_bytes(B, H, Lq, Lk, d, d, sdpa.SDPA_BF16)
    if case in DIRECT_CASES:
        assert need == 0
    announce("decode d=%d B=%d H=%d Lq=%d Lk=%d" % (d, B, H, Lq, Lk))
    got = decode(q, k, v, lengths)
    ref = oracle.attention(q, k, v, key_lengths=lengths, causal=False)
    assert_parity(got, ref, v, "bf16", "decode %s" % (case[:4],))
    if lengths is not None:
        for b, ln in enumerate(lengths):
            if ln <= 0:
                assert np.all(got[b] == 0.0), "no legal key must give 0"


# One query row (the vector-unit kernel: steps of 64 keys at d = 64, 32 at
# d = 128): (B, H, Lk, lengths or None).  Few heads split their keys into
# chunks of whole steps per wave (four-wave workgroups, merged by the second
# kernel); 256 heads or more, or short caches, take one chunk each (two waves
# up to four steps of keys, else four).
ROW_CASES = [
    (1, 1, 1, None),                             # one key
    (1, 1, 31, None), (1, 1, 32, None), (1, 1, 33, None),   # around one step (d = 128)
    (1, 1, 63, None), (1, 1, 64, None), (1, 1, 65, None),   # around one step (d = 64)
    (1, 1, 129, None),                           # second wave: one key
    (1, 1, 257, None),                           # third of four waves: one key
    (1, 1, 1025, None),                          # two chunks (d = 64), the second with one key
    (2, 3, 300, [300, 0]),                       # a sequence without keys
    (3, 2, 1000, [1, 999, 5000]),                # one key, one short of Lk, past Lk
    (2, 3, 700, [-5, 700]),                      # a negative length reads as no key
    (1, 2, 4096, [512]),                         # the length on a chunk boundary
    (1, 2, 4096, [513]),                         # one key into the next chunk
    (1, 4, 32768 + 5, None),                     # many chunks per head
    (64, 8, 256, "uniform"),                     # base model decode step: one chunk per head
    (300, 1, 70, [0, 1, 64, 65, 70] * 60),       # 300 heads, one chunk each, waves without keys
    (4, 64, 8192 + 3, [8192 + 3, 4000, 31, 8192]),
]


@pytest.mark.parametrize("case,d", [(c, d) for d in (64, 128) for c in ROW_CASES],
                         ids=["d%d-%s" % (d, c[:3]) for d in (64, 128) for c in ROW_CASES])
def test_single_row_parity(case, d):
    B, H, Lk, lengths = case
    seed = 4000 + B * 7 + H * 3 + Lk + d
    q, k, v, _ = workloads.draw(B, H, 1, Lk, d, d, dtype="bf16", seed=seed)
    if lengths == "uniform":
        lengths = list(np.random.default_rng(seed).integers(1, Lk, size=B, endpoint=True))
    need = sdpa.sdpa_decode_workspace_bytes(B, H, 1, Lk, d, d, sdpa.SDPA_BF16)
    if B * H >= 256:
        assert need == 0
    announce("decode one row d=%d B=%d H=%d Lk=%d workspace %d" % (d, B, H, Lk, need))
    got = decode(q, k, v, lengths)
    ref = oracle.attention(q, k, v, key_lengths=lengths, causal=False)
    assert_parity(got, ref, v, "bf16", "decode one row %s" % (case[:3],))
    if lengths is not None:
        for b, ln in enumerate(lengths):
            if ln <= 0:
                assert np.all(got[b] == 0.0), "no legal key must give 0"


def test_split_path_matches_forward_within_the_bars_and_is_deterministic():
    B, H, Lq, Lk = 2, 4, 3, 5000
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, 64, 64, dtype="bf16", seed=77)
    dev = require_gpu()
    dq, dk, dv = (to_dev(a, torch.bfloat16) for a in (q, k, v))
    announce("decode vs forward")
    a = sdpa.decode(dq, dk, dv)
    b = sdpa.decode(dq, dk, dv)
    f = sdpa.forward(dq, dk, dv, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle.attention(q, k, v, causal=False)
    assert_parity(a.float().cpu().numpy(), ref, v, "bf16", "decode")
    assert_parity(f.float().cpu().numpy(), ref, v, "bf16", "forward")
    assert dev.type == "cuda"


def test_workspace_reused_by_a_smaller_call():
    """One workspace, two calls in stream order, the second smaller: the first
    call's partial results must not leak into the second."""
    dev = require_gpu()
    big = sdpa.sdpa_decode_workspace_bytes(4, 8, 8, 6000, 64, 64, sdpa.SDPA_BF16)
    ws = torch.full((big,), 0x7F, dtype=torch.uint8, device=dev)   # NaN-ish fill
    announce("decode workspace reuse")
    q1, k1, v1, _ = workloads.draw(4, 8, 8, 6000, 64, 64, dtype="bf16", seed=3)
    q2, k2, v2, _ = workloads.draw(1, 2, 2, 900, 64, 64, dtype="bf16", seed=4)
    g1 = decode(q1, k1, v1, [6000, 10, 3000, 0], workspace=ws)
    g2 = decode(q2, k2, v2, None, workspace=ws)
    assert_parity(g1, oracle.attention(q1, k1, v1, key_lengths=[6000, 10, 3000, 0]), v1, "bf16", "first")
    assert_parity(g2, oracle.attention(q2, k2, v2), v2, "bf16", "second")


def test_workspace_too_small_raises():
    dev = require_gpu()
    q, k, v, _ = workloads.draw(1, 2, 1, 1000, 64, 64, dtype="bf16", seed=5)
    dq, dk, dv = (to_dev(a, torch.bfloat16) for a in (q, k, v))
    ws = torch.empty(64, dtype=torch.uint8, device=dev)
    with pytest.raises(sdpa.SdpaError) as e:
        sdpa.decode(dq, dk, dv, workspace=ws)
    assert e.value.status == sdpa.SDPA_ERR_WORKSPACE


@pytest.mark.parametrize("dtype,d,Lq", [("f32", 64, 1), ("bf16", 32, 2), ("bf16", 64, 33),
                                     ("bf16", 128, 33), ("bf16", 512, 1)])
def test_other_shapes_run_the_forward_kernels(dtype, d, Lq):
    """No split path: sdpa_decode must give exactly sdpa_forward(causal=0)."""
    B, H, Lk = 2, 2, 300
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, d, d, dtype=dtype, seed=11)
    assert sdpa.sdpa_decode_workspace_bytes(B, H, Lq, Lk, d, d,
                                            sdpa.SDPA_BF16 if dtype == "bf16" else sdpa.SDPA_F32) == 0
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    dq, dk, dv = (to_dev(a, td) for a in (q, k, v))
    announce("decode fallback %s d=%d Lq=%d" % (dtype, d, Lq))
    a = sdpa.decode(dq, dk, dv, key_lengths=[300, 17])
    f = sdpa.forward(dq, dk, dv, key_lengths=[300, 17])
    torch.cuda.synchronize()
    assert torch.equal(a, f)
    ref = oracle.attention(q, k, v, key_lengths=[300, 17])
    assert_parity(a.float().cpu().numpy(), ref, v, dtype, "fallback")
