"""GPU parity when scores jump far above a row's running maximum after the first
key tile, against the fp64 oracle, through the C ABI.

The matrix-core kernels keep a per-row reference maximum that moves only when
needed; on fully legal tiles they take the weights against it without a block
maximum and move it only when a block's weights sum past 2^20.  A query row's
32 keys of a block are held by two lanes (16 each), so a dominant key sits in
one of the two halves: these cases put such keys at key offsets falling in
either half, in tiles after the first, growing by about 20 nats each, and also
draw Q and K at 4 and 8 times unit scale so that the row maxima keep growing
throughout.  Every head size, the causal and padding masks, restricted
attention, the decode step's key-split path and the fp32 kernels are covered.
Softmax is unchanged by the shift of the maximum (page "Self-Attention คืออะไร
(แบบจับต้องได้)", the [100,100,100] vs [0,0,0] remark), so the oracle's rows are
exact references however large the scores.
"""
import numpy as np
import pytest
import torch

import head_attention_fwd_amd as sdpa
import oracle
import workloads
from gpu_helpers import announce, assert_parity, require_gpu, run, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

# (key, strength in nats): offsets within 32-key blocks 6, 8, 13, 5, 4, 22, 31
# (lane halves 0, 1, 1, 0, 0, 0, 1), tiles 1, 3, 5, 8, 14 of 64 keys and beyond
SPIKES = ((70, 20.0), (200, 40.0), (333, 60.0), (517, 80.0), (900, 100.0),
          (1398, 120.0), (2047, 140.0))


def _spiked(B, H, Lq, Lk, d, dtype="bf16", seed=0, qk_scale=1.0, spikes=SPIKES):
    return workloads.draw_spiked(B, H, Lq, Lk, d, dtype=dtype, seed=seed, spikes=spikes,
                                 qk_scale=qk_scale)


# (B, H, Lq, Lk, d, causal, lengths)
FORWARD = []
for _d in (16, 32, 64, 128, 256, 512):
    FORWARD += [
        (1, 2, 256, 1000, _d, False, None),
        (2, 2, 1000, 1000, _d, True, None),
        (2, 2, 300, 1000, _d, False, [1000, 600]),
    ]
FORWARD += [
    (1, 2, 200, 2100, 64, False, None),    # every spike, 64-key tiles up to 2100 keys
    (1, 2, 2100, 2100, 64, True, None),
    (1, 2, 512, 512, 64, True, None),      # short causal launch: 32-key tiles
]


@pytest.mark.parametrize("case", FORWARD, ids=lambda c: "x".join(map(str, c[:5])) +
                         ("c" if c[5] else "n") + ("p" if c[6] else ""))
def test_forward_dominant_keys(case):
    B, H, Lq, Lk, d, causal, lengths = case
    q, k, v = _spiked(B, H, Lq, Lk, d, seed=31 + d + Lq)
    announce("dominant keys forward %s" % (case,))
    got = run(q, k, v, lengths, causal, "bf16")
    ref = oracle.attention(q, k, v, key_lengths=lengths, causal=causal)
    assert_parity(got, ref, v, "bf16", "dominant keys %s" % (case,))


@pytest.mark.parametrize("qk_scale", [4.0, 8.0])
@pytest.mark.parametrize("d", [16, 32, 64, 128, 256, 512])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_scaled_scores(qk_scale, d, causal):
    """Q and K at 4 and 8 times unit scale: score spreads of tens to hundreds of nats."""
    B, H, L = 1, 2, 700
    q, k, v, _ = workloads.draw(B, H, L, L, d, d, dtype="bf16", seed=int(qk_scale) * 100 + d)
    q = workloads.round_to_bf16(q * qk_scale)
    k = workloads.round_to_bf16(k * qk_scale)
    lengths = None if causal else [L]
    announce("scaled scores x%g d=%d causal=%s" % (qk_scale, d, causal))
    got = run(q, k, v, lengths, causal, "bf16")
    ref = oracle.attention(q, k, v, key_lengths=lengths, causal=causal)
    assert_parity(got, ref, v, "bf16", "scaled x%g d=%d" % (qk_scale, d))


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_restricted_dominant_keys(d, causal):
    """Band kernel: dominant keys inside the neighbourhood's fully legal middle."""
    B, H, L, radius = 1, 2, 1200, 300
    q, k, v = _spiked(B, H, L, L, d, seed=77 + d)
    dev = require_gpu()
    announce("dominant keys restricted d=%d causal=%s" % (d, causal))
    out = sdpa.restricted(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16),
                          to_dev(v, torch.bfloat16), radius, causal=causal)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = oracle.attention(q, k, v, causal=causal, radius=radius)
    assert_parity(got, ref, v, "bf16", "restricted d=%d" % d)
    assert dev.type == "cuda"


@pytest.mark.parametrize("Lq,d", [(1, 64), (1, 128), (5, 64), (32, 64), (32, 128)])
def test_decode_dominant_keys(Lq, d):
    """Decode step (keys split over workgroups, log-sum-exp merge; one query
    row on the vector-unit kernel): dominant keys inside chunks after the first
    and in chunks of their own."""
    B, H, Lk = 2, 4, 5000
    spikes = SPIKES + ((3000, 160.0), (4999, 180.0))
    q, k, v = _spiked(B, H, Lq, Lk, d, seed=500 + Lq + d, spikes=spikes)
    lengths = [Lk, 3500]
    dev = require_gpu()
    announce("dominant keys decode Lq=%d d=%d" % (Lq, d))
    kl = torch.as_tensor(np.asarray(lengths, np.int32)).to(dev)
    out = sdpa.decode(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16),
                      to_dev(v, torch.bfloat16), key_lengths=kl)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = oracle.attention(q, k, v, key_lengths=lengths)
    assert_parity(got, ref, v, "bf16", "decode Lq=%d d=%d" % (Lq, d))


@pytest.mark.parametrize("d", [8, 64, 300])
def test_f32_dominant_keys(d):
    """fp32 kernels (one row per lane; 8 or 16 lanes per row above d = 128)."""
    B, H, L = 1, 2, 1000
    q, k, v = _spiked(B, H, L, L, d, dtype="f32", seed=900 + d)
    announce("dominant keys f32 d=%d" % d)
    got = run(q, k, v, None, True, "f32")
    ref = oracle.attention(q, k, v, causal=True)
    # Scores of up to ~140 nats: an fp32 dot product of d terms is within
    # d * u * sum_t |q_t k_t| of the exact one (u = 2^-24, the textbook forward
    # error bound of a recursive sum), and an error e in every score moves a
    # softmax-weighted mean of V by at most 2 e max|V|; on top of the 1e-5 bar.
    s_abs = np.einsum("bhid,bhjd->bhij", np.abs(q).astype(np.float64),
                      np.abs(k).astype(np.float64)) / np.sqrt(d)
    e = d * 2.0 ** -24 * float(s_abs.max())
    bar = 1e-5 + 2.0 * e * float(np.abs(v).max())
    err = float(np.abs(got - ref).max())
    assert np.all(np.isfinite(got))
    assert err <= bar, (err, bar)
    assert torch_dtype("f32") == torch.float32
