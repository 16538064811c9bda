"""Seeded random shapes through every attention entry point, element by element
against the fp64 oracle.

The fixed cases of the other GPU tests put tile and block edges where the
kernels' phases change; this sweep draws the rest at random from one seed:
batch, heads, query and key lengths (1 .. a few hundred), head sizes on and off
the matrix-core layouts (including d_k != d_v), the causal mask, per-entry key
lengths (including 0, negative and past Lk), restricted radii, and decode
steps of 1 .. 40 query rows against key caches up to 3000 long.  Every output
starts as NaN, so an element the kernels leave unwritten fails the comparison.
The cases are listed (and so stable) before any GPU call; the ids carry the
shape.
"""
import numpy as np
import pytest
import torch

import head_attention_fwd_amd as sdpa
import oracle
import workloads
from gpu_helpers import announce, assert_parity, require_gpu, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

MFMA_D = (16, 32, 64, 128, 256, 512)


def _lengths(rng, B, Lk):
    kind = rng.integers(0, 4)
    if kind == 0:
        return None
    ln = rng.integers(0, Lk, size=B, endpoint=True)
    if kind == 3:   # a few out-of-range values, clamped to [0, Lk] by both sides
        ln[rng.integers(0, B)] = -int(rng.integers(1, 50))
        ln[rng.integers(0, B)] = Lk + int(rng.integers(1, 50))
    return [int(x) for x in ln]


def _head_sizes(rng, dtype):
    r = rng.random()
    if r < 0.6:
        d = int(rng.choice(MFMA_D if dtype == "bf16" else (8, 16, 64, 100, 128)))
        return d, d
    if r < 0.8:
        d = int(rng.integers(1, 200))
        return d, d
    return int(rng.integers(1, 300)), int(rng.integers(1, 300))


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        entry = ("forward", "forward", "forward", "restricted", "decode")[rng.integers(0, 5)]
        dtype = "f32" if (entry != "decode" and rng.random() < 0.2) else "bf16"
        B, H = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        if entry == "decode":
            d = int(rng.choice((64, 64, 128, 128, 32, 96)))
            dk = dv = d
            Lq = int(rng.integers(1, 41))
            Lk = int(rng.integers(1, 3001))
        else:
            dk, dv = _head_sizes(rng, dtype)
            Lq, Lk = int(rng.integers(1, 400)), int(rng.integers(1, 400))
            if entry == "restricted":
                Lk = Lq if rng.random() < 0.7 else Lk
        # keep the oracle's work per case small (a fraction of a second)
        while B * H * Lq * Lk * (dk + dv) > 6e7 and B * H > 1:
            if B > 1:
                B -= 1
            else:
                H -= 1
        causal = bool(rng.integers(0, 2)) if entry != "decode" else False
        radius = int(rng.integers(0, 300)) if entry == "restricted" else None
        out.append((i, entry, dtype, B, H, Lq, Lk, dk, dv, causal, radius, _lengths(rng, B, Lk)))
    return out


CASES = _cases(160, seed=2026)


def _id(c):
    i, entry, dtype, B, H, Lq, Lk, dk, dv, causal, radius, ln = c
    return "%02d-%s-%s-%dx%dx%dx%d-d%d_%d%s%s%s" % (
        i, entry, dtype, B, H, Lq, Lk, dk, dv, "-c" if causal else "",
        "" if radius is None else "-w%d" % radius, "" if ln is None else "-pad")


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_fuzz_parity(case):
    i, entry, dtype, B, H, Lq, Lk, dk, dv, causal, radius, lengths = case
    announce("fuzz %s" % _id(case))
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, dk, dv, dtype=dtype, seed=9000 + i)
    td = torch_dtype(dtype)
    dev = require_gpu()
    dq, dk_, dv_ = to_dev(q, td), to_dev(k, td), to_dev(v, td)
    kl = None if lengths is None else torch.as_tensor(np.asarray(lengths, np.int32)).to(dev)
    out = torch.full((B, H, Lq, dv), float("nan"), dtype=td, device=dev)
    if entry == "forward":
        sdpa.forward(dq, dk_, dv_, key_lengths=kl, causal=causal, out=out)
    elif entry == "restricted":
        sdpa.restricted(dq, dk_, dv_, radius, key_lengths=kl, causal=causal, out=out)
    else:
        sdpa.decode(dq, dk_, dv_, key_lengths=kl, out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = oracle.attention(q, k, v, key_lengths=lengths, causal=causal, radius=radius)
    assert_parity(got, ref, v, dtype, _id(case))
