"""A seeded sweep of shapes, head sizes, masks and dtypes against the fp64 oracle.

Every case draws B, h, Lq, Lk, d_k, d_v, the dtype, the causal flag, the key
lengths (some outside [0, Lk], which both sides clamp) and, for a fifth of the
cases, a restricted-attention radius, from one fixed generator, so the list is
the same on every run.  Head sizes cover the matrix-core sizes (16, 32, 64,
128), the generic kernel (other sizes up to 128, d_k != d_v) and the wide kernel
(129 .. 512).  Sizes stay small enough for the oracle to finish in well under a
second per case.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import announce, assert_parity, run, require_gpu, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

D_SIZES = [8, 16, 24, 32, 48, 64, 96, 128, 136, 200, 256, 384, 512]


def _cases(n=48, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 4))
        H = int(rng.integers(1, 4))
        Lq = int(rng.integers(1, 300))
        Lk = 0 if rng.random() < 0.05 else int(rng.integers(1, 400))
        dk = int(rng.choice(D_SIZES))
        dv = dk if rng.random() < 0.7 else int(rng.choice(D_SIZES))
        dtype = "bf16" if rng.random() < 0.8 else "f32"
        causal = bool(rng.random() < 0.5)
        lengths = None if rng.random() < 0.4 else [int(x) for x in rng.integers(-2, Lk + 3, size=B)]
        radius = int(rng.integers(0, 300)) if rng.random() < 0.2 else None
        # keep the oracle's work small
        while B * H * Lq * max(Lk, 1) * (dk + dv) > 4e8:
            Lq = max(1, Lq // 2)
        out.append((B, H, Lq, Lk, dk, dv, dtype, causal, lengths, radius))
    return out


CASES = _cases()


def _id(c):
    B, H, Lq, Lk, dk, dv, dtype, causal, lengths, radius = c
    return "%dx%dx%dx%d_d%d-%d_%s%s%s%s" % (B, H, Lq, Lk, dk, dv, dtype, "_c" if causal else "",
                                           "_len" if lengths is not None else "",
                                           "" if radius is None else "_r%d" % radius)


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_sweep(case):
    import torch
    import head_attention_fwd_amd as sdpa
    B, H, Lq, Lk, dk, dv, dtype, causal, lengths, radius = case
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, dk, dv, dtype=dtype, seed=Lq * 131 + Lk * 7 + dk)
    announce("sweep %s" % _id(case))
    if radius is None:
        got = run(q, k, v, lengths, causal, dtype)
    else:
        td = torch_dtype(dtype)
        dev = require_gpu()
        kl = None if lengths is None else torch.as_tensor(np.asarray(lengths, np.int32)).to(dev)
        out = sdpa.restricted(to_dev(q, td), to_dev(k, td), to_dev(v, td), radius, key_lengths=kl,
                              causal=causal)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
    ref = oracle.attention(q, k, v, key_lengths=lengths, causal=causal, radius=radius)
    assert_parity(got, ref, v, dtype, _id(case))


def _balanced_cases(n=24, seed=20261203):
    """Shapes that take the balanced work order of the matrix-core kernel: bf16,
    d_k = d_v in {16, 32, 64, 128}, per-entry key lengths, at most 64 entries and
    a multiple of 8 (entry, head) pairs, few enough query tiles to be resident at
    once (the launcher decides; shapes past its limits take the fixed order and
    are checked the same way)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        H = int(rng.choice([1, 2, 4, 8, 16]))
        step = 8 // math.gcd(8, H)          # B * H a multiple of 8
        B = int(rng.integers(1, 65))
        B = max(step, B - B % step)
        Lq = int(rng.integers(1, 400))
        Lk = int(rng.integers(1, 700))
        d = int(rng.choice([16, 32, 64, 128]))
        causal = bool(rng.random() < 0.5)
        lengths = [int(x) for x in rng.integers(-2, Lk + 3, size=B)]
        while B * H * Lq * Lk * 2 * d > 4e8:
            Lq = max(1, Lq // 2)
        out.append((B, H, Lq, Lk, d, causal, lengths))
    return out


BALANCED_CASES = _balanced_cases()


@pytest.mark.parametrize("case", BALANCED_CASES,
                         ids=lambda c: "%dx%dx%dx%d_d%d%s" % (c[0], c[1], c[2], c[3], c[4], "_c" if c[5] else ""))
def test_sweep_balanced(case):
    B, H, Lq, Lk, d, causal, lengths = case
    assert (B * H) % 8 == 0 and B <= 64
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, d, d, dtype="bf16", seed=Lq * 17 + Lk + d)
    announce("balanced sweep %s" % (case[:6],))
    got = run(q, k, v, lengths, causal, "bf16", fill=float("nan"))
    ref = oracle.attention(q, k, v, key_lengths=lengths, causal=causal)
    assert_parity(got, ref, v, "bf16", "balanced sweep %s" % (case[:6],))
