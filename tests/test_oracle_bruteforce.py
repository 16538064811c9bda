"""Exhaustive tiny cases: the oracle against the pure-Python brute force.

Covers every key length 0..Lk (plus one beyond each end), both mask modes,
Lq < Lk, Lq = Lk and Lq > Lk, and d_k != d_v.
"""
import itertools

import numpy as np
import pytest

import bruteforce
import oracle


@pytest.mark.parametrize("Lq,Lk", [(1, 1), (1, 4), (3, 2), (4, 4), (6, 5), (2, 6)])
@pytest.mark.parametrize("dk,dv", [(1, 1), (3, 2), (4, 4)])
def test_exhaustive_tiny(Lq, Lk, dk, dv):
    rng = np.random.default_rng(1000 * Lq + 100 * Lk + 10 * dk + dv)
    B, H = 2, 2
    q = rng.standard_normal((B, H, Lq, dk))
    k = rng.standard_normal((B, H, Lk, dk))
    v = rng.standard_normal((B, H, Lk, dv))
    lengths = list(range(-1, Lk + 2))
    for causal, (l0, l1) in itertools.product((False, True), zip(lengths, reversed(lengths))):
        kl = [l0, l1]
        got = oracle.attention(q, k, v, key_lengths=kl, causal=causal)
        ref = np.array(bruteforce.attention(q, k, v, kl, causal))
        assert np.max(np.abs(got - ref)) <= 1e-12, (causal, kl)
    got = oracle.attention(q, k, v, causal=True)
    ref = np.array(bruteforce.attention(q, k, v, None, True))
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("Lq,Lk", [(1, 1), (1, 4), (3, 2), (4, 4), (6, 5), (2, 6), (7, 7)])
def test_exhaustive_tiny_restricted(Lq, Lk):
    """Every radius from 0 to beyond both lengths, with and without the causal
    mask and with every key length."""
    rng = np.random.default_rng(7000 + 10 * Lq + Lk)
    B, H, dk, dv = 2, 1, 3, 2
    q = rng.standard_normal((B, H, Lq, dk))
    k = rng.standard_normal((B, H, Lk, dk))
    v = rng.standard_normal((B, H, Lk, dv))
    lengths = list(range(0, Lk + 1))
    for radius in range(0, max(Lq, Lk) + 1):
        for causal, (l0, l1) in itertools.product((False, True), zip(lengths, reversed(lengths))):
            kl = [l0, l1]
            got = oracle.attention(q, k, v, key_lengths=kl, causal=causal, radius=radius)
            ref = np.array(bruteforce.attention(q, k, v, kl, causal, radius))
            assert np.max(np.abs(got - ref)) <= 1e-12, (radius, causal, kl)


@pytest.mark.parametrize("B,Lq,Lk,dm,h,dk,dv", [(1, 3, 3, 4, 2, 2, 2), (2, 4, 5, 6, 3, 2, 1),
                                                 (1, 1, 4, 3, 1, 3, 3), (2, 5, 2, 4, 2, 1, 3)])
def test_multihead_tiny(B, Lq, Lk, dm, h, dk, dv):
    """Multi-head attention against the plain-loop brute force, self- and
    cross-attention, every key length, with and without the causal mask."""
    rng = np.random.default_rng(900 + 10 * Lq + Lk)
    xq = rng.standard_normal((B, Lq, dm))
    xkv = rng.standard_normal((B, Lk, dm))
    ws = [rng.standard_normal(s) for s in ((dm, h * dk), (dm, h * dk), (dm, h * dv), (h * dv, dm))]
    for causal in (False, True):
        for ln in [None] + [[l] * B for l in range(0, Lk + 1)]:
            got = oracle.multihead(xq, xkv, *ws, h, key_lengths=ln, causal=causal)
            ref = np.array(bruteforce.multihead(xq, xkv, *ws, h, ln, causal))
            assert np.max(np.abs(got - ref)) <= 1e-10 * max(1.0, np.abs(ref).max()), (causal, ln)
    if Lq == Lk:
        got = oracle.multihead(xq, xq, *ws, h, causal=True)
        ref = np.array(bruteforce.multihead(xq, xq, *ws, h, None, True))
        assert np.max(np.abs(got - ref)) <= 1e-10 * max(1.0, np.abs(ref).max())
