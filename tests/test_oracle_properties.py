"""Property-based checks of the oracle over random shapes (hypothesis)."""
import numpy as np
from hypothesis import given, settings, strategies as st

import bruteforce
import oracle

shapes = st.tuples(st.integers(1, 2), st.integers(1, 3), st.integers(1, 6), st.integers(1, 7),
                   st.integers(1, 5), st.integers(1, 5))


@settings(max_examples=40, deadline=None)
@given(shapes, st.integers(0, 2**31 - 1), st.booleans(), st.data())
def test_against_bruteforce(shape, seed, causal, data):
    B, H, Lq, Lk, dk, dv = shape
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Lq, dk))
    k = rng.standard_normal((B, H, Lk, dk))
    v = rng.standard_normal((B, H, Lk, dv))
    kl = data.draw(st.one_of(st.none(), st.lists(st.integers(-2, Lk + 2), min_size=B, max_size=B)))
    got = oracle.attention(q, k, v, key_lengths=kl, causal=causal)
    ref = np.array(bruteforce.attention(q, k, v, kl, causal))
    assert np.max(np.abs(got - ref)) <= 1e-12


@settings(max_examples=30, deadline=None)
@given(shapes, st.integers(0, 2**31 - 1), st.booleans())
def test_weights_are_a_distribution(shape, seed, causal):
    B, H, Lq, Lk, dk, dv = shape
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Lq, dk)) * 3
    k = rng.standard_normal((B, H, Lk, dk)) * 3
    v = rng.standard_normal((B, H, Lk, dv))
    O, P, L = oracle.attention(q, k, v, causal=causal, return_weights=True)
    assert np.all(P >= 0)
    # with no padding every row has key 0 legal (top-left causal alignment)
    assert np.max(np.abs(P.sum(-1) - 1)) <= 1e-12
    if causal:
        i = np.arange(Lq)[:, None]
        j = np.arange(Lk)[None, :]
        assert np.all(P[..., j > i] == 0.0)
    # the output is a convex combination of values: inside their per-column range
    lo = v.min(axis=2, keepdims=True) - 1e-12
    hi = v.max(axis=2, keepdims=True) + 1e-12
    assert np.all((O >= lo) & (O <= hi))
    # LSE is the log of the softmax denominator of the scaled scores
    s = np.einsum("bhid,bhjd->bhij", q, k) / np.sqrt(dk)
    if causal:
        s = np.where(np.arange(Lk)[None, :] > np.arange(Lq)[:, None], -np.inf, s)
    assert np.allclose(np.exp(s - L[..., None]), P, rtol=1e-12, atol=1e-15)


@settings(max_examples=20, deadline=None)
@given(st.integers(0, 2**31 - 1), st.floats(-50, 50))
def test_shift_of_all_scores(seed, c):
    """Adding c * sqrt(d_k) * e_0-aligned offsets: with q_0 = 1 for every query and a
    constant added to every key's first component, every score moves by the same
    amount for a row, so the output is unchanged (softmax shift invariance)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 2, 4, 3)); q[..., 0] = 1.0
    k = rng.standard_normal((1, 2, 5, 3))
    v = rng.standard_normal((1, 2, 5, 2))
    k2 = k.copy(); k2[..., 0] += c
    a = oracle.attention(q, k, v, causal=True)
    b = oracle.attention(q, k2, v, causal=True)
    assert np.max(np.abs(a - b)) <= 1e-11
