"""The seeded input generator: shapes, determinism, rounding and score scale."""
import numpy as np
import pytest
import torch

import workloads


def test_round_to_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 0.0, -0.0,
                                  65504.0, 1e-40, 3.0e38], dtype=np.float32)])
    ours = workloads.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("name", ["tiny_causal_f32", "base_encoder_bf16", "big_cross_bf16"])
def test_generate_shapes_and_determinism(name):
    a = workloads.generate(name)
    b = workloads.generate(name)
    c = a.config
    assert a.q.shape == (c.B, c.H, c.Lq, c.d_k) and a.q.dtype == np.float32
    assert a.k.shape == (c.B, c.H, c.Lk, c.d_k)
    assert a.v.shape == (c.B, c.H, c.Lk, c.d_v)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        assert np.array_equal(x, y)
    if c.key_len_range is None:
        assert a.key_lengths is None
    else:
        lo, hi = c.key_len_range
        assert a.key_lengths.dtype == np.int32 and a.key_lengths.shape == (c.B,)
        assert a.key_lengths.min() >= lo and a.key_lengths.max() <= hi
    if c.dtype == "bf16":
        assert np.array_equal(workloads.round_to_bf16(a.q), a.q)


def test_score_variance_matches_footnote():
    """Page "Attention Is All You Need/paper/es", §3.2.1 footnote 1: for independent
    unit-variance components q.k has mean 0 and variance d_k."""
    q, k, _, _ = workloads.draw(1, 4, 256, 256, 64, 64, dtype="f32", seed=5)
    s = np.einsum("bhid,bhjd->bhij", q.astype(np.float64), k.astype(np.float64))
    assert abs(s.mean()) < 0.1
    assert abs(s.var() / 64.0 - 1.0) < 0.05


def test_pair_count_bruteforce():
    from head_attention_fwd_amd import perfmodel
    for Lq in range(0, 6):
        for Lk in range(1, 6):
            for lb in range(-1, 8):
                for causal in (False, True):
                    ref = sum(1 for i in range(Lq) for j in range(Lk)
                              if j < min(max(lb, 0), Lk) and (not causal or j <= i))
                    assert perfmodel.pair_count(1, 1, Lq, Lk, causal, [lb]) == ref
    assert perfmodel.flops(4, 16, 8192, 8192, 64, 64, True) == 549822922752
