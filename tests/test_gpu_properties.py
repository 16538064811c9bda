"""GPU checks of what the pages and the mathematics fix, through the C ABI.

The printed worked examples run through the fp32 kernel (d_k = 1); the d_k = 64
scale pin runs through both kernels; exact zeros, exact copies and robustness
to padding contents are checked bit for bit where the arithmetic allows it.
"""
import math

import numpy as np
import pytest
import torch

import head_attention_fwd_amd as sdpa
import oracle
import pins
import workloads
from gpu_helpers import announce, assert_parity, require_gpu, run, to_dev

pytestmark = pytest.mark.gpu


def test_worked_example_fp32():
    """Page "Arquitectura Transformer", "Cómo hacerlo": 3, and 2 with the second key
    forbidden (by padding and by the causal mask)."""
    g = pins.read_golden("transformer_worked_example.txt")
    q = np.array(g["query"]).reshape(1, 1, 1, 1)
    k = np.array(g["keys"]).reshape(1, 1, 2, 1)
    v = np.array(g["values"]).reshape(1, 1, 2, 1)
    announce("worked example fp32")
    assert abs(run(q, k, v, None, False, "f32")[0, 0, 0, 0] - g["output"][0]) <= 1e-6
    assert abs(run(q, k, v, [1], False, "f32")[0, 0, 0, 0] - g["masked_output"][0]) <= 1e-6
    q2 = np.repeat(q, 2, axis=2)
    o = run(q2, k, v, None, True, "f32")
    assert abs(o[0, 0, 0, 0] - g["masked_output"][0]) <= 1e-6
    assert abs(o[0, 0, 1, 0] - g["output"][0]) <= 1e-6


def test_toy_rows_fp32():
    """Page "Self-Attention คืออะไร (แบบจับต้องได้)", Fig. 2: 30.2, 31.6; causal row 0: 10."""
    g = pins.read_golden("self_attention_toy.txt")
    v = np.array(g["values"]).reshape(1, 1, 5, 1)
    q = np.ones((1, 1, 5, 1))
    for wk, ok in (("row0_weights", "row0_output"), ("row1_weights", "row1_output")):
        k = np.log(np.array(g[wk])).reshape(1, 1, 5, 1)
        announce("toy %s" % wk)
        assert abs(run(q, k, v, None, False, "f32")[0, 0, 0, 0] - g[ok][0]) <= 1e-4
    k = np.log(np.array(g["row0_weights"])).reshape(1, 1, 5, 1)
    assert run(q, k, v, None, True, "f32")[0, 0, 0, 0] == g["row0_causal_output"][0]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scale_pin_dk64(dtype):
    """d_k = 64 divides the scores by 8: q = e0, k1 = 8 ln3 e0, k2 = 0, v = (2, 6) -> 3.

    bf16 rounds 8 ln 3, so the oracle on the rounded inputs gives the expected value
    (2.9978).  The output itself is rounded to bf16, whose spacing at 3 is 2^-6: the
    bar for this single value is one bf16 spacing, not the mean bar of the
    configurations (which is sized for outputs of magnitude ~1)."""
    q = np.zeros((1, 1, 1, 64), np.float32); q[..., 0] = 1
    k = np.zeros((1, 1, 2, 64), np.float32); k[0, 0, 0, 0] = 8 * math.log(3)
    if dtype == "bf16":
        k = workloads.round_to_bf16(k)
    v = np.zeros((1, 1, 2, 64), np.float32); v[0, 0, 0] = 2; v[0, 0, 1] = 6
    announce("scale pin %s" % dtype)
    got = run(q, k, v, None, False, dtype)
    ref = oracle.attention(q, k, v)
    if dtype == "f32":
        assert_parity(got, ref, v, dtype, "scale pin")
        assert abs(got[0, 0, 0, 0] - 3.0) <= 1e-5
    else:
        assert np.max(np.abs(got - ref)) <= 2.0 ** -6
        assert abs(got[0, 0, 0, 0] - 3.0) <= 2.0 ** -6 + 3e-3


@pytest.mark.parametrize("causal", [False, True])
def test_identity_values_read_out_weights(causal):
    """V = I (Lk = d_v = 64) makes O = P: rows sum to ~1, illegal weights exactly 0."""
    B, H, Lq, Lk = 2, 2, 96, 64
    q, k, _, _ = workloads.draw(B, H, Lq, Lk, 64, 64, dtype="bf16", seed=31)
    v = np.broadcast_to(np.eye(64, dtype=np.float32), (B, H, 64, 64)).copy()
    lengths = [64, 37]
    announce("identity V causal=%d" % causal)
    got = run(q, k, v, lengths, causal, "bf16")
    _, P, _ = oracle.attention(q, k, v, key_lengths=lengths, causal=causal, return_weights=True)
    assert_parity(got, P, v, "bf16", "O = P")
    assert np.max(np.abs(got.sum(-1) - 1.0)) <= 0.02
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    for b, lb in enumerate(lengths):
        illegal = (j >= lb) | ((j > i) if causal else np.zeros_like(j > i))
        assert np.all(got[b][:, illegal] == 0.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_causal_row0_is_first_value_exactly(dtype):
    q, k, v, _ = workloads.draw(2, 4, 130, 130, 64, 64, dtype=dtype, seed=41)
    announce("causal row 0 %s" % dtype)
    got = run(q, k, v, None, True, dtype)
    assert np.array_equal(got[:, :, 0], v[:, :, 0].astype(np.float64))


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 32), ("bf16", 16), ("bf16", 128),
                                     ("f32", 64)])
def test_padding_contents_do_not_matter(dtype, d):
    """Key/value rows j >= len_b filled with NaN and huge values change nothing."""
    B, H, Lq, Lk = 3, 2, 150, 200
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, d, d, dtype=dtype, seed=51)
    lengths = [200, 131, 64]
    announce("padding garbage %s d=%d" % (dtype, d))
    clean = run(q, k, v, lengths, False, dtype)
    k2, v2 = k.copy(), v.copy()
    for b, lb in enumerate(lengths):
        k2[b, :, lb:] = np.nan
        v2[b, :, lb:] = np.nan
        k2[b, :, lb + 1::3] = 3e38
        v2[b, :, lb + 1::3] = -3e38
    dirty = run(q, k2, v2, lengths, False, dtype)
    assert np.array_equal(clean, dirty)


def test_causal_locality_gpu():
    """Changing keys/values after position i (finite values) leaves row i unchanged."""
    q, k, v, _ = workloads.draw(1, 2, 256, 256, 64, 64, dtype="bf16", seed=61)
    base = run(q, k, v, None, True, "bf16")
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 100:] = workloads.round_to_bf16(np.random.default_rng(1).standard_normal(
        k2[:, :, 100:].shape).astype(np.float32) * 4)
    v2[:, :, 100:] = 7.0
    announce("causal locality")
    new = run(q, k2, v2, None, True, "bf16")
    assert np.array_equal(base[:, :, :100], new[:, :, :100])


@pytest.mark.parametrize("name", ["base_decoder_causal_bf16", "big_cross_bf16"])
def test_deterministic_and_fully_written(name):
    x = workloads.generate(name)
    c = x.config
    dev = require_gpu()
    dq, dk, dv = (to_dev(a, torch.bfloat16) for a in (x.q, x.k, x.v))
    kl = torch.as_tensor(x.key_lengths).to(dev)
    announce("determinism %s" % name)
    out1 = torch.full((c.B, c.H, c.Lq, c.d_v), float("nan"), dtype=torch.bfloat16, device=dev)
    out2 = torch.full_like(out1, float("nan"))
    sdpa.forward(dq, dk, dv, key_lengths=kl, causal=c.causal, out=out1)
    sdpa.forward(dq, dk, dv, key_lengths=kl, causal=c.causal, out=out2)
    torch.cuda.synchronize()
    assert not torch.isnan(out1).any()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 8), ("bf16", 16), ("bf16", 128)])
def test_no_legal_key_gives_zero(dtype, d):
    q, k, v, _ = workloads.draw(3, 2, 70, 40, d, d, dtype=dtype, seed=71)
    announce("zero-length rows %s d=%d" % (dtype, d))
    got = run(q, k, v, [0, 40, -3], True, dtype)
    assert np.all(got[0] == 0.0) and np.all(got[2] == 0.0)
    ref = oracle.attention(q, k, v, key_lengths=[0, 40, -3], causal=True)
    assert_parity(got, ref, v, dtype, "zero-length rows")


def test_zero_keys_and_empty_calls():
    dev = require_gpu()
    q = torch.randn(2, 2, 33, 64, device=dev).to(torch.bfloat16)
    k = torch.empty(2, 2, 0, 64, device=dev, dtype=torch.bfloat16)
    out = torch.full((2, 2, 33, 64), float("nan"), device=dev, dtype=torch.bfloat16)
    announce("Lk = 0")
    sdpa.forward(q, k, k, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    e = torch.empty(0, 2, 5, 64, device=dev, dtype=torch.bfloat16)
    assert sdpa.forward(e, e, e).shape == (0, 2, 5, 64)
    # decode steps against an empty cache: the single-row kernel (Lq = 1) and
    # the matrix-core decode kernels (Lq = 3) also give 0
    for lq, d in ((1, 64), (1, 128), (3, 64)):
        q = torch.randn(2, 2, lq, d, device=dev).to(torch.bfloat16)
        k = torch.empty(2, 2, 0, d, device=dev, dtype=torch.bfloat16)
        out = torch.full((2, 2, lq, d), float("nan"), device=dev, dtype=torch.bfloat16)
        announce("decode Lk = 0, Lq = %d, d = %d" % (lq, d))
        sdpa.decode(q, k, k, out=out)
        torch.cuda.synchronize()
        assert torch.all(out == 0)


def test_error_paths_raise():
    dev = require_gpu()
    q = torch.zeros(1, 1, 4, 520, device=dev, dtype=torch.bfloat16)   # head size above 512
    with pytest.raises(sdpa.SdpaError) as ei:
        sdpa.forward(q, q, q)
    assert ei.value.status == sdpa.SDPA_ERR_UNSUPPORTED
    q = torch.zeros(1, 1, 4, 64, device=dev, dtype=torch.bfloat16)
    with pytest.raises(sdpa.SdpaError) as ei:
        sdpa.forward(q, q, q, out=q)
    assert ei.value.status == sdpa.SDPA_ERR_ALIAS


def test_stream_ordering_on_side_stream():
    """The kernel runs on the caller's current stream."""
    dev = require_gpu()
    x = workloads.generate("base_encoder_bf16")
    dq, dk, dv = (to_dev(a, torch.bfloat16) for a in (x.q, x.k, x.v))
    kl = torch.as_tensor(x.key_lengths).to(dev)
    ref = sdpa.forward(dq, dk, dv, key_lengths=kl)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    announce("side stream")
    with torch.cuda.stream(s):
        out = sdpa.forward(dq, dk, dv, key_lengths=kl)
    s.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("causal", [False, True])
def test_lds_left_by_earlier_launches_never_reaches_result(causal):
    """Launches whose K/V are all NaN (and an fp32 launch) leave NaN bit patterns in
    LDS; a following ragged launch must still match the oracle exactly as it does
    from a clean state: rows past the key length are zero-filled, and no operand
    is read before its copy has landed."""
    dev = require_gpu()
    B, H, Lq, Lk = 16, 4, 256, 256
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, 64, 64, dtype="bf16", seed=81)
    lengths = [100, 130, 200, 250, 256, 64, 65, 191] * 2
    ref = oracle.attention(q, k, v, key_lengths=lengths, causal=causal)
    nan = torch.full((B, H, Lk, 64), float("nan"), device=dev, dtype=torch.bfloat16)
    zq = torch.zeros((B, H, Lq, 64), device=dev, dtype=torch.bfloat16)
    t = workloads.generate("tiny_causal_f32")
    tq, tk, tv = (to_dev(a, torch.float32) for a in (t.q, t.k, t.v))
    dq, dk, dv = (to_dev(a, torch.bfloat16) for a in (q, k, v))
    kl = torch.as_tensor(np.asarray(lengths, np.int32)).to(dev)
    announce("stale LDS causal=%d" % causal)
    first = None
    for rep in range(4):
        sdpa.forward(zq, nan, nan)
        sdpa.forward(tq, tk, tv, causal=True)
        out = sdpa.forward(dq, dk, dv, key_lengths=kl, causal=causal)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got)), "repetition %d" % rep
        if first is None:
            first = got
            assert_parity(got, ref, v, "bf16", "after NaN-filled launches")
        else:
            assert np.array_equal(got, first)


def test_restricted_and_multihead_deterministic_and_fully_written():
    """The restricted and multi-head entry points: run to run bit for bit, every
    output element written (outputs pre-filled with NaN), padding contents
    irrelevant to the restricted path."""
    dev = require_gpu()
    q, k, v, _ = workloads.draw(2, 2, 500, 500, 64, 64, dtype="bf16", seed=71)
    lengths = [500, 321]
    dq, dk, dv = (to_dev(a, torch.bfloat16) for a in (q, k, v))
    kl = torch.as_tensor(np.asarray(lengths, np.int32)).to(dev)
    announce("restricted determinism")
    o1 = torch.full((2, 2, 500, 64), float("nan"), dtype=torch.bfloat16, device=dev)
    o2 = torch.full_like(o1, float("nan"))
    sdpa.restricted(dq, dk, dv, 40, key_lengths=kl, causal=True, out=o1)
    k2, v2 = k.copy(), v.copy()
    k2[1, :, 321:] = np.nan
    v2[1, :, 321:] = np.nan
    sdpa.restricted(dq, to_dev(k2, torch.bfloat16), to_dev(v2, torch.bfloat16), 40, key_lengths=kl,
                    causal=True, out=o2)
    torch.cuda.synchronize()
    assert not torch.isnan(o1).any()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))

    xq, _, wq, wk, wv, wo, _ = workloads.draw_multihead(2, 130, 130, 128, 4, 32, 32, seed=72)
    dx = to_dev(xq, torch.bfloat16)
    w = [to_dev(a, torch.bfloat16) for a in (wq, wk, wv, wo)]
    announce("multihead determinism")
    m1 = torch.full((2, 130, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    m2 = torch.full_like(m1, float("nan"))
    sdpa.multihead(dx, dx, *w, 4, causal=True, out=m1)
    sdpa.multihead(dx, dx, *w, 4, causal=True, out=m2)
    torch.cuda.synchronize()
    assert not torch.isnan(m1).any()
    assert torch.equal(m1.view(torch.int16), m2.view(torch.int16))
