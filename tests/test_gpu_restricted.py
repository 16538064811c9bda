"""GPU parity of sdpa_forward_restricted (restricted self-attention: key j legal
for query i only when |i - j| <= radius) against the fp64 oracle, through the C
ABI.

The radii put the neighbourhood's edges at and around the 32-key blocks, the
64-key tiles and the 128-row query tiles, so that the first fully legal tile of
a wave falls on every phase of the three-buffer ring; shapes cover key padding,
the causal mask, Lq != Lk, every matrix-core head size and the generic kernel.
"""
import numpy as np
import pytest
import torch

import head_attention_fwd_amd as sdpa
import oracle
import workloads
from gpu_helpers import announce, assert_parity, require_gpu, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


def run_restricted(q, k, v, radius, lengths=None, causal=False, dtype="bf16"):
    td = torch_dtype(dtype)
    dq, dk, dv = to_dev(q, td), to_dev(k, td), to_dev(v, td)
    kl = None if lengths is None else torch.as_tensor(np.asarray(lengths, np.int32)).to(require_gpu())
    out = sdpa.restricted(dq, dk, dv, radius, key_lengths=kl, causal=causal)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


# (B, H, Lq, Lk, d, causal, lengths, radius)
CASES = [
    (2, 2, 1000, 1000, 64, False, None, 0),
    (2, 2, 1000, 1000, 64, False, None, 1),
    (2, 2, 1000, 1000, 64, False, None, 31),
    (2, 2, 1000, 1000, 64, False, None, 32),
    (2, 2, 1000, 1000, 64, False, None, 63),
    (2, 2, 1000, 1000, 64, False, None, 64),
    (1, 2, 1000, 1000, 64, False, None, 100),
    (1, 2, 1000, 1000, 64, False, None, 127),
    (1, 2, 1000, 1000, 64, False, None, 128),
    (1, 2, 1000, 1000, 64, False, None, 191),
    (1, 2, 1000, 1000, 64, False, None, 255),
    (1, 2, 1000, 1000, 64, False, None, 300),
    (1, 2, 1000, 1000, 64, False, None, 998),       # reaches every key from row 0 or 999 only
    (1, 2, 1000, 1000, 64, True, None, 0),
    (1, 2, 1000, 1000, 64, True, None, 5),
    (1, 2, 1000, 1000, 64, True, None, 64),
    (1, 2, 1000, 1000, 64, True, None, 200),
    (3, 2, 700, 700, 64, False, [700, 333, 0], 50),  # padding inside and before the band
    (3, 2, 700, 700, 64, True, [650, 97, 1], 129),
    (2, 2, 300, 900, 64, False, [900, 400], 80),     # Lq < Lk
    (2, 2, 900, 300, 64, False, [300, 211], 80),     # Lq > Lk: late rows see no key
    (2, 2, 900, 300, 64, True, None, 40),
    (2, 2, 10, 1000, 64, False, [1000, 600], 10),    # radius >= Lq but < Lk: still restricts
    (2, 2, 1000, 10, 64, False, None, 10),           # radius >= Lk but < Lq
    (1, 2, 100, 700, 64, False, None, 150),
    (2, 2, 10, 1000, 16, False, None, 10),
    (1, 3, 1, 1, 64, False, None, 0),
    (1, 1, 65, 65, 64, False, None, 2),
    (2, 2, 1000, 1000, 32, False, [1000, 555], 70),
    (2, 2, 1000, 1000, 32, True, None, 33),
    (2, 2, 1000, 1000, 128, False, [1000, 555], 70),
    (2, 2, 1000, 1000, 128, True, None, 33),
    (1, 2, 1000, 1000, 128, False, None, 16),
    (2, 2, 1000, 1000, 16, False, [1000, 555], 70),
    (2, 2, 1000, 1000, 16, True, None, 129),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%dx%dx%dx%d_d%d_%s_r%d" % (
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "n", c[7]))
def test_restricted_bf16(case):
    B, H, Lq, Lk, d, causal, lengths, radius = case
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, d, d, dtype="bf16", seed=Lq + 7 * radius + d)
    announce("restricted bf16 %s" % (case,))
    got = run_restricted(q, k, v, radius, lengths, causal)
    ref = oracle.attention(q, k, v, key_lengths=lengths, causal=causal, radius=radius)
    assert_parity(got, ref, v, "bf16", str(case))
    if lengths is not None:
        for b, ln in enumerate(lengths):
            # rows whose whole neighbourhood is padding get exactly 0
            for i in range(Lq):
                if max(i - radius, 0) >= ln:
                    assert np.all(got[b, :, i] == 0.0), (b, i)


GENERIC_CASES = [
    (2, 3, 100, 77, 8, 8, True, [77, 5], 3),
    (2, 2, 130, 130, 64, 64, False, None, 20),
    (1, 2, 90, 120, 16, 48, False, [100], 7),
    (1, 1, 200, 200, 128, 40, True, None, 65),
    (1, 2, 150, 150, 512, 512, False, [140], 20),
]
# fp32 for every case; bf16 only where the head sizes have no matrix-core layout
# (bf16 with d_k = d_v in {16, 32, 64, 128} runs the band kernel, covered above)
GENERIC_RUNS = [(c, dt) for c in GENERIC_CASES for dt in ("f32", "bf16")
                if not (dt == "bf16" and c[4] == c[5] and c[4] in (16, 32, 64, 128))]


@pytest.mark.parametrize("case,dtype", GENERIC_RUNS,
                         ids=["x".join(map(str, c[:6])) + "-" + dt for c, dt in GENERIC_RUNS])
def test_restricted_generic_kernel(case, dtype):
    """fp32 inputs, and bf16 head sizes without a matrix-core layout."""
    B, H, Lq, Lk, dk, dv, causal, lengths, radius = case
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, dk, dv, dtype=dtype, seed=Lq * 3 + radius)
    announce("restricted %s %s" % (dtype, case))
    got = run_restricted(q, k, v, radius, lengths, causal, dtype)
    ref = oracle.attention(q, k, v, key_lengths=lengths, causal=causal, radius=radius)
    assert_parity(got, ref, v, dtype, str(case))


def test_restricted_wide_radius_is_forward():
    """radius >= max(Lq, Lk) - 1 restricts nothing: exactly sdpa_forward's result;
    radius = L - 2 (band kernel, one pair excluded per corner) agrees with the
    oracle within the bars."""
    B, H, L = 2, 2, 300
    q, k, v, _ = workloads.draw(B, H, L, L, 64, 64, dtype="bf16", seed=5)
    dq, dk, dv = (to_dev(a, torch.bfloat16) for a in (q, k, v))
    announce("restricted wide radius")
    for causal in (False, True):
        f = sdpa.forward(dq, dk, dv, causal=causal)
        r = sdpa.restricted(dq, dk, dv, L - 1, causal=causal)
        r2 = sdpa.restricted(dq, dk, dv, 10 ** 12, causal=causal)
        b = sdpa.restricted(dq, dk, dv, L - 2, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(f.view(torch.int16), r.view(torch.int16))
        assert torch.equal(f.view(torch.int16), r2.view(torch.int16))
        ref = oracle.attention(q, k, v, causal=causal, radius=L - 2)
        assert_parity(b.float().cpu().numpy(), ref, v, "bf16", "radius L-2")


def test_restricted_negative_radius_raises():
    q, k, v, _ = workloads.draw(1, 1, 8, 8, 64, 64, dtype="bf16", seed=1)
    dq, dk, dv = (to_dev(a, torch.bfloat16) for a in (q, k, v))
    with pytest.raises(sdpa.SdpaError) as e:
        sdpa.restricted(dq, dk, dv, -1)
    assert e.value.status == sdpa.SDPA_ERR_BAD_SHAPE


@pytest.mark.parametrize("name", ["restricted_long_bf16", "restricted_long_causal_bf16"])
def test_restricted_long_sampled_rows(name):
    """The restricted workloads at full size, in the launch configuration the
    benchmark times; the oracle recomputes a sample of rows one by one."""
    x = workloads.generate(name)
    c = x.config
    announce("config %s (full size)" % name)
    got = run_restricted(x.q, x.k, x.v, c.radius, x.key_lengths, c.causal)
    rng = np.random.default_rng(11)
    rows = []
    for b in range(c.B):
        for h in range(c.H):
            for i in [0, 1, 31, 32, 127, 128, c.radius, c.radius + 1, c.Lq - c.radius - 1,
                      c.Lq - 129, c.Lq - 1] + list(rng.integers(0, c.Lq, size=6)):
                if 0 <= i < c.Lq:
                    rows.append((b, h, int(i)))
    rows = np.array(sorted(set(rows)), dtype=np.int64)
    ref, _ = oracle.attention_rows(x.q, x.k, x.v, rows, key_lengths=x.key_lengths,
                                   causal=c.causal, radius=c.radius)
    assert_parity(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref, x.v, "bf16", name)
    assert np.all(np.isfinite(got))
