"""GPU parity of sdpa_multihead_forward (MultiHead(Q, K, V) = Concat(head_i) W^O,
head_i = Attention(Q W_i^Q, K W_i^K, V W_i^V)) against the fp64 oracle, through
the C ABI.

Bar for this entry point, relative to the largest output magnitude R =
max|oracle|: max |gpu - oracle| <= 2e-2 * R and mean |gpu - oracle| <= 2e-3 * R.
Reason: on top of the attention's own rounding, the GPU path rounds the
projected heads Q W_i^Q, K W_i^K, V W_i^V and the attention output to bf16
(relative error <= 2^-9 each) before the next product, and the result to bf16;
with unit-scale inputs and weights of scale 1/sqrt(fan_in) each stage adds an
error of a few 1e-3 of the output scale, and the largest of millions of outputs
stays well inside 2e-2 * R.
"""
import numpy as np
import pytest
import torch

import head_attention_fwd_amd as sdpa
import oracle
import workloads
from gpu_helpers import announce, require_gpu

pytestmark = pytest.mark.gpu

MAX_REL = 2e-2
MEAN_REL = 2e-3


def assert_mh_parity(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    R = max(float(np.abs(ref).max()), 1e-30)
    err = np.abs(got - ref)
    assert err.max() <= MAX_REL * R, "%s: max err %.3g > %.3g" % (what, err.max(), MAX_REL * R)
    assert err.mean() <= MEAN_REL * R, "%s: mean err %.3g > %.3g" % (what, err.mean(), MEAN_REL * R)


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to(require_gpu())


def run_mh(xq, xkv, ws, h, lengths, causal, self_attn, workspace=None):
    dq = dev_bf16(xq)
    dkv = dq if self_attn else dev_bf16(xkv)
    w = [dev_bf16(a) for a in ws]
    kl = None if lengths is None else torch.as_tensor(np.asarray(lengths, np.int32)).to(require_gpu())
    out = sdpa.multihead(dq, dkv, *w, h, key_lengths=kl, causal=causal, workspace=workspace)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


# (B, Lq, Lk, d_model, h, d_k, d_v, causal, lengths, self-attention)
CASES = [
    (2, 100, 100, 64, 2, 32, 32, False, None, True),
    (2, 100, 100, 64, 2, 32, 32, True, [100, 37], True),
    (3, 70, 130, 128, 4, 32, 32, False, [130, 1, 0], False),    # cross, padding, empty keys
    (1, 300, 300, 256, 2, 128, 128, True, None, True),          # d = 128 heads
    (2, 129, 129, 512, 8, 64, 64, False, [129, 64], True),      # base-model width, ragged rows
    (2, 70, 70, 512, 1, 512, 512, True, [70, 33], True),        # Table 3 row (A): h = 1, d = 512
    (2, 50, 90, 256, 2, 256, 128, False, [90, 5], False),       # wide heads, cross, d_k != d_v
    (1, 50, 50, 96, 3, 16, 32, False, None, True),              # d_k != d_v: generic attention
    (2, 1, 1, 64, 2, 32, 32, False, None, True),                # one position
    (1, 5, 300, 1024, 16, 64, 64, False, None, False),          # few queries, big-model width
    (2, 200, 40, 160, 5, 32, 64, True, [40, 17], False),        # Lq > Lk, causal, ragged columns
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_Lq%d_Lk%d_dm%d_h%d_dk%d_dv%d_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "c" if c[7] else "n", "self" if c[9] else "cross"))
def test_multihead_parity(case):
    B, Lq, Lk, dm, h, dk, dv, causal, lengths, self_attn = case
    xq, xkv, wq, wk, wv, wo, _ = workloads.draw_multihead(
        B, Lq, Lk, dm, h, dk, dv, seed=Lq * 3 + Lk + dm, self_attention=self_attn)
    announce("multihead %s" % (case,))
    got = run_mh(xq, xkv, (wq, wk, wv, wo), h, lengths, causal, self_attn)
    ref = oracle.multihead(xq, xkv, wq, wk, wv, wo, h, key_lengths=lengths, causal=causal)
    assert_mh_parity(got, ref, str(case))


def test_multihead_base_encoder_full():
    """The base-model encoder workload at full size, every output compared."""
    x = workloads.generate("mha_base_encoder_bf16")
    c = x.config
    announce("config %s (full size)" % c.name)
    got = run_mh(x.xq, x.xkv, (x.wq, x.wk, x.wv, x.wo), c.H, x.key_lengths, c.causal, True)
    ref = oracle.multihead(x.xq, x.xkv, x.wq, x.wk, x.wv, x.wo, c.H, key_lengths=x.key_lengths,
                           causal=c.causal)
    assert_mh_parity(got, ref, c.name)


@pytest.mark.parametrize("name", ["mha_big_cross_bf16", "mha_long_causal_bf16"])
def test_multihead_sampled_rows(name):
    """Full-size launches as the benchmark runs them; the oracle recomputes
    sampled output rows of two batch entries."""
    x = workloads.generate(name)
    c = x.config
    announce("config %s (full size)" % name)
    got = run_mh(x.xq, x.xkv, (x.wq, x.wk, x.wv, x.wo), c.H, x.key_lengths, c.causal,
                 c.self_attention)
    rng = np.random.default_rng(5)
    rows = []
    for b in (0, c.B - 1):
        for i in [0, 1, 127, 128, c.Lq // 2, c.Lq - 1] + list(rng.integers(0, c.Lq, size=6)):
            rows.append((b, int(i)))
    rows = np.array(sorted(set(rows)), dtype=np.int64)
    ref = oracle.multihead_rows(x.xq, x.xkv, x.wq, x.wk, x.wv, x.wo, c.H, rows,
                                key_lengths=x.key_lengths, causal=c.causal)
    assert_mh_parity(got[rows[:, 0], rows[:, 1]], ref, name)


def test_multihead_cross_path_equals_self_path_and_workspace_reuse():
    """Keys/values from a copy of the query sequence take the two-launch path and
    give exactly the fused path's result; one workspace serves calls of
    different sizes in stream order."""
    B, L, dm, h, d = 2, 150, 128, 4, 32
    xq, _, wq, wk, wv, wo, _ = workloads.draw_multihead(B, L, L, dm, h, d, d, seed=77)
    dq = dev_bf16(xq)
    w = [dev_bf16(a) for a in (wq, wk, wv, wo)]
    need = sdpa.sdpa_multihead_workspace_bytes(B, L, L, dm, h, d, d, sdpa.SDPA_BF16)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=require_gpu())
    announce("multihead self vs cross path")
    a = sdpa.multihead(dq, dq, *w, h, causal=True, workspace=ws)
    b = sdpa.multihead(dq, dq.clone(), *w, h, causal=True, workspace=ws)
    xs, _, ws2q, ws2k, ws2v, ws2o, _ = workloads.draw_multihead(1, 20, 20, 64, 2, 32, 32, seed=78)
    small = sdpa.multihead(dev_bf16(xs), dev_bf16(xs), *(dev_bf16(t) for t in (ws2q, ws2k, ws2v, ws2o)),
                           2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert_mh_parity(small.float().cpu().numpy(),
                     oracle.multihead(xs, xs, ws2q, ws2k, ws2v, ws2o, 2), "small after large")
    assert_mh_parity(a.float().cpu().numpy(), oracle.multihead(xq, xq, wq, wk, wv, wo, h, causal=True),
                     "large")


def test_multihead_rejects_small_workspace():
    xq, _, wq, wk, wv, wo, _ = workloads.draw_multihead(1, 10, 10, 64, 2, 32, 32, seed=3)
    dq = dev_bf16(xq)
    ws = torch.empty(128, dtype=torch.uint8, device=require_gpu())
    with pytest.raises(sdpa.SdpaError) as e:
        sdpa.multihead(dq, dq, *(dev_bf16(t) for t in (wq, wk, wv, wo)), 2, workspace=ws)
    assert e.value.status == sdpa.SDPA_ERR_WORKSPACE
