"""Shared helpers of the GPU tests: device transfer and the parity bars.

Parity bars (stated for this method; a bf16 result is compared with the fp64
oracle evaluated on the same bf16-rounded inputs):
  fp32 inputs: max |gpu - oracle| <= 1e-5;
  bf16 inputs: max |gpu - oracle| <= 2e-2 * max|V| and mean |gpu - oracle| <= 2e-3.
"""
import sys

import numpy as np
import torch

import head_attention_fwd_amd as sdpa

F32_MAX_ABS = 1e-5
BF16_MAX_ABS_REL = 2e-2
BF16_MEAN_ABS = 2e-3


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def announce(msg):
    """Name the case before a GPU step, flushed, so a crash log says what ran."""
    sys.stdout.write("[gpu case] %s\n" % msg)
    sys.stdout.flush()


def to_dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(dtype).to(require_gpu())


def torch_dtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def run(q, k, v, key_lengths=None, causal=False, dtype="bf16", fill=None):
    """Upload, run sdpa.forward, synchronize, return float64 numpy output.

    fill: if given, the output buffer is allocated here and filled with this
    value first (NaN shows any element the kernel leaves unwritten)."""
    td = torch_dtype(dtype)
    dq, dk, dv = to_dev(q, td), to_dev(k, td), to_dev(v, td)
    kl = None if key_lengths is None else torch.as_tensor(
        np.asarray(key_lengths, dtype=np.int32)).to(require_gpu())
    out = None
    if fill is not None:
        B, H, Lq, _ = q.shape
        out = torch.full((B, H, Lq, v.shape[3]), fill, dtype=td, device=require_gpu())
    out = sdpa.forward(dq, dk, dv, key_lengths=kl, causal=causal, out=out)
    torch.cuda.synchronize()
    return out.to(torch.float32).cpu().numpy().astype(np.float64)


def assert_parity(got, ref, v, dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    err = np.abs(got - ref)
    max_err = float(err.max()) if err.size else 0.0
    if dtype == "f32":
        assert max_err <= F32_MAX_ABS, "%s: max abs err %.3g > %.1g" % (what, max_err, F32_MAX_ABS)
    else:
        vmax = float(np.abs(v).max()) if np.size(v) else 0.0
        mean_err = float(err.mean()) if err.size else 0.0
        assert max_err <= BF16_MAX_ABS_REL * vmax, \
            "%s: max abs err %.3g > %.3g" % (what, max_err, BF16_MAX_ABS_REL * vmax)
        assert mean_err <= BF16_MEAN_ABS, "%s: mean abs err %.3g > %.1g" % (what, mean_err,
                                                                          BF16_MEAN_ABS)
    return max_err
