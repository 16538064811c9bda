"""The entry points under HIP graph capture: each call captured once on a side
stream (default priority), the graph replayed several times with eager work and
synchronisations in between, every replay compared bit for bit with the eager
result.  The library records only kernel launches (no memsets, no allocations),
so the replays must reproduce the eager output exactly."""
import numpy as np
import pytest
import torch

import head_attention_fwd_amd as sdpa
import workloads
from gpu_helpers import announce, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _bf(a):
    return to_dev(a, torch.bfloat16)


def _check_graph(call, out):
    dev = require_gpu()
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), "replay %d differs" % rep
        call()          # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))


@pytest.mark.parametrize("name", ["base_decoder_causal_bf16", "big_cross_bf16"])
def test_forward_graph_replays(name):
    x = workloads.generate(name)
    c = x.config
    dev = require_gpu()
    q, k, v = _bf(x.q), _bf(x.k), _bf(x.v)
    kl = torch.as_tensor(x.key_lengths).to(dev)
    out = torch.empty((c.B, c.H, c.Lq, c.d_v), dtype=torch.bfloat16, device=dev)
    announce("graph forward %s" % name)
    _check_graph(lambda: sdpa.forward(q, k, v, key_lengths=kl, causal=c.causal, out=out), out)


def test_decode_restricted_multihead_graph_replays():
    dev = require_gpu()
    q, k, v, _ = workloads.draw(4, 8, 1, 3000, 64, 64, dtype="bf16", seed=91)
    dq, dk, dv = _bf(q), _bf(k), _bf(v)
    kl = torch.as_tensor(np.array([3000, 17, 1500, 0], np.int32)).to(dev)
    ws = torch.empty(sdpa.sdpa_decode_workspace_bytes(4, 8, 1, 3000, 64, 64, sdpa.SDPA_BF16),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((4, 8, 1, 64), dtype=torch.bfloat16, device=dev)
    announce("graph decode")
    _check_graph(lambda: sdpa.decode(dq, dk, dv, key_lengths=kl, out=out, workspace=ws), out)

    q, k, v, _ = workloads.draw(2, 2, 500, 500, 64, 64, dtype="bf16", seed=92)
    dq, dk, dv = _bf(q), _bf(k), _bf(v)
    out = torch.empty((2, 2, 500, 64), dtype=torch.bfloat16, device=dev)
    announce("graph restricted")
    _check_graph(lambda: sdpa.restricted(dq, dk, dv, 40, causal=True, out=out), out)

    xq, xkv, wq, wk, wv, wo, _ = workloads.draw_multihead(2, 100, 100, 128, 4, 32, 32, seed=93)
    t = [_bf(a) for a in (xq, wq, wk, wv, wo)]
    out = torch.empty((2, 100, 128), dtype=torch.bfloat16, device=dev)
    wsm = torch.empty(sdpa.sdpa_multihead_workspace_bytes(2, 100, 100, 128, 4, 32, 32, sdpa.SDPA_BF16),
                      dtype=torch.uint8, device=dev)
    announce("graph multihead")
    _check_graph(lambda: sdpa.multihead(t[0], t[0], t[1], t[2], t[3], t[4], 4, causal=True, out=out,
                                        workspace=wsm), out)
