"""A second, independent formulation of attention for tiny inputs (pure Python).

Used only to pin the oracle.  It differs from the oracle on purpose:
  * illegal keys are left out of the sums instead of being scored -inf;
  * no maximum is subtracted before exponentiating (inputs are tiny and finite);
  * the normalisation divides the weighted sum once, after summing, and every
    sum is an exactly rounded ``math.fsum``.

Definition followed: page "Attention Is All You Need/paper/es", §3.2.1,
Eq. (1) -- dot product of the query with each key, divided by sqrt(d_k),
softmax over keys, weighted sum of the values; §3.2.3 -- a decoder position
may use every position up to and including its own; §4 and Table 1 -- restricted
self-attention looks only at a neighbourhood centred on the output position
(here: the positions within ``radius`` of it, when a radius is given).
"""
import math


def _legal_keys(i, Lk, length, causal, radius):
    if radius is None:
        lo, hi = 0, Lk - 1
    else:
        lo, hi = i - radius, i + radius
    return [j for j in range(max(lo, 0), min(hi, Lk - 1) + 1)
            if j < length and (not causal or j <= i)]


def attention(q, k, v, key_lengths=None, causal=False, radius=None):
    """q [B][H][Lq][d_k], k [B][H][Lk][d_k], v [B][H][Lk][d_v] (nested sequences
    or numpy arrays).  Returns nested lists O [B][H][Lq][d_v]."""
    B, H = len(q), len(q[0])
    Lq, dk = len(q[0][0]), len(q[0][0][0])
    Lk, dv = len(k[0][0]), len(v[0][0][0])
    root = math.sqrt(dk)
    out = []
    for b in range(B):
        length = Lk if key_lengths is None else min(max(int(key_lengths[b]), 0), Lk)
        out_b = []
        for h in range(H):
            out_h = []
            for i in range(Lq):
                legal = _legal_keys(i, Lk, length, causal, radius)
                if not legal:
                    out_h.append([0.0] * dv)
                    continue
                e = {}
                for j in legal:
                    s = math.fsum(float(q[b][h][i][t]) * float(k[b][h][j][t]) for t in range(dk))
                    e[j] = math.exp(s / root)
                Z = math.fsum(e.values())
                row = []
                for t in range(dv):
                    row.append(math.fsum(e[j] * float(v[b][h][j][t]) for j in legal) / Z)
                out_h.append(row)
            out_b.append(out_h)
        out.append(out_b)
    return out
