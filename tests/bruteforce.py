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


def multihead(xq, xkv, wq, wk, wv, wo, h, key_lengths=None, causal=False):
    """MultiHead(Q, K, V) = Concat(head_1..head_h) W^O, head_i = Attention(Q W_i^Q,
    K W_i^K, V W_i^V) (same page, §3.2.2), by plain loops: every projection is an
    exactly rounded sum over d_model, the heads go through ``attention`` above,
    and the concatenation is built explicitly before the product with W^O.

    xq [B][Lq][d_model], xkv [B][Lk][d_model], wq/wk [d_model][h*d_k],
    wv [d_model][h*d_v], wo [h*d_v][d_model].  Returns nested lists [B][Lq][d_model].
    """
    B, Lq, dm = len(xq), len(xq[0]), len(xq[0][0])
    Lk = len(xkv[0])
    dk = len(wq[0]) // h
    dv = len(wv[0]) // h

    def project(x, w, L, d):
        # [B][h][L][d]: head i of position j is row j of x times columns i*d.. of w
        return [[[[math.fsum(float(x[b][j][c]) * float(w[c][i * d + t]) for c in range(dm))
                   for t in range(d)] for j in range(L)] for i in range(h)] for b in range(B)]

    q = project(xq, wq, Lq, dk)
    k = project(xkv, wk, Lk, dk)
    v = project(xkv, wv, Lk, dv)
    heads = attention(q, k, v, key_lengths, causal)          # [B][h][Lq][dv]
    out = []
    for b in range(B):
        rows = []
        for i in range(Lq):
            concat = [heads[b][hd][i][t] for hd in range(h) for t in range(dv)]
            rows.append([math.fsum(concat[r] * float(wo[r][c]) for r in range(h * dv))
                         for c in range(dm)])
        out.append(rows)
    return out
