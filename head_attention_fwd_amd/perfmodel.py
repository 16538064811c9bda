"""Work model of attention: allowed (query, key) pairs and algorithmic FLOPs/bytes.

Complexity per layer of self-attention is O(n^2 * d) (page "Attention Is All
You Need/paper/es", §4, Table 1); counted exactly here from the mask: each
allowed pair costs 2*d_k FLOPs for its score and 2*d_v for its share of the
weighted sum of values.  Softmax work (exp, max, sum) is not counted.
"""


def clamp_length(length, Lk):
    return int(min(max(int(length), 0), Lk))


def _band_pairs(Lq, lb, causal, radius):
    """Allowed pairs of one sequence when |i - j| <= radius is also required."""
    import numpy as np
    i = np.arange(Lq, dtype=np.int64)
    lo = np.maximum(i - radius, 0)
    hi = np.minimum(i + radius, lb - 1)
    if causal:
        hi = np.minimum(hi, i)
    return int(np.maximum(hi - lo + 1, 0).sum())


def pair_count(B, H, Lq, Lk, causal, key_lengths=None, radius=None):
    """Number of (query, key) pairs the mask allows, summed over batch and heads.

    Key j is allowed for query i when j < len_b and, for causal attention, j <= i;
    len_b = clamp(key_lengths[b], 0, Lk), or Lk without key_lengths.  With a
    radius (restricted self-attention, §4 of the same page), also |i - j| <= radius.
    """
    if radius is not None:
        return H * sum(_band_pairs(Lq, Lk if key_lengths is None else clamp_length(key_lengths[b], Lk),
                                   causal, int(radius)) for b in range(B))
    total = 0
    for b in range(B):
        lb = Lk if key_lengths is None else clamp_length(key_lengths[b], Lk)
        if not causal:
            total += Lq * lb
        elif lb <= Lq:
            # rows i < lb see i+1 keys, rows i >= lb see lb keys
            total += lb * (lb + 1) // 2 + (Lq - lb) * lb
        else:
            total += Lq * (Lq + 1) // 2
    return total * H


def flops(B, H, Lq, Lk, d_k, d_v, causal, key_lengths=None, radius=None):
    """Algorithmic FLOPs: (2*d_k + 2*d_v) per allowed pair."""
    return (2 * d_k + 2 * d_v) * pair_count(B, H, Lq, Lk, causal, key_lengths, radius)


def min_bytes(B, H, Lq, Lk, d_k, d_v, causal, key_lengths=None, elem=2, radius=None):
    """Algorithmic HBM bytes: Q and O once, and every key/value row some query may use.

    Rows j >= len_b are never needed; causal attention with Lq < Lk never needs
    rows j >= Lq, and with a radius no row needs keys j >= Lq + radius.
    """
    rows_kv = 0
    for b in range(B):
        lb = Lk if key_lengths is None else clamp_length(key_lengths[b], Lk)
        if causal:
            lb = min(lb, Lq)
        if radius is not None:
            lb = min(lb, Lq + int(radius)) if Lq > 0 else 0
        rows_kv += lb
    return elem * H * (B * Lq * (d_k + d_v) + rows_kv * (d_k + d_v))


def multihead_flops(B, Lq, Lk, d_model, h, d_k, d_v, causal, key_lengths=None):
    """Algorithmic FLOPs of MultiHead(Q, K, V) (same page, §3.2.2): the products
    with W^Q (every query position), W^K and W^V (every key position), W^O, and
    the attention's allowed pairs."""
    proj = 2 * B * Lq * d_model * h * d_k + 2 * B * Lk * d_model * h * (d_k + d_v) \
        + 2 * B * Lq * h * d_v * d_model
    return proj + flops(B, h, Lq, Lk, d_k, d_v, causal, key_lengths)


def multihead_min_bytes(B, Lq, Lk, d_model, h, d_k, d_v, self_attention, elem=2):
    """Algorithmic HBM bytes of one MultiHead call: the input sequence(s), the
    four weight matrices and the output once."""
    x = B * Lq * d_model + (0 if self_attention else B * Lk * d_model)
    w = d_model * h * (2 * d_k + d_v) + h * d_v * d_model
    return elem * (x + w + B * Lq * d_model)
