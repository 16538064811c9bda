"""Checks that pin the fp64 oracle to facts fixed outside of itself.

Every check takes an ``oracle.Oracle`` instance and raises AssertionError when
the oracle disagrees with what the pages print, a closed form, an invariant of
the mathematics, or the independent brute force of ``bruteforce.py``.
The same battery is run against deliberately broken builds of the oracle in
``test_oracle_mutations.py`` to show that a plausible mistake fails at least
one check.
"""
import math
import os

import numpy as np

import bruteforce

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Parse a ``key value...`` fixture; 'ln3' stands for the natural log of 3."""
    vals = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = [math.log(3.0) if r == "ln3" else float(r) for r in rest]
    return vals


def t4(a):
    """[n, d] -> [1, 1, n, d] float64."""
    return np.asarray(a, dtype=np.float64).reshape(1, 1, len(a), -1)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert a.shape == b.shape and err <= tol, "%s: max abs err %g > %g" % (what, err, tol)


# ---------------------------------------------------------------- printed values

def check_worked_example(orc):
    """Page "Arquitectura Transformer", "Cómo hacerlo": output 3, weights 3/4, 1/4."""
    g = read_golden("transformer_worked_example.txt")
    q = t4([g["query"]])
    k = t4([[x] for x in g["keys"]])
    v = t4([[x] for x in g["values"]])
    O, P, LSE = orc.attention(q, k, v, return_weights=True)
    _close(O[0, 0, 0], g["output"], 1e-12, "worked example output")
    _close(P[0, 0, 0], g["weights"], 1e-12, "worked example weights")
    _close(LSE[0, 0, 0], math.log(4.0), 1e-12, "worked example log-sum-exp (ln 4)")


def check_worked_example_masked(orc):
    """Same section: the second key forbidden -> weights 1 and exactly 0, output 2.

    Forbidden once by key padding (length 1) and once by the causal mask (the
    first query of a two-position self-attention sees only the first key).
    """
    g = read_golden("transformer_worked_example.txt")
    k = t4([[x] for x in g["keys"]])
    v = t4([[x] for x in g["values"]])
    O, P, _ = orc.attention(t4([g["query"]]), k, v, key_lengths=[1], return_weights=True)
    _close(O[0, 0, 0], g["masked_output"], 1e-12, "padding-masked output")
    assert P[0, 0, 0, 1] == 0.0 and P[0, 0, 0, 0] == 1.0, "padding-masked weights not (1, 0)"
    q2 = t4([g["query"], g["query"]])
    O, P, _ = orc.attention(q2, k, v, causal=True, return_weights=True)
    _close(O[0, 0, 0], g["masked_output"], 1e-12, "causal row 0 output")
    assert P[0, 0, 0, 1] == 0.0, "causal weight above the diagonal is not exactly 0"
    _close(O[0, 0, 1], g["output"], 1e-12, "causal row 1 (sees both keys) output")


def _toy(orc, weights, causal=False):
    g = read_golden("self_attention_toy.txt")
    n = len(g["values"])
    # d_k = 1, every query 1, key j = ln(w_j): the scaled score is ln(w_j).
    q = t4([[1.0]] * n)
    k = t4([[math.log(w)] for w in weights])
    v = t4([[x] for x in g["values"]])
    return orc.attention(q, k, v, causal=causal, return_weights=True)


def check_toy_rows(orc):
    """Page "Self-Attention คืออะไร (แบบจับต้องได้)", Fig. 2: 30.2 and 31.6."""
    g = read_golden("self_attention_toy.txt")
    for wk, ok in (("row0_weights", "row0_output"), ("row1_weights", "row1_output")):
        O, P, _ = _toy(orc, g[wk])
        _close(O[0, 0, 0], g[ok], 1e-9, "toy " + ok)
        _close(P[0, 0, 0], g[wk], 1e-12, "toy " + wk)


def check_toy_causal_row0(orc):
    """Same page, Fig. 2 right (decoder): the first position gets 100% -> value 10."""
    g = read_golden("self_attention_toy.txt")
    O, P, _ = _toy(orc, g["row0_weights"], causal=True)
    _close(O[0, 0, 0], g["row0_causal_output"], 0.0, "toy causal row 0 output")
    assert list(P[0, 0, 0]) == g["row0_causal_weights"], "toy causal row 0 weights"


# ---------------------------------------------------------------- closed forms

def check_scale_dk64(orc):
    """Scale 1/sqrt(d_k) at d_k = 64 (divide by 8), derived from the worked example.

    q = e_0, k_1 = 8 ln(3) e_0, k_2 = 0, so the scaled scores are ln 3 and 0 and
    the output is 3 again; without the scale it would be ~2.0006.  d_v = 3 with
    the value pair (2, 6) repeated in every column, so d_v never enters the scale.
    """
    d = 64
    q = np.zeros((1, 1, 1, d)); q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, 2, d)); k[0, 0, 0, 0] = 8.0 * math.log(3.0)
    v = np.array([[2.0] * 3, [6.0] * 3]).reshape(1, 1, 2, 3)
    _close(orc.attention(q, k, v)[0, 0, 0], [3.0] * 3, 1e-12, "d_k=64 scale pin")


def check_uniform_prefix_means(orc):
    """All-zero queries make every legal score equal: O_i = mean of the legal values.

    With the causal mask the legal keys of row i are j <= min(i, len-1), so the
    output is a prefix mean; this pins the mask geometry for every row.
    """
    rng = np.random.default_rng(11)
    B, H, Lq, Lk, dk, dv = 2, 2, 7, 6, 3, 4
    q = np.zeros((B, H, Lq, dk))
    k = rng.standard_normal((B, H, Lk, dk))
    v = rng.standard_normal((B, H, Lk, dv))
    lens = [4, 9]
    for causal in (False, True):
        O = orc.attention(q, k, v, key_lengths=lens, causal=causal)
        for b in range(B):
            lb = min(lens[b], Lk)
            for i in range(Lq):
                hi = min(i + 1, lb) if causal else lb
                _close(O[b, :, i], v[b, :, :hi].mean(axis=1), 1e-12,
                       "uniform mean b=%d i=%d causal=%d" % (b, i, causal))


def check_special_cases(orc):
    """Lk = 1 -> V_0; no legal key -> 0 (LSE -inf); one dominant score -> its value."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 2, 3, 4))
    k = rng.standard_normal((1, 2, 1, 4))
    v = rng.standard_normal((1, 2, 1, 5))
    O = orc.attention(q, k, v)
    _close(O, np.broadcast_to(v, O.shape), 1e-15, "Lk=1")
    O, P, L = orc.attention(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2),
                            key_lengths=[0], return_weights=True)
    assert np.all(O == 0.0) and np.all(P == 0.0) and np.all(np.isneginf(L)), "empty rows"
    # one key whose scaled score exceeds the others by ~500: weight 1 - O(e^-500)
    q = np.zeros((1, 1, 1, 4)); q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, 5, 4)); k[0, 0, 3, 0] = 1000.0
    v = rng.standard_normal((1, 1, 5, 2))
    _close(orc.attention(q, k, v)[0, 0, 0], v[0, 0, 3], 1e-12, "dominant key")


# ---------------------------------------------------------------- invariants

def _rand(seed, B=2, H=3, Lq=7, Lk=9, dk=5, dv=3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, Lq, dk)), rng.standard_normal((B, H, Lk, dk)),
            rng.standard_normal((B, H, Lk, dv)))


def check_rows_sum_to_one_and_masked_zero(orc):
    """Weights of a row sum to 1 and illegal weights are exactly 0 (both pages)."""
    q, k, v = _rand(1)
    lens = [4, 9]
    for causal in (False, True):
        O, P, _ = orc.attention(q, k, v, key_lengths=lens, causal=causal, return_weights=True)
        _close(P.sum(axis=-1), np.ones(P.shape[:-1]), 1e-12, "row sums")
        for b in range(2):
            for i in range(7):
                for j in range(9):
                    legal = j < lens[b] and (not causal or j <= i)
                    assert (P[b, :, i, j] > 0).all() if legal else (P[b, :, i, j] == 0).all(), \
                        "weight legality b=%d i=%d j=%d causal=%d" % (b, i, j, causal)
        # O is P V, head by head
        _close(O, np.einsum("bhij,bhjd->bhid", P, v), 1e-12, "O = P V")


def check_bruteforce_random(orc):
    """Agreement with the pure-Python brute force on multi-head, ragged inputs."""
    for seed, causal, lens in ((2, False, [3, 9]), (3, True, [9, 5]), (4, True, [0, 12]),
                               (5, False, [-1, 2])):
        q, k, v = _rand(seed)
        ref = np.array(bruteforce.attention(q, k, v, lens, causal))
        _close(orc.attention(q, k, v, key_lengths=lens, causal=causal), ref, 1e-12,
               "brute force seed=%d" % seed)
    q, k, v = _rand(6, B=1, H=2, Lq=5, Lk=3, dk=2, dv=4)
    _close(orc.attention(q, k, v, causal=True), np.array(bruteforce.attention(q, k, v, None, True)),
           1e-12, "brute force Lq > Lk")


def check_shift_invariance(orc):
    """Adding the same vector u to every key shifts row i's scores by q_i.u/sqrt(d_k)."""
    q, k, v = _rand(7)
    u = np.random.default_rng(8).standard_normal(5)
    for causal in (False, True):
        a = orc.attention(q, k, v, key_lengths=[6, 9], causal=causal)
        b = orc.attention(q, k + u, v, key_lengths=[6, 9], causal=causal)
        _close(a, b, 1e-12, "shift invariance")


def check_permutation(orc):
    """Non-causal: permuting (key, value) pairs inside [0, len) leaves O unchanged;
    self-attention with no mask: permuting positions permutes the outputs."""
    q, k, v = _rand(9)
    lens = [6, 9]
    a = orc.attention(q, k, v, key_lengths=lens)
    rng = np.random.default_rng(10)
    k2, v2 = k.copy(), v.copy()
    for b, lb in enumerate(lens):
        p = rng.permutation(lb)
        k2[b, :, :lb] = k[b][:, p]
        v2[b, :, :lb] = v[b][:, p]
    _close(a, orc.attention(q, k2, v2, key_lengths=lens), 1e-12, "key/value permutation")
    x = np.random.default_rng(13).standard_normal((1, 2, 6, 4))
    p = rng.permutation(6)
    o = orc.attention(x, x, x)
    _close(orc.attention(x[:, :, p], x[:, :, p], x[:, :, p]), o[:, :, p], 1e-12,
           "self-attention equivariance")


def check_locality(orc):
    """Changing keys/values a row may not see leaves that row unchanged."""
    q, k, v = _rand(14)
    lens = [5, 9]
    base = orc.attention(q, k, v, key_lengths=lens, causal=True)
    rng = np.random.default_rng(15)
    for i in range(7):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, i + 1:] = rng.standard_normal(k2[:, :, i + 1:].shape) * 5
        v2[:, :, i + 1:] = rng.standard_normal(v2[:, :, i + 1:].shape) * 5
        o = orc.attention(q, k2, v2, key_lengths=lens, causal=True)
        _close(o[:, :, i], base[:, :, i], 0.0, "causal locality row %d" % i)
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 5:] = 1e3
    v2[0, :, 5:] = -1e3
    _close(orc.attention(q, k2, v2, key_lengths=lens), orc.attention(q, k, v, key_lengths=lens),
           0.0, "padding independence")


def check_rows_api(orc):
    """attention_rows gives the same rows as the full call; heads are independent."""
    q, k, v = _rand(16)
    lens = [3, 8]
    full = orc.attention(q, k, v, key_lengths=lens, causal=True)
    rows = [(0, 0, 0), (1, 2, 6), (1, 1, 3), (0, 2, 5)]
    o, _ = orc.attention_rows(q, k, v, rows, key_lengths=lens, causal=True)
    for n, (b, h, i) in enumerate(rows):
        _close(o[n], full[b, h, i], 0.0, "row (%d,%d,%d)" % (b, h, i))
    for b in range(2):
        for h in range(3):
            one = orc.attention(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                                key_lengths=lens[b:b + 1], causal=True)
            _close(one[0, 0], full[b, h], 0.0, "head (%d,%d) alone" % (b, h))


# ---------------------------------------------------------------- restricted

def check_restricted_radius0(orc):
    """Radius 0 leaves only key j = i: the weight is exactly 1 and O[i] = V[i]
    (0 where position i is padding or beyond the keys)."""
    q, k, v = _rand(21, Lq=7, Lk=5)
    lens = [5, 3]
    for causal in (False, True):
        O = orc.attention(q, k, v, key_lengths=lens, causal=causal, radius=0)
        for b in range(2):
            for i in range(7):
                want = v[b, :, i] if i < lens[b] else np.zeros((3, 3))
                _close(O[b, :, i], want, 0.0, "radius 0 b=%d i=%d causal=%d" % (b, i, causal))


def check_restricted_toy(orc):
    """Page "Self-Attention คืออะไร (แบบจับต้องได้)", Fig. 1/2 weights with the
    neighbourhood of §4 of the paper page: the printed weights of the positions
    within the radius, renormalised (softmax restricted to those keys); e.g. row
    0 at radius 1 keeps 18 % and 12 % -> (0.18*10 + 0.12*20) / 0.30 = 14."""
    g = read_golden("self_attention_toy.txt")
    vals = g["values"]
    n = len(vals)
    for wk in ("row0_weights", "row1_weights"):
        w = g[wk]
        for radius in (1, 2):
            O, P, _ = _toy_r(orc, w, radius)
            for i in range(n):
                keep = [j for j in range(n) if abs(i - j) <= radius]
                z = sum(w[j] for j in keep)
                want_p = [w[j] / z if j in keep else 0.0 for j in range(n)]
                _close(P[0, 0, i], want_p, 1e-12, "restricted toy %s r=%d weights row %d" % (wk, radius, i))
                _close(O[0, 0, i], [sum(w[j] * vals[j] for j in keep) / z], 1e-9,
                       "restricted toy %s r=%d output row %d" % (wk, radius, i))
    O, _, _ = _toy_r(orc, g["row0_weights"], 1)
    _close(O[0, 0, 0], [14.0], 1e-9, "restricted toy row 0 radius 1 = 14")


def _toy_r(orc, weights, radius):
    g = read_golden("self_attention_toy.txt")
    n = len(g["values"])
    q = t4([[1.0]] * n)
    k = t4([[math.log(w)] for w in weights])
    v = t4([[x] for x in g["values"]])
    return orc.attention(q, k, v, return_weights=True, radius=radius)


def check_restricted_bruteforce(orc):
    """Agreement with the brute force for several radii, masks and shapes."""
    for seed, causal, lens, radius in ((31, False, [3, 9], 1), (32, True, [9, 5], 2),
                                       (33, False, None, 3), (34, True, [0, 12], 1),
                                       (35, False, [7, 9], 4), (36, True, None, 0)):
        q, k, v = _rand(seed)
        ref = np.array(bruteforce.attention(q, k, v, lens, causal, radius))
        _close(orc.attention(q, k, v, key_lengths=lens, causal=causal, radius=radius), ref, 1e-12,
               "restricted brute force seed=%d" % seed)
    q, k, v = _rand(37, B=1, H=2, Lq=9, Lk=4, dk=2, dv=4)
    for radius in (0, 2, 5):
        _close(orc.attention(q, k, v, radius=radius),
               np.array(bruteforce.attention(q, k, v, None, False, radius)), 1e-12,
               "restricted brute force Lq > Lk r=%d" % radius)
    o, _ = orc.attention_rows(q, k, v, [(0, 1, 6), (0, 0, 2)], radius=2)
    _close(o, np.array(bruteforce.attention(q, k, v, None, False, 2))[0, [1, 0], [6, 2]], 1e-12,
           "restricted rows api")


def check_restricted_locality(orc):
    """Keys and values outside row i's neighbourhood do not change row i; a change
    inside it does."""
    q, k, v = _rand(38, Lq=9, Lk=9)
    radius = 2
    base = orc.attention(q, k, v, radius=radius)
    rng = np.random.default_rng(39)
    for i in range(9):
        k2, v2 = k.copy(), v.copy()
        out = [j for j in range(9) if abs(i - j) > radius]
        k2[:, :, out] = rng.standard_normal(k2[:, :, out].shape) * 5
        v2[:, :, out] = rng.standard_normal(v2[:, :, out].shape) * 5
        _close(orc.attention(q, k2, v2, radius=radius)[:, :, i], base[:, :, i], 0.0,
               "restricted locality row %d" % i)
        v3 = v.copy()
        v3[:, :, min(i + radius, 8)] += 1.0
        assert np.all(np.abs(orc.attention(q, k, v3, radius=radius)[:, :, i] - base[:, :, i]) > 1e-6), \
            "row %d must see its neighbourhood's edge" % i
    wide = orc.attention(q, k, v, radius=8)
    _close(wide, orc.attention(q, k, v), 0.0, "radius >= L - 1 is unrestricted")


# ---------------------------------------------------------------- multi-head

def _mh_rand(seed, B=2, Lq=5, Lk=6, dm=6, h=2, dk=3, dv=2):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Lq, dm)), rng.standard_normal((B, Lk, dm)),
            rng.standard_normal((dm, h * dk)) / math.sqrt(dm),
            rng.standard_normal((dm, h * dk)) / math.sqrt(dm),
            rng.standard_normal((dm, h * dv)) / math.sqrt(dm),
            rng.standard_normal((h * dv, dm)) / math.sqrt(h * dv))


def check_multihead_identity_is_attention(orc):
    """h = 1, d_k = d_v = d_model and every W the identity: MultiHead(X, X, X) is
    Attention(X, X, X) of Eq. (1) (scale 1/sqrt(d_model))."""
    rng = np.random.default_rng(41)
    x = rng.standard_normal((2, 5, 4))
    eye = np.eye(4)
    for causal, lens in ((False, None), (True, [5, 3])):
        got = orc.multihead(x, x, eye, eye, eye, eye, 1, key_lengths=lens, causal=causal)
        ref = orc.attention(x[:, None], x[:, None], x[:, None], key_lengths=lens, causal=causal)
        _close(got, ref[:, 0], 1e-12, "multihead identity causal=%d" % causal)


def check_multihead_bruteforce(orc):
    """Agreement with the plain-loop brute force: self- and cross-attention,
    masks, d_k != d_v."""
    for seed, causal, lens, self_attn in ((42, False, None, True), (43, True, [5, 2], True),
                                          (44, False, [6, 1], False), (45, True, None, False)):
        xq, xkv, wq, wk, wv, wo = _mh_rand(seed)
        if self_attn:
            xkv = xq
        ref = np.array(bruteforce.multihead(xq, xkv, wq, wk, wv, wo, 2, lens, causal))
        _close(orc.multihead(xq, xkv, wq, wk, wv, wo, 2, key_lengths=lens, causal=causal), ref,
               1e-12, "multihead brute force seed=%d" % seed)


def check_multihead_uniform_keys(orc):
    """W^K = 0 makes every score 0: each head's weights are uniform over the legal
    keys, so the output is the mean of the legal rows of (X_kv W^V), times W^O."""
    xq, xkv, wq, wk, wv, wo = _mh_rand(46, Lk=6)
    lens = [6, 4]
    got = orc.multihead(xq, xkv, wq, np.zeros_like(wk), wv, wo, 2, key_lengths=lens)
    for b, lb in enumerate(lens):
        mean_v = (xkv[b, :lb] @ wv).mean(axis=0)            # [h*d_v], heads concatenated
        _close(got[b], np.tile(mean_v @ wo, (xq.shape[1], 1)), 1e-12, "uniform keys b=%d" % b)


def check_multihead_head_order(orc):
    """Renumbering the heads (the column blocks of W^Q, W^K, W^V and the row
    blocks of W^O together) leaves MultiHead unchanged; swapping only W^O's
    blocks changes it."""
    xq, xkv, wq, wk, wv, wo = _mh_rand(47, h=3, dk=2, dv=3, dm=5)
    base = orc.multihead(xq, xkv, wq, wk, wv, wo, 3, causal=True)
    perm = [2, 0, 1]
    cols = lambda w, d: np.concatenate([w[:, p * d:(p + 1) * d] for p in perm], axis=1)
    rows = lambda w, d: np.concatenate([w[p * d:(p + 1) * d] for p in perm], axis=0)
    got = orc.multihead(xq, xkv, cols(wq, 2), cols(wk, 2), cols(wv, 3), rows(wo, 3), 3, causal=True)
    _close(got, base, 1e-12, "head renumbering")
    other = orc.multihead(xq, xkv, wq, wk, wv, rows(wo, 3), 3, causal=True)
    assert np.max(np.abs(other - base)) > 1e-3, "W^O blocks must follow their heads"


def check_multihead_rows_api(orc):
    """multihead_rows gives the full call's rows; batch entries are independent."""
    xq, xkv, wq, wk, wv, wo = _mh_rand(48, Lq=6, Lk=6)
    xkv = xq
    lens = [6, 3]
    full = orc.multihead(xq, xkv, wq, wk, wv, wo, 2, key_lengths=lens, causal=True)
    rows = [(0, 0), (1, 5), (1, 2), (0, 4), (1, 0)]
    got = orc.multihead_rows(xq, xkv, wq, wk, wv, wo, 2, rows, key_lengths=lens, causal=True)
    for n, (b, i) in enumerate(rows):
        _close(got[n], full[b, i], 1e-12, "multihead row (%d,%d)" % (b, i))
    ref = np.array(bruteforce.multihead(xq, xkv, wq, wk, wv, wo, 2, lens, True))
    _close(got, ref[[r[0] for r in rows], [r[1] for r in rows]], 1e-12, "rows vs brute force")


ALL_CHECKS = [
    check_worked_example, check_worked_example_masked, check_toy_rows, check_toy_causal_row0,
    check_scale_dk64, check_uniform_prefix_means, check_special_cases,
    check_rows_sum_to_one_and_masked_zero, check_bruteforce_random, check_shift_invariance,
    check_permutation, check_locality, check_rows_api,
    check_restricted_radius0, check_restricted_toy, check_restricted_bruteforce,
    check_restricted_locality,
    check_multihead_identity_is_attention, check_multihead_bruteforce, check_multihead_uniform_keys,
    check_multihead_head_order, check_multihead_rows_api,
]
