"""GPU parity: libsdpa against the fp64 oracle on the same seeded inputs.

Full element-by-element comparison on every configuration (the two long causal
ones included, in the benchmark's launch configuration), and ragged /
degenerate shapes that cross tile boundaries.  All calls go through the C ABI
via the Python binding.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import announce, assert_parity, run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny_causal_f32", "base_encoder_bf16",
                                  "base_decoder_causal_bf16", "big_cross_bf16",
                                  "rowA_h4_d128_encoder_bf16", "rowA_h16_d32_encoder_bf16",
                                  "rowA_h32_d16_encoder_bf16", "rowA_h1_d512_encoder_bf16",
                                  "base_encoder_f32", "encoder_d96_bf16"])
def test_config_full(name):
    x = workloads.generate(name)
    c = x.config
    announce("config %s" % name)
    # NaN-filled output: an element the kernels leave unwritten fails
    got = run(x.q, x.k, x.v, x.key_lengths, c.causal, c.dtype, fill=float("nan"))
    ref = oracle.attention(x.q, x.k, x.v, key_lengths=x.key_lengths, causal=c.causal)
    assert_parity(got, ref, x.v, c.dtype, name)


def _sample_rows(B, H, Lq, n_random, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, Lq // 2, Lq - 129, Lq - 128,
             Lq - 65, Lq - 64, Lq - 2, Lq - 1]
    rows = []
    for b in range(B):
        for h in range(H):
            for i in fixed:
                if 0 <= i < Lq:
                    rows.append((b, h, i))
            for i in rng.integers(0, Lq, size=n_random):
                rows.append((b, h, int(i)))
    return np.array(sorted(set(rows)), dtype=np.int64)


@pytest.mark.parametrize("name", ["long_causal_bf16", "long_causal_d128_bf16"])
def test_long_causal_full(name):
    """The long causal configurations at full size, in the launch configuration the
    benchmark times (grouped longest-first causal order), compared with the oracle
    element by element.  The output starts as NaN, so a query tile the work
    order skipped would fail.  Reports max |gpu - oracle| / max |oracle| per band
    of rows: late causal rows average thousands of values and are small, so the
    bars (scaled by max |V|) alone would be a weak signal there."""
    x = workloads.generate(name)
    c = x.config
    announce("config %s (full size, every element)" % name)
    got = run(x.q, x.k, x.v, None, True, "bf16", fill=float("nan"))
    ref = oracle.attention(x.q, x.k, x.v, causal=True)
    bands = [(0, 64), (64, 512), (512, 2048), (2048, c.Lq)]
    for lo, hi in bands:
        e = np.abs(got[:, :, lo:hi] - ref[:, :, lo:hi])
        r = np.abs(ref[:, :, lo:hi])
        rel_max = float(e.max() / r.max())
        rel_mean = float(e.mean() / r.mean())
        sys.stdout.write("[%s] rows %d-%d: max|d| %.3g (%.3g of max|O|), mean|d| %.3g "
                         "(%.3g of mean|O|)\n" % (name, lo, hi - 1, float(e.max()), rel_max,
                                                  float(e.mean()), rel_mean))
        # bf16 rounds each weight and the output to 8 significant bits
        # (relative error <= 2^-8 each): a few such units per row
        assert rel_mean <= 2.0 ** -6, (lo, hi, rel_mean)
    assert_parity(got, ref, x.v, "bf16", name)


# Ragged and degenerate shapes on both kernels: (B, H, Lq, Lk, d_k, d_v, causal, lengths)
RAGGED = [
    (2, 3, 200, 333, 64, 64, False, [0, 500]),
    (2, 3, 200, 333, 64, 64, True, [1, 333]),
    (4, 2, 129, 65, 64, 64, True, [64, 65, 63, -5]),
    (4, 2, 129, 65, 64, 64, False, [64, 65, 63, 1]),
    (1, 2, 300, 100, 64, 64, True, None),     # Lq > Lk, causal (top-left aligned)
    (1, 2, 100, 300, 64, 64, True, None),     # Lq < Lk, causal
    (1, 1, 1, 1, 64, 64, False, None),
    (1, 1, 1, 300, 64, 64, False, None),
    (1, 1, 200, 1, 64, 64, True, None),
    (3, 1, 257, 511, 64, 64, True, [511, 200, 7]),
    (2, 2, 70, 90, 16, 48, True, None),        # bf16 generic path
    (1, 1, 5, 7, 16, 16, False, None),
]
# The same shapes on the matrix-core kernel's other head sizes (d = 128 uses
# 32-key tiles and loads Q straight into registers; d = 32 packs 4 rows per 256 B;
# d = 16 uses 128-key tiles and half of each 32-row output block).
for _d in (16, 32, 128):
    RAGGED += [(B, H, Lq, Lk, _d, _d, c, ln) for (B, H, Lq, Lk, dk, dv, c, ln) in RAGGED[:10]]
for _d in (256, 512):
    RAGGED += [(B, H, Lq, Lk, _d, _d, c, ln) for (B, H, Lq, Lk, dk, dv, c, ln) in RAGGED[:10]]
RAGGED += [
    (2, 2, 70, 90, 32, 32, True, [50, 90]),
    (2, 2, 70, 90, 128, 128, False, [90, 3]),
    (2, 3, 160, 97, 128, 128, True, [97, 33]),   # several 32-key tiles, ragged tail
    # d = 128 past 1024 keys: the form budgeted for three waves per SIMD
    (2, 2, 300, 1500, 128, 128, True, [1500, 1100]),
    (2, 2, 129, 1100, 128, 128, False, [1100, 1025]),
    (2, 3, 300, 700, 16, 16, True, [700, 250]),  # several 128-key tiles, ragged tail
    # d = 64 causal: 32-key tiles up to 512 keys, 64-key tiles beyond
    (2, 2, 300, 512, 64, 64, True, [512, 129]),
    (2, 2, 300, 513, 64, 64, True, [513, 129]),
    # d = 256 and 512: the matrix-core kernel for wide heads (16 rows per wave,
    # 64 per workgroup, 32-key tiles)
    (2, 2, 70, 90, 256, 256, True, None),
    (2, 1, 100, 130, 512, 512, False, [130, 17]),
    (2, 3, 160, 700, 256, 256, True, [700, 33]),
    (2, 1, 129, 95, 512, 512, True, [95, 0]),
    # other head sizes up to 512: fp32 vector kernel (8 or 16 lanes per query row)
    (2, 2, 33, 40, 200, 320, True, [40, 0]),
    (3, 1, 65, 300, 512, 136, True, [300, 77, 1]),
    (1, 1, 1, 5, 129, 512, False, None),
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "x".join(map(str, c[:6])) +
                         ("c" if c[6] else "n"))
def test_ragged_bf16(case):
    B, H, Lq, Lk, dk, dv, causal, lengths = case
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, dk, dv, dtype="bf16", seed=Lq * 7 + Lk)
    announce("bf16 ragged %s" % (case,))
    got = run(q, k, v, lengths, causal, "bf16")
    ref = oracle.attention(q, k, v, key_lengths=lengths, causal=causal)
    assert_parity(got, ref, v, "bf16", str(case))


F32_CASES = [
    (2, 2, 16, 16, 8, 8, True, None),
    (2, 3, 100, 77, 1, 1, True, [77, 5]),
    (2, 3, 100, 77, 3, 17, False, [0, 60]),
    (1, 2, 65, 130, 64, 64, True, None),
    (2, 2, 65, 130, 64, 64, False, [129, 130]),
    (1, 1, 40, 33, 100, 128, True, None),
    (1, 1, 40, 33, 128, 40, False, [20]),
    (1, 1, 40, 50, 512, 512, True, None),
    (2, 1, 33, 17, 300, 129, False, [17, 5]),
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "x".join(map(str, c[:6])) +
                         ("c" if c[6] else "n"))
def test_ragged_f32(case):
    B, H, Lq, Lk, dk, dv, causal, lengths = case
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, dk, dv, dtype="f32", seed=Lq + 3 * Lk)
    announce("f32 ragged %s" % (case,))
    got = run(q, k, v, lengths, causal, "f32")
    ref = oracle.attention(q, k, v, key_lengths=lengths, causal=causal)
    assert_parity(got, ref, v, "f32", str(case))


@pytest.mark.parametrize("d", [16, 32, 64, 128, 256, 512])
def test_long_keys_sampled_rows(d):
    """A long key sequence (32768 keys) on the matrix-core kernel, non-causal with
    padding, rows sampled for the oracle."""
    B, H, Lq, Lk = 2, 2, 256, 32768
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, d, d, dtype="bf16", seed=21 + d)
    lengths = [32768, 20001]
    announce("long keys %d" % Lk)
    got = run(q, k, v, lengths, False, "bf16")
    rows = _sample_rows(B, H, Lq, n_random=4, seed=3)
    ref, _ = oracle.attention_rows(q, k, v, rows, key_lengths=lengths)
    assert_parity(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref, v, "bf16", "long keys")


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_tile_ring_phases(d, causal):
    """Every entry into the unrolled loop over fully legal key tiles: one batch
    entry per count of fully legal tiles (1 .. 9 tiles of 64 keys, alternately
    whole and with a ragged tail that the masked path takes after the loop),
    and, causal, waves whose diagonal ends the loop at every tile of the ring.
    Q rows past the last full query tile test the bounded row range."""
    B, H, Lq, Lk = 9, 2, 600, 600
    lengths = [64 * n + (7 if n % 2 else 0) for n in range(1, 10)]
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, d, d, dtype="bf16", seed=600 + d + causal)
    announce("tile ring phases d=%d causal=%s lengths=%s" % (d, causal, lengths))
    got = run(q, k, v, lengths, causal, "bf16", fill=float("nan"))
    ref = oracle.attention(q, k, v, key_lengths=lengths, causal=causal)
    assert_parity(got, ref, v, "bf16", "ring phases d=%d causal=%s" % (d, causal))


PADDED_CASES = [
    # (B, H, Lq, Lk, lengths): non-causal launches whose batch entries end at
    # every kind of tile boundary, with empty entries, ties, negative and
    # over-long lengths (clamped to [0, Lk])
    (16, 4, 200, 300, [300, 0, 17, 64, 65, 300, 1, -3, 999, 128, 129, 250, 64, 200, 33, 300]),
    (64, 1, 130, 256, None),   # 64 entries, lengths drawn below
    (8, 3, 64, 96, [96, 96, 0, 0, 40, 40, 96, 1]),
]


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("case", PADDED_CASES, ids=lambda c: "B%d_h%d" % (c[0], c[1]))
def test_padded_lengths_full(case, d):
    """Per-entry key lengths of every kind on each matrix-core head size; the
    output is NaN-filled first (each query tile must be written) and compared
    element by element."""
    B, H, Lq, Lk, lengths = case
    if lengths is None:
        lengths = np.random.default_rng(64).integers(0, Lk, size=B, endpoint=True).tolist()
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, d, d, dtype="bf16", seed=700 + d + B)
    announce("padded lengths B=%d h=%d d=%d lengths=%s" % (B, H, d, lengths))
    got = run(q, k, v, lengths, False, "bf16", fill=float("nan"))
    ref = oracle.attention(q, k, v, key_lengths=lengths, causal=False)
    assert_parity(got, ref, v, "bf16", "padded lengths B=%d h=%d d=%d" % (B, H, d))


# Launches with per-entry key lengths whose workgroups are all resident at
# once take the balanced work order (entries ranked by their count of key
# tiles in every wave, query tiles dealt over XCDs and dispatch rounds from
# that rank), causal or not: every query tile must still be computed exactly
# once, for any mix of lengths (ties, empty and over-long entries).
BALANCED = [
    (64, 8, 256, 256, 64),    # the base encoder's shape, d = 64 (32-key tiles)
    (32, 16, 256, 320, 64),   # the big cross-attention shape
    (64, 4, 256, 256, 128),
    (8, 1, 300, 200, 64),     # three query tiles per head, one round
    (1, 8, 500, 700, 64),     # a single entry
    (24, 3, 129, 96, 128),
    (64, 2, 64, 1000, 64),    # one query tile per head, up to 16 key tiles of 64
]


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("case", BALANCED, ids=lambda c: "B%d_h%d_Lq%d_Lk%d_d%d" % c)
def test_balanced_order_full(case, causal):
    B, H, Lq, Lk, d = case
    rng = np.random.default_rng(B * 131 + H)
    lengths = rng.integers(-3, Lk + 5, size=B).tolist()
    lengths[0] = Lk                      # at least one full entry
    if B > 2:
        lengths[1] = 0                   # and an empty one
        lengths[2] = lengths[3 % B] if B > 3 else lengths[2]   # a tie
    q, k, v, _ = workloads.draw(B, H, Lq, Lk, d, d, dtype="bf16", seed=900 + B + H + d)
    announce("balanced order B=%d h=%d Lq=%d Lk=%d d=%d causal=%s" % (case + (causal,)))
    got = run(q, k, v, lengths, causal, "bf16", fill=float("nan"))
    ref = oracle.attention(q, k, v, key_lengths=lengths, causal=causal)
    assert_parity(got, ref, v, "bf16", "balanced order %s causal=%s" % (case, causal))
