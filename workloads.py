"""Seeded synthetic inputs for multi-head scaled dot-product attention.

This module is the only code shared by the CPU oracle (``oracle/``) and the HIP
path (``head_attention_fwd_amd/``).  It draws random numbers and rounds them to
the storage type; it performs none of the attention arithmetic.

Shapes follow the base and big models of "Attention Is All You Need"
(page "Attention Is All You Need/paper/es", §3.2.2: h = 8 heads with
d_k = d_v = d_model / h = 64 for d_model = 512; Table 3, row "big": d_model =
1024, h = 16).  The pages train on length-bucketed batches (§5.1), so the
key-padding configurations draw one key length per sequence.

Recipe (identical for every configuration):
  rng = numpy.random.Generator(numpy.random.PCG64(seed))
  Q, K, V = rng.standard_normal(shape) each, in that order, as float64,
            multiplied by ``scale`` (0.5 for the long causal case), rounded to
            float32 (round to nearest even), then, for bf16 configurations,
            rounded again to bfloat16 (round to nearest even);
  key_lengths = rng.integers(lo, hi, size=B, endpoint=True) as int32, drawn
            after V, only for configurations with key padding.
All arrays are returned as float32 numpy arrays whose values are exactly
representable in the configuration's storage type.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    description: str
    dtype: str            # "f32" or "bf16": storage and arithmetic type of the GPU path
    B: int
    H: int
    Lq: int
    Lk: int
    d_k: int
    d_v: int
    causal: bool
    key_len_range: Optional[tuple]   # inclusive (lo, hi) or None for "no padding"
    scale: float
    seed: int
    entry: str = "forward"   # "forward": sdpa_forward; "decode": sdpa_decode (causal = False);
    #                          "restricted": sdpa_forward_restricted with `radius`
    radius: Optional[int] = None
    d_model: Optional[int] = None   # entry "multihead": model width; H heads of d_k, d_v
    self_attention: bool = True     # entry "multihead": keys and values from the query sequence


CONFIGS = {
    "tiny_causal_f32": Config(
        "tiny_causal_f32", "tiny causal self-attention, fp32", "f32",
        B=2, H=2, Lq=16, Lk=16, d_k=8, d_v=8, causal=True, key_len_range=None,
        scale=1.0, seed=0),
    "base_encoder_bf16": Config(
        "base_encoder_bf16", "base-model encoder self-attention with key padding", "bf16",
        B=64, H=8, Lq=256, Lk=256, d_k=64, d_v=64, causal=False, key_len_range=(64, 256),
        scale=1.0, seed=1),
    "base_decoder_causal_bf16": Config(
        "base_decoder_causal_bf16", "base-model decoder causal self-attention with key padding",
        "bf16", B=64, H=8, Lq=256, Lk=256, d_k=64, d_v=64, causal=True,
        key_len_range=(64, 256), scale=1.0, seed=2),
    "big_cross_bf16": Config(
        "big_cross_bf16", "big-model encoder-decoder cross-attention with encoder padding",
        "bf16", B=32, H=16, Lq=256, Lk=320, d_k=64, d_v=64, causal=False,
        key_len_range=(128, 320), scale=1.0, seed=3),
    "long_causal_bf16": Config(
        "long_causal_bf16", "long-sequence causal self-attention, inputs scaled by 0.5", "bf16",
        B=4, H=16, Lq=8192, Lk=8192, d_k=64, d_v=64, causal=True, key_len_range=None,
        scale=0.5, seed=4),
    # Table 3, row (A): d_model = 512 split into other head counts, d_k = d_v =
    # 512 / h, on the base encoder's batch shape.
    "rowA_h4_d128_encoder_bf16": Config(
        "rowA_h4_d128_encoder_bf16", "encoder self-attention with key padding, "
        "h = 4 heads of d_k = d_v = 128 (Table 3 row A)", "bf16",
        B=64, H=4, Lq=256, Lk=256, d_k=128, d_v=128, causal=False, key_len_range=(64, 256),
        scale=1.0, seed=7),
    "rowA_h16_d32_encoder_bf16": Config(
        "rowA_h16_d32_encoder_bf16", "encoder self-attention with key padding, "
        "h = 16 heads of d_k = d_v = 32 (Table 3 row A)", "bf16",
        B=64, H=16, Lq=256, Lk=256, d_k=32, d_v=32, causal=False, key_len_range=(64, 256),
        scale=1.0, seed=8),
    "rowA_h32_d16_encoder_bf16": Config(
        "rowA_h32_d16_encoder_bf16", "encoder self-attention with key padding, "
        "h = 32 heads of d_k = d_v = 16 (Table 3 row A)", "bf16",
        B=64, H=32, Lq=256, Lk=256, d_k=16, d_v=16, causal=False, key_len_range=(64, 256),
        scale=1.0, seed=15),
    "rowA_h1_d512_encoder_bf16": Config(
        "rowA_h1_d512_encoder_bf16", "encoder self-attention with key padding, "
        "h = 1 head of d_k = d_v = 512 (Table 3 row A)", "bf16",
        B=64, H=1, Lq=256, Lk=256, d_k=512, d_v=512, causal=False, key_len_range=(64, 256),
        scale=1.0, seed=16),
    # The vector-unit paths at the base encoder's shape: fp32 (all head sizes)
    # and bf16 with a head size the matrix-core kernels do not take.
    "base_encoder_f32": Config(
        "base_encoder_f32", "base-model encoder self-attention with key padding, fp32", "f32",
        B=64, H=8, Lq=256, Lk=256, d_k=64, d_v=64, causal=False, key_len_range=(64, 256),
        scale=1.0, seed=19),
    "encoder_d96_bf16": Config(
        "encoder_d96_bf16", "encoder self-attention with key padding, h = 8 heads of "
        "d_k = d_v = 96 (a head size without a matrix-core layout)", "bf16",
        B=64, H=8, Lq=256, Lk=256, d_k=96, d_v=96, causal=False, key_len_range=(64, 256),
        scale=1.0, seed=20),
    "long_causal_d128_bf16": Config(
        "long_causal_d128_bf16", "long-sequence causal self-attention, d_model = 1024 as "
        "h = 8 heads of d_k = d_v = 128, inputs scaled by 0.5", "bf16",
        B=4, H=8, Lq=8192, Lk=8192, d_k=128, d_v=128, causal=True, key_len_range=None,
        scale=0.5, seed=9),
    # Restricted self-attention (§4, Table 1): the long sequence with a
    # neighbourhood of r = 2 * 255 + 1 = 511 positions around each output.
    "restricted_long_bf16": Config(
        "restricted_long_bf16", "long-sequence restricted self-attention, radius 255 "
        "(neighbourhood of 511 positions), inputs scaled by 0.5", "bf16",
        B=4, H=16, Lq=8192, Lk=8192, d_k=64, d_v=64, causal=False, key_len_range=None,
        scale=0.5, seed=10, entry="restricted", radius=255),
    "restricted_long_causal_bf16": Config(
        "restricted_long_causal_bf16", "long-sequence restricted causal self-attention "
        "(the 256 positions up to each output), inputs scaled by 0.5", "bf16",
        B=4, H=16, Lq=8192, Lk=8192, d_k=64, d_v=64, causal=True, key_len_range=None,
        scale=0.5, seed=11, entry="restricted", radius=255),
    # Multi-head attention with its projections (§3.2.2, sdpa_multihead_forward):
    # random-init weights of the base and big models' shapes.
    "mha_base_encoder_bf16": Config(
        "mha_base_encoder_bf16", "base-model encoder multi-head self-attention with the "
        "projections (d_model 512, h 8), key padding", "bf16",
        B=64, H=8, Lq=256, Lk=256, d_k=64, d_v=64, causal=False, key_len_range=(64, 256),
        scale=1.0, seed=12, entry="multihead", d_model=512),
    "mha_big_cross_bf16": Config(
        "mha_big_cross_bf16", "big-model encoder-decoder multi-head attention with the "
        "projections (d_model 1024, h 16), encoder padding", "bf16",
        B=32, H=16, Lq=256, Lk=320, d_k=64, d_v=64, causal=False, key_len_range=(128, 320),
        scale=1.0, seed=13, entry="multihead", d_model=1024, self_attention=False),
    "mha_long_causal_bf16": Config(
        "mha_long_causal_bf16", "long-sequence causal multi-head self-attention with the "
        "projections (d_model 1024, h 16), inputs scaled by 0.5", "bf16",
        B=4, H=16, Lq=8192, Lk=8192, d_k=64, d_v=64, causal=True, key_len_range=None,
        scale=0.5, seed=14, entry="multihead", d_model=1024),
    # Decode steps (sdpa_decode): the new position of an autoregressive decoder
    # against the cache of the positions generated so far (§3.1, §3.2.3).
    "decode_long_bf16": Config(
        "decode_long_bf16", "decode step after the long sequence: one new position per head "
        "against an 8192-key cache, inputs scaled by 0.5", "bf16",
        B=4, H=16, Lq=1, Lk=8192, d_k=64, d_v=64, causal=False, key_len_range=None,
        scale=0.5, seed=5, entry="decode"),
    "decode_base_bf16": Config(
        "decode_base_bf16", "base-model decode step: 64 sequences (e.g. 16 sentences x 4 beams), "
        "one new position against caches of up to 256 positions", "bf16",
        B=64, H=8, Lq=1, Lk=256, d_k=64, d_v=64, causal=False, key_len_range=(64, 256),
        scale=1.0, seed=6, entry="decode"),
    # Table 3 row (A), h = 4 heads of d_k = d_v = 128, decode steps
    "decode_long_d128_bf16": Config(
        "decode_long_d128_bf16", "decode step after the long sequence, h = 4 heads of "
        "d_k = d_v = 128 (Table 3 row A): one new position per head against an 8192-key cache, "
        "inputs scaled by 0.5", "bf16",
        B=4, H=4, Lq=1, Lk=8192, d_k=128, d_v=128, causal=False, key_len_range=None,
        scale=0.5, seed=17, entry="decode"),
    "decode_base_d128_bf16": Config(
        "decode_base_d128_bf16", "base-model decode step with h = 4 heads of d_k = d_v = 128 "
        "(Table 3 row A): 64 sequences, caches of up to 256 positions", "bf16",
        B=64, H=4, Lq=1, Lk=256, d_k=128, d_v=128, causal=False, key_len_range=(64, 256),
        scale=1.0, seed=18, entry="decode"),
}

#: Configuration order used by tests and reports (smallest first): the five
#: forward configurations, the other head sizes, then the decode steps.
ORDER = ["tiny_causal_f32", "base_encoder_bf16", "base_decoder_causal_bf16",
         "big_cross_bf16", "long_causal_bf16", "rowA_h4_d128_encoder_bf16",
         "rowA_h16_d32_encoder_bf16", "rowA_h32_d16_encoder_bf16", "rowA_h1_d512_encoder_bf16",
         "long_causal_d128_bf16", "restricted_long_bf16",
         "restricted_long_causal_bf16", "mha_base_encoder_bf16", "mha_big_cross_bf16",
         "mha_long_causal_bf16", "decode_base_bf16", "decode_long_bf16", "decode_base_d128_bf16",
         "decode_long_d128_bf16", "base_encoder_f32", "encoder_d96_bf16"]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Inputs must be finite.  bfloat16 is the upper 16 bits of an IEEE float32.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16) << np.uint64(16)
    return bits.astype(np.uint32).view(np.float32)


@dataclasses.dataclass
class Inputs:
    config: Config
    q: np.ndarray                       # [B, H, Lq, d_k] float32
    k: np.ndarray                       # [B, H, Lk, d_k] float32
    v: np.ndarray                       # [B, H, Lk, d_v] float32
    key_lengths: Optional[np.ndarray]   # [B] int32 or None


def draw(B: int, H: int, Lq: int, Lk: int, d_k: int, d_v: int, *, dtype: str = "bf16",
         seed: int = 0, scale: float = 1.0, key_len_range: Optional[tuple] = None):
    """Draw (q, k, v, key_lengths) with the module's recipe for any shape."""
    rng = np.random.Generator(np.random.PCG64(seed))

    def one(shape):
        a = rng.standard_normal(shape)
        if scale != 1.0:
            a = a * scale
        a = a.astype(np.float32)
        return round_to_bf16(a) if dtype == "bf16" else a

    q = one((B, H, Lq, d_k))
    k = one((B, H, Lk, d_k))
    v = one((B, H, Lk, d_v))
    kl = None
    if key_len_range is not None:
        lo, hi = key_len_range
        kl = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    return q, k, v, kl


def draw_spiked(B: int, H: int, Lq: int, Lk: int, d: int, *, dtype: str = "bf16", seed: int = 0,
                spikes=(), lift: float = 3.0, qk_scale: float = 1.0):
    """Inputs whose scores jump far above the running maximum part-way along the keys.

    Recipe: the same generator; Q, K (standard normal times ``qk_scale``) and V
    (standard normal) in that order, then one direction u per (b, h) (standard
    normal, normalised to length 1).  Every Q row gets ``lift * u`` added; for
    each (j, t) in ``spikes`` key row j becomes ``t * sqrt(d) / lift * u``, so
    that its score against a query row is about t (in nats) times
    (q . u) / lift, i.e. near t for most rows and spread around it.  Rounded to
    float32 and, for bf16, to bfloat16 (nearest even), as ``draw``.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, H, Lq, d)) * qk_scale
    k = rng.standard_normal((B, H, Lk, d)) * qk_scale
    v = rng.standard_normal((B, H, Lk, d))
    u = rng.standard_normal((B, H, d))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    q += lift * u[:, :, None, :]
    for j, t in spikes:
        if 0 <= j < Lk:
            k[:, :, j, :] = (t * np.sqrt(d) / lift) * u

    def store(a):
        a = a.astype(np.float32)
        return round_to_bf16(a) if dtype == "bf16" else a

    return store(q), store(k), store(v)


@dataclasses.dataclass
class MultiHeadInputs:
    config: Config
    xq: np.ndarray                      # [B, Lq, d_model] float32
    xkv: np.ndarray                     # [B, Lk, d_model]; xq itself for self-attention
    wq: np.ndarray                      # [d_model, h*d_k]
    wk: np.ndarray                      # [d_model, h*d_k]
    wv: np.ndarray                      # [d_model, h*d_v]
    wo: np.ndarray                      # [h*d_v, d_model]
    key_lengths: Optional[np.ndarray]   # [B] int32 or None


def draw_multihead(B: int, Lq: int, Lk: int, d_model: int, h: int, d_k: int, d_v: int, *,
                   seed: int = 0, scale: float = 1.0, self_attention: bool = True,
                   key_len_range: Optional[tuple] = None, dtype: str = "bf16"):
    """Draw (xq, xkv, wq, wk, wv, wo, key_lengths) with the module's recipe.

    Recipe: the same generator; xq (then xkv unless self-attention; then xkv is
    xq and Lk must equal Lq) standard normal times ``scale``; then wq, wk, wv,
    wo standard normal divided by sqrt(fan_in) (d_model for wq, wk, wv; h*d_v for
    wo), so that every projection keeps unit scale; key_lengths last.  All
    rounded to float32 and, for bf16, to bfloat16 (nearest even)."""
    rng = np.random.Generator(np.random.PCG64(seed))

    def one(shape, mult):
        a = rng.standard_normal(shape)
        if mult != 1.0:
            a = a * mult
        a = a.astype(np.float32)
        return round_to_bf16(a) if dtype == "bf16" else a

    xq = one((B, Lq, d_model), scale)
    if self_attention:
        if Lk != Lq:
            raise ValueError("self-attention needs Lk == Lq")
        xkv = xq
    else:
        xkv = one((B, Lk, d_model), scale)
    wq = one((d_model, h * d_k), 1.0 / np.sqrt(d_model))
    wk = one((d_model, h * d_k), 1.0 / np.sqrt(d_model))
    wv = one((d_model, h * d_v), 1.0 / np.sqrt(d_model))
    wo = one((h * d_v, d_model), 1.0 / np.sqrt(h * d_v))
    kl = None
    if key_len_range is not None:
        lo, hi = key_len_range
        kl = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    return xq, xkv, wq, wk, wv, wo, kl


def generate(name: str):
    """Inputs for one named configuration (MultiHeadInputs for entry "multihead")."""
    c = CONFIGS[name]
    if c.entry == "multihead":
        return MultiHeadInputs(c, *draw_multihead(c.B, c.Lq, c.Lk, c.d_model, c.H, c.d_k, c.d_v,
                                                  seed=c.seed, scale=c.scale,
                                                  self_attention=c.self_attention,
                                                  key_len_range=c.key_len_range, dtype=c.dtype))
    q, k, v, kl = draw(c.B, c.H, c.Lq, c.Lk, c.d_k, c.d_v, dtype=c.dtype, seed=c.seed,
                       scale=c.scale, key_len_range=c.key_len_range)
    return Inputs(c, q, k, v, kl)
