"""Plain fp64 CPU oracle for multi-head scaled dot-product attention (forward).

TEST INFRASTRUCTURE ONLY.  The oracle is what the HIP path is checked against.
Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import it.  It shares no code with ``head_attention_fwd_amd`` and the
product path never calls it.

The arithmetic lives in ``sdpa_oracle.c`` (plain C, fp64, OpenMP over query
rows); this module only builds that file with gcc, converts numpy arrays to
contiguous fp64 and calls it through ctypes.

Computes, for every batch entry b, head h and query row i
(page "Attention Is All You Need/paper/es", §3.2.1, Eq. (1) and §3.2.3):
    O[b,h,i,:] = sum_j softmax_j( Q[b,h,i,:].K[b,h,j,:] / sqrt(d_k) + mask ) V[b,h,j,:]
with mask = -inf where j >= len_b (key padding, len_b = clamp(key_lengths[b],
0, Lk)), for causal attention where j > i, and for restricted self-attention
with radius w (same page, §4 and Table 1: a neighbourhood of size r = 2w + 1
centred on the output position) where |i - j| > w.  A row with no legal key
is 0.  ``multihead`` adds the projections of §3.2.2 around it:
MultiHead(Q, K, V) = Concat(head_1..head_h) W^O, head_i = Attention(Q W_i^Q,
K W_i^K, V W_i^V).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "sdpa_oracle.c")
LIBRARY = os.path.join(_HERE, "libsdpa_oracle.so")


def compile_oracle(src: str, out: str) -> str:
    """Compile a C source of the oracle with gcc into a shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                    "-Wall", "-Wextra", "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile sdpa_oracle.c into oracle/libsdpa_oracle.so."""
    if not force and os.path.exists(LIBRARY) and \
            os.path.getmtime(LIBRARY) >= os.path.getmtime(SOURCE):
        return LIBRARY
    return compile_oracle(SOURCE, LIBRARY)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, ctype=ctypes.c_double):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctype))


def _shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, Lq, dk = q.shape
    Bk, Hk, Lk, dk2 = k.shape
    Bv, Hv, Lv, dv = v.shape
    if (Bk, Hk, dk2) != (B, H, dk) or (Bv, Hv, Lv) != (B, H, Lk):
        raise ValueError("inconsistent q/k/v shapes %s %s %s" % (q.shape, k.shape, v.shape))
    return B, H, Lq, Lk, dk, dv


def _lengths(key_lengths, B):
    if key_lengths is None:
        return None
    kl = np.ascontiguousarray(key_lengths, dtype=np.int32)
    if kl.shape != (B,):
        raise ValueError("key_lengths must have shape [B]")
    return kl


def _radius(radius):
    if radius is None:
        return -1
    if int(radius) < 0:
        raise ValueError("radius must be None or >= 0")
    return int(radius)


class Oracle:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        i64 = ctypes.c_int64
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [dp, dp, dp, ip, ctypes.c_int, i64, i64, i64, i64,
                                         i64, i64, i64, dp, dp, dp, ctypes.c_int]
        lib.oracle_attention_rows.restype = ctypes.c_int
        lib.oracle_attention_rows.argtypes = [dp, dp, dp, ip, ctypes.c_int, i64, i64, i64,
                                              i64, i64, i64, i64,
                                              ctypes.POINTER(ctypes.c_int64), i64, dp, dp,
                                              ctypes.c_int]
        lib.oracle_multihead.restype = ctypes.c_int
        lib.oracle_multihead.argtypes = [dp, dp, dp, dp, dp, dp, ip, ctypes.c_int, i64, i64, i64,
                                         i64, i64, i64, i64, dp, ctypes.c_int]
        lib.oracle_multihead_rows.restype = ctypes.c_int
        lib.oracle_multihead_rows.argtypes = [dp, dp, dp, dp, dp, dp, ip, ctypes.c_int, i64, i64,
                                              i64, i64, i64, i64, i64,
                                              ctypes.POINTER(ctypes.c_int64), i64, dp,
                                              ctypes.c_int]
        self.lib = lib
        self.path = path

    def _mh_args(self, xq, xkv, wq, wk, wv, wo, h, key_lengths):
        xq, xkv = _f64(xq), _f64(xkv)
        wq, wk, wv, wo = _f64(wq), _f64(wk), _f64(wv), _f64(wo)
        if xq.ndim != 3 or xkv.ndim != 3:
            raise ValueError("xq and xkv must be [B, L, d_model]")
        B, Lq, dm = xq.shape
        Lk = xkv.shape[1]
        if xkv.shape != (B, Lk, dm) or wq.shape[0] != dm or wq.shape[1] % h:
            raise ValueError("inconsistent shapes")
        dk = wq.shape[1] // h
        dv = wv.shape[1] // h
        if wk.shape != (dm, h * dk) or wv.shape != (dm, h * dv) or wo.shape != (h * dv, dm):
            raise ValueError("inconsistent weight shapes")
        return xq, xkv, wq, wk, wv, wo, _lengths(key_lengths, B), (B, Lq, Lk, dm, dk, dv)

    def multihead_rows(self, xq, xkv, wq, wk, wv, wo, h, rows, key_lengths=None, causal=False,
                       nthreads=0):
        """Rows of multihead(): ``rows`` is an int array of (b, i) pairs.
        Returns O_rows [n, d_model]."""
        xq, xkv, wq, wk, wv, wo, kl, (B, Lq, Lk, dm, dk, dv) = self._mh_args(
            xq, xkv, wq, wk, wv, wo, h, key_lengths)
        rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
        flat = np.ascontiguousarray(rows[:, 0] * Lq + rows[:, 1])
        O = np.empty((rows.shape[0], dm), dtype=np.float64)
        rc = self.lib.oracle_multihead_rows(_ptr(xq), _ptr(xkv), _ptr(wq), _ptr(wk), _ptr(wv),
                                            _ptr(wo), _ptr(kl, ctypes.c_int32), int(bool(causal)),
                                            B, Lq, Lk, dm, h, dk, dv, _ptr(flat, ctypes.c_int64),
                                            len(flat), _ptr(O), int(nthreads))
        if rc != 0:
            raise RuntimeError("oracle_multihead_rows failed with code %d" % rc)
        return O

    def multihead(self, xq, xkv, wq, wk, wv, wo, h, key_lengths=None, causal=False, nthreads=0):
        """MultiHead(Q, K, V) = Concat(head_1..head_h) W^O in fp64 (§3.2.2).

        xq [B, Lq, d_model] (queries' sequence), xkv [B, Lk, d_model] (keys' and
        values' sequence), wq and wk [d_model, h*d_k], wv [d_model, h*d_v],
        wo [h*d_v, d_model]; head i uses columns i*d .. i*d + d - 1 of wq, wk,
        wv.  Returns O [B, Lq, d_model]."""
        xq, xkv = _f64(xq), _f64(xkv)
        wq, wk, wv, wo = _f64(wq), _f64(wk), _f64(wv), _f64(wo)
        if xq.ndim != 3 or xkv.ndim != 3:
            raise ValueError("xq and xkv must be [B, L, d_model]")
        B, Lq, dm = xq.shape
        Lk = xkv.shape[1]
        if xkv.shape != (B, Lk, dm) or wq.shape[0] != dm or wq.shape[1] % h:
            raise ValueError("inconsistent shapes")
        dk = wq.shape[1] // h
        dv = wv.shape[1] // h
        if wk.shape != (dm, h * dk) or wv.shape != (dm, h * dv) or wo.shape != (h * dv, dm):
            raise ValueError("inconsistent weight shapes")
        kl = _lengths(key_lengths, B)
        O = np.empty((B, Lq, dm), dtype=np.float64)
        rc = self.lib.oracle_multihead(_ptr(xq), _ptr(xkv), _ptr(wq), _ptr(wk), _ptr(wv),
                                       _ptr(wo), _ptr(kl, ctypes.c_int32), int(bool(causal)), B,
                                       Lq, Lk, dm, h, dk, dv, _ptr(O), int(nthreads))
        if rc != 0:
            raise RuntimeError("oracle_multihead failed with code %d" % rc)
        return O

    def attention(self, q, k, v, key_lengths=None, causal=False, return_weights=False,
                  nthreads=0, radius=None):
        """Full attention in fp64.  Returns O, or (O, P, LSE) if return_weights.
        radius: None (no restriction) or w >= 0 (keys with |i - j| <= w only)."""
        B, H, Lq, Lk, dk, dv = _shapes(q, k, v)
        q, k, v = _f64(q), _f64(k), _f64(v)
        kl = _lengths(key_lengths, B)
        O = np.empty((B, H, Lq, dv), dtype=np.float64)
        P = np.empty((B, H, Lq, Lk), dtype=np.float64) if return_weights else None
        LSE = np.empty((B, H, Lq), dtype=np.float64) if return_weights else None
        rc = self.lib.oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(kl, ctypes.c_int32),
                                       int(bool(causal)), _radius(radius), B, H, Lq, Lk, dk, dv,
                                       _ptr(O), _ptr(P), _ptr(LSE), int(nthreads))
        if rc != 0:
            raise RuntimeError("oracle_attention failed with code %d" % rc)
        return (O, P, LSE) if return_weights else O

    def attention_rows(self, q, k, v, rows, key_lengths=None, causal=False, nthreads=0,
                       radius=None):
        """Attention for selected rows only.

        ``rows`` is an int array of (b, head, i) triples, shape [n, 3].  Returns
        (O_rows [n, d_v], LSE_rows [n]).  Rows are grouped by head so that only
        the heads involved are converted to fp64.
        """
        B, H, Lq, Lk, dk, dv = _shapes(q, k, v)
        rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
        kl = _lengths(key_lengths, B)
        out = np.empty((rows.shape[0], dv), dtype=np.float64)
        lse = np.empty((rows.shape[0],), dtype=np.float64)
        heads = {}
        for n, (b, h, i) in enumerate(rows):
            if not (0 <= b < B and 0 <= h < H and 0 <= i < Lq):
                raise ValueError("row (%d, %d, %d) out of range" % (b, h, i))
            heads.setdefault((int(b), int(h)), []).append(n)
        for (b, h), idx in heads.items():
            qh = _f64(q[b, h])[None, None]
            kh = _f64(k[b, h])[None, None]
            vh = _f64(v[b, h])[None, None]
            klh = None if kl is None else kl[b:b + 1].copy()
            sel = np.ascontiguousarray(rows[idx, 2])
            o = np.empty((len(idx), dv), dtype=np.float64)
            l = np.empty((len(idx),), dtype=np.float64)
            rc = self.lib.oracle_attention_rows(_ptr(qh), _ptr(kh), _ptr(vh),
                                                _ptr(klh, ctypes.c_int32), int(bool(causal)),
                                                _radius(radius), 1, 1, Lq, Lk, dk, dv,
                                                _ptr(sel, ctypes.c_int64), len(idx),
                                                _ptr(o), _ptr(l), int(nthreads))
            if rc != 0:
                raise RuntimeError("oracle_attention_rows failed with code %d" % rc)
            out[idx] = o
            lse[idx] = l
        return out, lse


_default = None


def default() -> Oracle:
    """The oracle built from oracle/sdpa_oracle.c (compiled on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        _default = Oracle(LIBRARY)
    return _default


def attention(q, k, v, key_lengths=None, causal=False, return_weights=False, nthreads=0,
              radius=None):
    """Full fp64 attention; see Oracle.attention."""
    return default().attention(q, k, v, key_lengths, causal, return_weights, nthreads, radius)


def multihead(xq, xkv, wq, wk, wv, wo, h, key_lengths=None, causal=False, nthreads=0):
    """fp64 multi-head attention; see Oracle.multihead."""
    return default().multihead(xq, xkv, wq, wk, wv, wo, h, key_lengths, causal, nthreads)


def multihead_rows(xq, xkv, wq, wk, wv, wo, h, rows, key_lengths=None, causal=False, nthreads=0):
    """fp64 multi-head attention for selected (b, i) rows; see Oracle.multihead_rows."""
    return default().multihead_rows(xq, xkv, wq, wk, wv, wo, h, rows, key_lengths, causal,
                                    nthreads)


def attention_rows(q, k, v, rows, key_lengths=None, causal=False, nthreads=0, radius=None):
    """fp64 attention for selected (b, head, i) rows; see Oracle.attention_rows."""
    return default().attention_rows(q, k, v, rows, key_lengths, causal, nthreads, radius)
