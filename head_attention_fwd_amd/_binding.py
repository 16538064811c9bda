"""ctypes binding of libsdpa (include/sdpa.h): argument marshalling only.

Every step of the computation runs in the HIP kernels of libsdpa.so.  PyTorch
tensors only provide device memory and the stream.  If libsdpa.so is missing
or fails to load, every call raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libsdpa.so")

SDPA_OK = 0
SDPA_ERR_NULL_POINTER = 1
SDPA_ERR_BAD_SHAPE = 2
SDPA_ERR_UNSUPPORTED = 3
SDPA_ERR_ALIAS = 4
SDPA_ERR_HIP = 5
SDPA_ERR_WORKSPACE = 6
SDPA_ERR_SCRATCH_LIMIT = 7

#: SDPA_DECODE_NOALLOC_SCRATCH_BYTES of include/sdpa.h: the static device
#: scratch of sdpa_decode_noalloc, per device.
DECODE_NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024

SDPA_F32 = 0
SDPA_BF16 = 1

#: Symbols include/sdpa.h declares.
EXPORTED = ("sdpa_decode", "sdpa_decode_noalloc", "sdpa_decode_workspace_bytes", "sdpa_forward",
            "sdpa_forward_restricted", "sdpa_last_hip_error", "sdpa_multihead_forward",
            "sdpa_multihead_workspace_bytes", "sdpa_status_str")

# the package's public names (head_attention_fwd_amd re-exports exactly these)
__all__ = [
    "DECODE_NOALLOC_SCRATCH_BYTES", "EXPORTED", "LIBRARY", "SDPA_BF16", "SDPA_ERR_ALIAS",
    "SDPA_ERR_BAD_SHAPE", "SDPA_ERR_HIP", "SDPA_ERR_NULL_POINTER", "SDPA_ERR_SCRATCH_LIMIT",
    "SDPA_ERR_UNSUPPORTED", "SDPA_ERR_WORKSPACE", "SDPA_F32", "SDPA_OK", "SdpaError", "decode",
    "decode_noalloc", "forward", "load_library", "multihead", "restricted", "sdpa_decode",
    "sdpa_decode_noalloc", "sdpa_decode_workspace_bytes", "sdpa_forward", "sdpa_forward_restricted",
    "sdpa_last_hip_error", "sdpa_multihead_forward", "sdpa_multihead_workspace_bytes",
    "sdpa_status_str",
]

_lib = None


class SdpaError(RuntimeError):
    """A non-zero sdpa_status returned by the library."""

    def __init__(self, status: int, message: str, entry: str = "sdpa_forward"):
        super().__init__("%s failed (%d): %s" % (entry, status, message))
        self.status = status


def load_library(path: str = LIBRARY):
    """Load libsdpa.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libsdpa.so is not built (%s); run __graft_entry__.build() or "
                           "python head_attention_fwd_amd/build.py" % path)
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.sdpa_forward.restype = ctypes.c_int
    lib.sdpa_forward.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, i64, i64, i64, i64, i64,
                                 i64, ctypes.c_int, vp]
    lib.sdpa_forward_restricted.restype = ctypes.c_int
    lib.sdpa_forward_restricted.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, vp, i64, i64, i64,
                                            i64, i64, i64, ctypes.c_int, vp]
    lib.sdpa_multihead_forward.restype = ctypes.c_int
    lib.sdpa_multihead_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, i64, i64,
                                           i64, i64, i64, i64, i64, ctypes.c_int, vp, i64, vp]
    lib.sdpa_multihead_workspace_bytes.restype = i64
    lib.sdpa_multihead_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i64, ctypes.c_int]
    lib.sdpa_decode.restype = ctypes.c_int
    lib.sdpa_decode.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                vp, i64, vp]
    lib.sdpa_decode_noalloc.restype = ctypes.c_int
    lib.sdpa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                        ctypes.c_int, vp]
    lib.sdpa_decode_workspace_bytes.restype = i64
    lib.sdpa_decode_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int]
    lib.sdpa_status_str.restype = ctypes.c_char_p
    lib.sdpa_status_str.argtypes = [ctypes.c_int]
    lib.sdpa_last_hip_error.restype = ctypes.c_int
    lib.sdpa_last_hip_error.argtypes = []
    _lib = lib
    return lib


def sdpa_forward(Q: int, K: int, V: int, key_lengths: int, causal: int, out: int,
                 B: int, H: int, Lq: int, Lk: int, d_k: int, d_v: int, dtype: int,
                 stream: int) -> int:
    """Raw C call; pointers and the stream are integers (0 = NULL).  Returns the status."""
    return load_library().sdpa_forward(Q or None, K or None, V or None, key_lengths or None,
                                       int(causal), out or None, B, H, Lq, Lk, d_k, d_v,
                                       int(dtype), stream or None)


def sdpa_forward_restricted(Q: int, K: int, V: int, key_lengths: int, causal: int, radius: int,
                            out: int, B: int, H: int, Lq: int, Lk: int, d_k: int, d_v: int,
                            dtype: int, stream: int) -> int:
    """Raw C call; pointers and the stream are integers (0 = NULL).  Returns the status."""
    return load_library().sdpa_forward_restricted(Q or None, K or None, V or None,
                                                  key_lengths or None, int(causal), int(radius),
                                                  out or None, B, H, Lq, Lk, d_k, d_v, int(dtype),
                                                  stream or None)


def sdpa_multihead_forward(Xq: int, Xkv: int, Wq: int, Wk: int, Wv: int, Wo: int,
                           key_lengths: int, causal: int, out: int, B: int, Lq: int, Lk: int,
                           d_model: int, h: int, d_k: int, d_v: int, dtype: int, workspace: int,
                           workspace_bytes: int, stream: int) -> int:
    """Raw C call; pointers and the stream are integers (0 = NULL).  Returns the status."""
    return load_library().sdpa_multihead_forward(
        Xq or None, Xkv or None, Wq or None, Wk or None, Wv or None, Wo or None,
        key_lengths or None, int(causal), out or None, B, Lq, Lk, d_model, h, d_k, d_v,
        int(dtype), workspace or None, workspace_bytes, stream or None)


def sdpa_multihead_workspace_bytes(B: int, Lq: int, Lk: int, d_model: int, h: int, d_k: int,
                                   d_v: int, dtype: int) -> int:
    return load_library().sdpa_multihead_workspace_bytes(B, Lq, Lk, d_model, h, d_k, d_v,
                                                         int(dtype))


def sdpa_decode(Q: int, K: int, V: int, key_lengths: int, out: int, B: int, H: int, Lq: int,
                Lk: int, d_k: int, d_v: int, dtype: int, workspace: int, workspace_bytes: int,
                stream: int) -> int:
    """Raw C call; pointers and the stream are integers (0 = NULL).  Returns the status."""
    return load_library().sdpa_decode(Q or None, K or None, V or None, key_lengths or None,
                                      out or None, B, H, Lq, Lk, d_k, d_v, int(dtype),
                                      workspace or None, workspace_bytes, stream or None)


def sdpa_decode_noalloc(Q: int, K: int, V: int, key_lengths: int, out: int, B: int, H: int,
                        Lq: int, Lk: int, d_k: int, d_v: int, dtype: int, stream: int) -> int:
    """Raw C call; pointers and the stream are integers (0 = NULL).  Returns the status."""
    return load_library().sdpa_decode_noalloc(Q or None, K or None, V or None,
                                              key_lengths or None, out or None, B, H, Lq, Lk,
                                              d_k, d_v, int(dtype), stream or None)


def sdpa_decode_workspace_bytes(B: int, H: int, Lq: int, Lk: int, d_k: int, d_v: int,
                                dtype: int) -> int:
    return load_library().sdpa_decode_workspace_bytes(B, H, Lq, Lk, d_k, d_v, int(dtype))


def sdpa_status_str(status: int) -> str:
    return load_library().sdpa_status_str(int(status)).decode()


def sdpa_last_hip_error() -> int:
    return load_library().sdpa_last_hip_error()


def _check(q, k, v, key_lengths, out):
    """Validate torch tensors for the calls below; returns (sizes, dtype code, key_lengths, out)."""
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, L, d]")
    B, H, Lq, d_k = q.shape
    Lk = k.shape[2]
    d_v = v.shape[3]
    if tuple(k.shape) != (B, H, Lk, d_k) or tuple(v.shape) != (B, H, Lk, d_v):
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape),
                                                             tuple(v.shape)))
    if q.dtype == torch.bfloat16:
        dtype = SDPA_BF16
    elif q.dtype == torch.float32:
        dtype = SDPA_F32
    else:
        raise TypeError("unsupported dtype %s" % q.dtype)
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype or t.device != dev:
            raise ValueError("%s must match q in dtype and device" % name)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if key_lengths is not None and not isinstance(key_lengths, torch.Tensor):
        key_lengths = torch.as_tensor(list(key_lengths), dtype=torch.int32, device=dev)
    if key_lengths is not None:
        if key_lengths.dtype != torch.int32 or key_lengths.device != dev or \
                tuple(key_lengths.shape) != (B,) or not key_lengths.is_contiguous():
            raise ValueError("key_lengths must be a contiguous int32 [B] tensor on q's device")
    if out is None:
        out = torch.empty((B, H, Lq, d_v), dtype=q.dtype, device=dev)
    elif tuple(out.shape) != (B, H, Lq, d_v) or out.dtype != q.dtype or out.device != dev or \
            not out.is_contiguous():
        raise ValueError("out must be a contiguous [B,H,Lq,d_v] tensor like q")
    return (B, H, Lq, Lk, d_k, d_v), dtype, key_lengths, out


def _check_workspace(workspace, dev):
    """A caller-given workspace: a contiguous tensor on the calls' device (its size in
    bytes is checked by the library)."""
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")


def _raise(st, entry):
    if st != SDPA_OK:
        msg = sdpa_status_str(st)
        if st == SDPA_ERR_HIP:
            msg += " (hipError %d)" % sdpa_last_hip_error()
        raise SdpaError(st, msg, entry)


def forward(q, k, v, key_lengths=None, causal: bool = False, out=None):
    """Attention forward on torch CUDA tensors (HIP on ROCm).

    q [B,H,Lq,d_k], k [B,H,Lk,d_k], v [B,H,Lk,d_v]: contiguous, one dtype
    (torch.float32 or torch.bfloat16), one device.  key_lengths: None, or an
    int32 tensor [B] on that device (other integer sequences are copied there).
    out: optional preallocated contiguous [B,H,Lq,d_v] tensor of the same dtype.
    The kernel is enqueued on the device's current stream; returns out.
    """
    import torch

    (B, H, Lq, Lk, d_k, d_v), dtype, key_lengths, out = _check(q, k, v, key_lengths, out)
    dev = q.device
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = sdpa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                          0 if key_lengths is None else key_lengths.data_ptr(), int(bool(causal)),
                          out.data_ptr(), B, H, Lq, Lk, d_k, d_v, dtype, stream)
    _raise(st, "sdpa_forward")
    return out


def restricted(q, k, v, radius: int, key_lengths=None, causal: bool = False, out=None):
    """Restricted self-attention (sdpa_forward_restricted): forward() with key j
    also illegal for query i when |i - j| > radius.  Tensors as for forward()."""
    import torch

    (B, H, Lq, Lk, d_k, d_v), dtype, key_lengths, out = _check(q, k, v, key_lengths, out)
    dev = q.device
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = sdpa_forward_restricted(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     0 if key_lengths is None else key_lengths.data_ptr(),
                                     int(bool(causal)), int(radius), out.data_ptr(), B, H, Lq, Lk,
                                     d_k, d_v, dtype, stream)
    _raise(st, "sdpa_forward_restricted")
    return out


def multihead(xq, xkv, wq, wk, wv, wo, h: int, key_lengths=None, causal: bool = False, out=None,
              workspace=None):
    """MultiHead(Q, K, V) = Concat(head_1..head_h) W^O (sdpa_multihead_forward).

    xq [B, Lq, d_model], xkv [B, Lk, d_model] (pass xq itself for
    self-attention), wq and wk [d_model, h*d_k], wv [d_model, h*d_v],
    wo [h*d_v, d_model]: contiguous torch.bfloat16 tensors on one GPU.
    key_lengths, causal as for forward().  workspace: optional uint8 tensor of
    at least sdpa_multihead_workspace_bytes(...) bytes (allocated here if None).
    Returns out [B, Lq, d_model].
    """
    import torch

    if int(h) < 1:
        raise ValueError("h must be at least 1")
    if xq.dim() != 3 or xkv.dim() != 3:
        raise ValueError("xq and xkv must be [B, L, d_model]")
    B, Lq, dm = xq.shape
    Lk = xkv.shape[1]
    if tuple(xkv.shape) != (B, Lk, dm) or wq.dim() != 2 or wq.shape[0] != dm or wq.shape[1] % h:
        raise ValueError("inconsistent shapes")
    dk, dv = wq.shape[1] // h, wv.shape[1] // h
    if tuple(wk.shape) != (dm, h * dk) or tuple(wv.shape) != (dm, h * dv) or \
            tuple(wo.shape) != (h * dv, dm):
        raise ValueError("inconsistent weight shapes")
    dev = xq.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    for name, t in (("xq", xq), ("xkv", xkv), ("wq", wq), ("wk", wk), ("wv", wv), ("wo", wo)):
        if t.dtype != torch.bfloat16 or t.device != dev or not t.is_contiguous():
            raise ValueError("%s must be a contiguous bfloat16 tensor on xq's device" % name)
    if key_lengths is not None and not isinstance(key_lengths, torch.Tensor):
        key_lengths = torch.as_tensor(list(key_lengths), dtype=torch.int32, device=dev)
    if key_lengths is not None and (key_lengths.dtype != torch.int32 or key_lengths.device != dev
                                    or tuple(key_lengths.shape) != (B,)
                                    or not key_lengths.is_contiguous()):
        raise ValueError("key_lengths must be a contiguous int32 [B] tensor on xq's device")
    if out is None:
        out = torch.empty((B, Lq, dm), dtype=torch.bfloat16, device=dev)
    elif tuple(out.shape) != (B, Lq, dm) or out.dtype != torch.bfloat16 or out.device != dev or \
            not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 [B, Lq, d_model] tensor")
    need = sdpa_multihead_workspace_bytes(B, Lq, Lk, dm, h, dk, dv, SDPA_BF16)
    if need < 0:
        raise SdpaError(SDPA_ERR_UNSUPPORTED, "sizes rejected", "sdpa_multihead_forward")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_workspace(workspace, dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = sdpa_multihead_forward(xq.data_ptr(), xkv.data_ptr(), wq.data_ptr(), wk.data_ptr(),
                                    wv.data_ptr(), wo.data_ptr(),
                                    0 if key_lengths is None else key_lengths.data_ptr(),
                                    int(bool(causal)), out.data_ptr(), B, Lq, Lk, dm, h, dk, dv,
                                    SDPA_BF16, workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), stream)
    _raise(st, "sdpa_multihead_forward")
    return out


def decode(q, k, v, key_lengths=None, out=None, workspace=None):
    """Decode-step attention (sdpa_decode): the result of forward(..., causal=False)
    for a few query rows per head against a long key/value cache.

    Tensors as for forward().  workspace: optional uint8 tensor on the device of
    at least sdpa_decode_workspace_bytes(...) bytes; allocated here when None.
    Returns out.
    """
    import torch

    (B, H, Lq, Lk, d_k, d_v), dtype, key_lengths, out = _check(q, k, v, key_lengths, out)
    dev = q.device
    need = sdpa_decode_workspace_bytes(B, H, Lq, Lk, d_k, d_v, dtype)
    if need < 0:
        raise SdpaError(SDPA_ERR_BAD_SHAPE, "sizes rejected", "sdpa_decode")
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check_workspace(workspace, dev)
    ws_ptr = 0 if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = sdpa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                         0 if key_lengths is None else key_lengths.data_ptr(), out.data_ptr(),
                         B, H, Lq, Lk, d_k, d_v, dtype, ws_ptr, ws_bytes, stream)
    _raise(st, "sdpa_decode")
    return out


def decode_noalloc(q, k, v, out, key_lengths=None):
    """sdpa_decode_noalloc: decode() without a workspace and without any allocation.

    The split partial results go to the library's static device scratch
    (DECODE_NOALLOC_SCRATCH_BYTES per device; larger requests raise SdpaError
    with SDPA_ERR_SCRATCH_LIMIT).  out (the [B,H,Lq,d_v] result) is required and
    key_lengths must be None or an int32 [B] tensor on the inputs' device, so that
    nothing is allocated here either.  Calls on one device that may overlap in
    time race on that scratch.  Returns out.
    """
    import torch

    if out is None:
        raise ValueError("decode_noalloc needs a preallocated out tensor")
    if key_lengths is not None and not isinstance(key_lengths, torch.Tensor):
        raise ValueError("decode_noalloc needs key_lengths as a device tensor (or None)")
    (B, H, Lq, Lk, d_k, d_v), dtype, key_lengths, out = _check(q, k, v, key_lengths, out)
    dev = q.device
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = sdpa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                 0 if key_lengths is None else key_lengths.data_ptr(),
                                 out.data_ptr(), B, H, Lq, Lk, d_k, d_v, dtype, stream)
    _raise(st, "sdpa_decode_noalloc")
    return out
