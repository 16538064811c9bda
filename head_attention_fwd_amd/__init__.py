"""libsdpa: MI355X-native multi-head scaled dot-product attention, forward pass.

softmax(Q K^T / sqrt(d_k) + mask) V over h heads (page "Attention Is All You
Need/paper/es", §3.2.1 Eq. (1), §3.2.2, §3.2.3), computed by hand-written HIP
kernels for gfx950 behind the C ABI of include/sdpa.h.  This package is the
thin Python binding of that library; it loads head_attention_fwd_amd/libsdpa.so
on first use and raises if it is missing.
"""
from ._binding import (  # noqa: F401
    DECODE_NOALLOC_SCRATCH_BYTES,
    EXPORTED,
    LIBRARY,
    SDPA_BF16,
    SDPA_ERR_ALIAS,
    SDPA_ERR_BAD_SHAPE,
    SDPA_ERR_HIP,
    SDPA_ERR_NULL_POINTER,
    SDPA_ERR_SCRATCH_LIMIT,
    SDPA_ERR_UNSUPPORTED,
    SDPA_ERR_WORKSPACE,
    SDPA_F32,
    SDPA_OK,
    SdpaError,
    decode,
    decode_noalloc,
    forward,
    load_library,
    multihead,
    sdpa_decode,
    sdpa_decode_noalloc,
    sdpa_decode_workspace_bytes,
    restricted,
    sdpa_forward,
    sdpa_forward_restricted,
    sdpa_last_hip_error,
    sdpa_multihead_forward,
    sdpa_multihead_workspace_bytes,
    sdpa_status_str,
)
