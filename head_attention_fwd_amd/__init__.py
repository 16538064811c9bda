"""libsdpa: MI355X-native multi-head scaled dot-product attention, forward pass.

softmax(Q K^T / sqrt(d_k) + mask) V over h heads (page "Attention Is All You
Need/paper/es", §3.2.1 Eq. (1), §3.2.2, §3.2.3), computed by hand-written HIP
kernels for gfx950 behind the C ABI of include/sdpa.h.  This package is the
thin Python binding of that library; it loads head_attention_fwd_amd/libsdpa.so
on first use and raises if it is missing.
"""
from ._binding import *  # noqa: F401,F403 -- the public names listed in _binding.__all__
from ._binding import __all__  # noqa: F401
