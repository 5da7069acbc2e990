"""MI355X-native fused causal flash-attention, forward and backward.

The computation lives in libxfa.so (hand-written HIP for gfx950, C ABI in
include/xfa.h); this package is its thin Python binding.
"""

from ._binding import (  # noqa: F401
    LIB_PATH,
    XFA_DTYPE_BF16,
    XFA_DTYPE_F32,
    XFA_ERR_HIP,
    XFA_ERR_INVALID_ARGUMENT,
    XFA_ERR_UNSUPPORTED,
    XFA_OK,
    XfaError,
    backward,
    forward,
    lib,
    xfa_bwd,
    xfa_bwd_dropout,
    xfa_bwd_preprocess,
    xfa_bwd_workspace_bytes,
    xfa_fwd,
    xfa_fwd_dropout,
    xfa_status_string,
)

from .autograd import CORES, FlashAttentionFn, flash_attention  # noqa: E402,F401

# short names: out, lse = fwd(q, k, v, scale=None, causal=True);
# dq, dk, dv = bwd(q, k, v, out, dout, lse, scale=None, causal=True)
fwd = forward
bwd = backward
