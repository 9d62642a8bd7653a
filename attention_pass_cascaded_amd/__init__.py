"""Single-pass fused cascaded-reduction attention for AMD MI355X (gfx950).

The product is the C-ABI library ``librfattn.so`` (``include/rf_attn.h``),
built from the HIP sources in ``csrc/``.  This package is its thin Python
binding: ``fwd``, ``bwd``, ``splitkv_fwd``, ``lse_merge``, ``decode`` and ``rope_rotate`` marshal torch
tensors (device memory and the current stream) into the C calls.
"""
from ._binding import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    RFError,
    bwd,
    bwd_noalloc,
    decode,
    fwd,
    fwd_prerotated,
    layernorm,
    softmax_topk,
    rope_rotate,
    load_library,
    lse_merge,
    num_splits_for,
    splitkv_fwd,
    workspace_bytes,
)

__all__ = ["fwd", "bwd", "bwd_noalloc", "splitkv_fwd", "lse_merge", "decode", "rope_rotate", "fwd_prerotated", "layernorm", "softmax_topk", "workspace_bytes", "num_splits_for", "load_library",
           "RFError", "LIB_PATH", "EXPORTED"]
