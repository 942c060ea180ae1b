"""libzeros: ZeroS (zero-sum linear attention) forward pass for MI355X (gfx950).

The compute path is the HIP library libzeros.so (C ABI in include/zeros.h); this package is its
Python binding. Importing it does not load the library; the first call does, and fails loudly if
the library is missing.
"""
from ._lib import (  # noqa: F401
    DecodeState,
    ZerosError,
    load_library,
    zeros_bwd_causal,
    zeros_bwd_causal_workspace_bytes,
    zeros_decode_step,
    zeros_fwd_causal,
    zeros_fwd_causal_noalloc,
    zeros_fwd_causal_workspace_bytes,
    zeros_fwd_encoder,
    zeros_fwd_encoder_workspace_bytes,
    zeros_sm_fwd_causal,
    zeros_sm_fwd_causal_workspace_bytes,
)
