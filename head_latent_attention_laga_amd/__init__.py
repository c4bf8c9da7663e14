"""LAGA (Latent All-Gather Attention) per-rank hot path for MI355X (gfx950).

The compute lives in liblaga.so (hand-written HIP kernels behind the C ABI of
include/laga.h); this package only binds it and allocates device buffers.
"""
from ._lib import (  # noqa: F401
    LAGA_BF16,
    LAGA_F32,
    LAGA_OPERANDS_FP16,
    LAGA_OPERANDS_SPLIT,
    LagaError,
    attn_bwd,
    attn_bwd_workspace_bytes,
    attn_fwd,
    kv_elem_bytes,
    kv_up,
    latent_norm,
    load,
    make_dims,
)
from .path import LagaPath  # noqa: F401
