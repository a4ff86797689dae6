"""Causal grouped-query attention for MI355X (gfx950).

FlashAttention-2-style forward and backward over packed variable-length
fp16 sequences and a paged-KV single-token decode, as hand-written HIP
kernels behind the C ABI declared in include/attn.h. ``fwd``, ``bwd`` and
``decode_paged`` are thin ctypes wrappers of attn_fwd, attn_bwd and
attn_decode_paged; the shared library is loaded on first use and every call
raises if it is missing.
"""
from .attn import (  # noqa: F401
    AttnError,
    PagedDims,
    VarlenDims,
    bwd,
    bwd_workspace_bytes,
    decode_paged,
    decode_workspace_bytes,
    fwd,
    load_library,
    paged_dims,
    varlen_dims,
)
