"""Causal grouped-query attention for MI355X (gfx950).

FlashAttention-2-style forward and backward over packed variable-length
fp16 sequences, a paged-KV single-token decode, and the chunked prefill over
the paged cache (key/value append plus causal attention of the new tokens),
as hand-written HIP kernels behind the C ABI declared in include/attn.h.
``fwd``, ``bwd``, ``decode_paged``, ``kv_append`` and ``prefill_paged`` are
thin ctypes wrappers of attn_fwd, attn_bwd, attn_decode_paged,
attn_kv_append and attn_prefill_paged; the shared library is loaded on first
use and every call raises if it is missing. ``decode_paged_noalloc`` wraps
attn_decode_paged_noalloc, the decode for callers that cannot allocate.
``rmsnorm_fwd`` / ``rmsnorm_bwd`` wrap attn_rmsnorm_fwd / attn_rmsnorm_bwd,
the layer normalisation next to attention. ``rope_tables`` / ``rope`` wrap attn_rope_tables_init / attn_rope
(rotary position embedding of q and k, and its inverse); ``kv_append`` and
``prefill_paged`` take ``rope=(cos, sin)`` to rotate inside those kernels.
"""
from .attn import (  # noqa: F401
    AttnError,
    NormDims,
    PagedDims,
    PrefillDims,
    VarlenDims,
    bwd,
    bwd_workspace_bytes,
    decode_paged,
    decode_paged_noalloc,
    decode_workspace_bytes,
    fwd,
    kv_append,
    load_library,
    paged_dims,
    prefill_dims,
    prefill_paged,
    RopeTables,
    rope,
    rope_tables,
    rmsnorm_bwd,
    rmsnorm_bwd_workspace_bytes,
    rmsnorm_fwd,
    sample,
    varlen_dims,
)
