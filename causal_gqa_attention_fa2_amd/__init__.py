"""Causal grouped-query attention for MI355X (gfx950).

FlashAttention-2-style forward and backward over packed variable-length
fp16 sequences and a paged-KV single-token decode, as hand-written HIP
kernels behind the C ABI declared in include/attn.h.
"""
