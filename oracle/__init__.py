"""Plain, slow fp64 CPU oracle for causal grouped-query softmax attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check of the entry
module and the CPU-baseline leg of the benchmark may import this package.
The product path (the HIP library and its Python binding) never imports,
calls or links anything here, and nothing here imports the product path.

What it computes (RL.cu project pages: pitchhut "Project Highlights" and
mlllm.io "What happened" name hand-written FlashAttention-2 forward and
backward kernels; pitchhut "Key Features" items 1-2 name FP16 inputs with
FP32 accumulation and a paged key/value cache in the inference engine).
FlashAttention-2 is an exact method, so the oracle is the plain definition
of masked softmax attention, evaluated naively in float64:

* ``attn_fwd_ref``   -- causal GQA forward over packed variable-length
  sequences: O and the natural-log log-sum-exp of the scaled scores.
* ``attn_bwd_ref``   -- its analytic backward (dQ, dK, dV) for a cotangent
  on O only.
* ``attn_decode_ref`` -- one query token per sequence attending to its whole
  context held in a paged key/value pool.
* ``kv_append_ref`` and ``attn_prefill_ref`` -- the rollout engine's chunked
  prefill: new tokens written into the paged pool, then causal attention of
  the new queries against the whole paged context.
* ``rmsnorm_fwd_ref`` and ``rmsnorm_bwd_ref`` (module ``oracle.rmsnorm``) --
  RMSNorm, the layer operation next to attention, and its backward.
* ``sample_ref`` (module ``oracle.sampling``) -- temperature / top-k / top-p
  sampling over logits with a caller-supplied uniform.
* ``rope_ref`` and ``rope_tables_ref`` (module ``oracle.rope``) -- rotary
  position embedding of q and k and its inverse (the backward).

Every function is pinned by tests that do not re-use its formulas: closed
forms, invariants, finite differences, a hand-derived worked example and
PyTorch's own CPU fp64 attention routine.
"""
from .attention import (  # noqa: F401
    attn_fwd_ref,
    attn_bwd_ref,
    attn_decode_ref,
    attn_prefill_ref,
    kv_append_ref,
    kv_head_of,
)
from .rmsnorm import rmsnorm_bwd_ref, rmsnorm_fwd_ref  # noqa: F401,E402
from .sampling import sample_ref  # noqa: F401,E402
from .rope import (  # noqa: F401,E402
    chunk_positions,
    rope_fp16_ref,
    rope_ref,
    rope_tables_ref,
    varlen_positions,
)
