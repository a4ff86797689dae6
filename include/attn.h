/*
 * attn.h -- C ABI of the MI355X (gfx950) causal grouped-query attention library.
 *
 * What the library computes. The RL.cu project pages (pitchhut "Project
 * Highlights"; mlllm.io "What happened") name hand-written FlashAttention-2
 * forward and backward kernels and an inference engine with a paged key/value
 * cache (pitchhut "Key Features", items 1-2), with FP16 inputs and FP32
 * accumulation (pitchhut "Key Features", item 1). FlashAttention-2 is exact
 * softmax attention, so every entry point below returns, up to floating-point
 * rounding, the plain definition:
 *
 *   S_ij = scale * <q_i, k_j>  for key position j <= query position i
 *          (positions counted from the start of each packed sequence),
 *   LSE_i = ln sum_j exp(S_ij),   O_i = sum_j exp(S_ij - LSE_i) v_j,
 *
 * with query head h reading key/value head h / (h_q / h_kv) (contiguous
 * grouped-query groups). Attention never crosses a sequence boundary.
 *
 * Conventions shared by every entry point.
 *  - Tensor arguments are DEVICE pointers to dense row-major arrays; fp16 is
 *    IEEE binary16, fp32 is IEEE binary32. Every tensor pointer must be
 *    16-byte aligned.
 *  - The caller owns every buffer (inputs, outputs, workspace). The library
 *    never allocates, frees or keeps a pointer after the call returns, never
 *    synchronizes and never copies device data to the host. The one
 *    library-held buffer is the fixed device array of
 *    attn_decode_paged_noalloc, part of the loaded code itself.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL means the null
 *    stream) and the call returns before it finishes. Calls are stateless and
 *    may be captured into a HIP graph.
 *  - Argument checks run before any HIP call. A failed check returns a
 *    status code and enqueues nothing. A launch failure reported by the HIP
 *    runtime returns ATTN_ERR_HIP. Faults inside kernels surface at the
 *    caller's next synchronization. Nothing aborts or throws across the ABI.
 *  - The contents of device index arrays (cu_seqlens, block_table, ctx_lens)
 *    are NOT checked by the compute entry points; attn_check_cu_seqlens and
 *    attn_check_paged check host copies of them.
 */
#ifndef CGQA_ATTN_H
#define CGQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer  */
    ATTN_ERR_UNSUPPORTED = 2, /* head_dim not 64/128, group size above 16,
                                 block size not 16, or a batch too large for
                                 32-bit indexing: total_tokens * h_q or
                                 ceil(max_seqlen / 32) * n_seqs * h_q above
                                 INT32_MAX                                   */
    ATTN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required  */
    ATTN_ERR_HIP = 4          /* the HIP runtime reported a launch error     */
} attn_status;

/* Shape of a packed variable-length batch of n_seqs sequences.
 *   total_tokens = cu_seqlens[n_seqs] (T), max_seqlen = max sequence length,
 *   h_q query heads, h_kv key/value heads (h_q % h_kv == 0, h_q / h_kv <= 16),
 *   head_dim in {64, 128}.
 * total_tokens and max_seqlen are host copies so no device read is needed to
 * size the launch; they must agree with cu_seqlens. n_seqs = 0 or
 * total_tokens = 0 is a valid empty batch (nothing is enqueued). */
typedef struct attn_varlen_dims {
    int32_t n_seqs;
    int32_t total_tokens;
    int32_t max_seqlen;
    int32_t h_q;
    int32_t h_kv;
    int32_t head_dim;
} attn_varlen_dims;

/* Shape of a paged decode batch: n_seqs sequences with one query token each,
 * pools of num_blocks blocks of block_size (= 16) tokens, a block table of
 * max_blocks_per_seq entries per sequence, and max_ctx_len >= every ctx_lens
 * entry (host copy, sizes the launch and the workspace). */
typedef struct attn_paged_dims {
    int32_t n_seqs;
    int32_t h_q;
    int32_t h_kv;
    int32_t head_dim;
    int32_t block_size;
    int32_t max_blocks_per_seq;
    int32_t num_blocks;
    int32_t max_ctx_len;
} attn_paged_dims;

/*
 * attn_fwd -- causal GQA attention forward over a packed varlen batch
 * (FlashAttention-2 forward: online softmax, saved log-sum-exp; pitchhut
 * "Project Highlights").
 *   q          fp16 [T, h_q, d]          queries
 *   k, v       fp16 [T, h_kv, d]         keys, values
 *   cu_seqlens int32 [n_seqs + 1]        0 = cu[0] <= cu[1] <= ... = T
 *   scale      multiplies q.k before the softmax (usually 1/sqrt(d))
 *   o          fp16 [T, h_q, d]          output, fully overwritten
 *   lse        fp32 [h_q, T]             natural-log log-sum-exp of the scaled
 *                                        scores of each (head, token) row,
 *                                        fully overwritten; attn_bwd needs it
 * Rounding: fp32 accumulation, softmax weights rounded to fp16 before the
 * weighted sum of values, O rounded to nearest-even fp16.
 * Runs are bitwise reproducible for identical inputs.
 */
attn_status attn_fwd(const attn_varlen_dims* dims, const void* q, const void* k,
                     const void* v, const int32_t* cu_seqlens, float scale, void* o,
                     float* lse, void* stream);

/* Bytes of device workspace attn_bwd needs for `dims` (0 for an empty
 * batch). Holds two fp32 [h_q, T] arrays of per-row terms: -D = -rowsum(dO * O)
 * and LSE * log2(e). For batches of very unequal lengths (n_seqs >= 2 and
 * n_seqs * max_seqlen >= 1.25 total_tokens) it also holds fp16 dS blocks,
 * n_seqs * h_q * ceil(max_seqlen / 32)^2 * 2 KiB (when that is at most
 * 4 GiB): the backward then stores dS once instead of recomputing it for dQ.
 * The result depends on dims only. */
size_t attn_bwd_workspace_bytes(const attn_varlen_dims* dims);

/*
 * attn_bwd -- backward of attn_fwd for the loss <O, dO> (FlashAttention-2
 * backward, dQ/dK/dV by recomputing the softmax from the saved LSE; pitchhut
 * "Project Highlights", gradient checkpointing in "Key Features" item 3).
 *   q, k, v, cu_seqlens, scale   as given to attn_fwd (same scale)
 *   o          fp16 [T, h_q, d]   attn_fwd's output
 *   lse        fp32 [h_q, T]      attn_fwd's log-sum-exp
 *   dO         fp16 [T, h_q, d]   cotangent of O (no cotangent on the LSE)
 *   dq         fp16 [T, h_q, d]   outputs, fully overwritten (no zeroing
 *   dk, dv     fp16 [T, h_kv, d]  needed); dk and dv sum over the group's
 *                                 query heads
 *   workspace  device buffer of at least attn_bwd_workspace_bytes(dims)
 *              bytes, 256-byte aligned; the library initialises it.
 * No atomics are used: dq, dk and dv are bitwise reproducible for identical
 * inputs.
 */
attn_status attn_bwd(const attn_varlen_dims* dims, const void* q, const void* k,
                     const void* v, const void* o, const float* lse, const void* dO,
                     const int32_t* cu_seqlens, void* dq, void* dk, void* dv, float scale,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace attn_decode_paged needs for `dims`: fp32
 * partial outputs, maxima and sums of the context splits, and the int32 work
 * plan (per-sequence block offsets). The library initialises it. */
size_t attn_decode_workspace_bytes(const attn_paged_dims* dims);

/*
 * attn_decode_paged -- single-token decode attention over a paged key/value
 * cache (the rollout engine's "paged key-value caching"; pitchhut "Key
 * Features" item 2, mlllm.io "What happened").
 *   q           fp16 [n, h_q, d]            one query token per sequence
 *   k_pool      fp16 [num_blocks, 16, h_kv, d]   key pool
 *   v_pool      fp16 [num_blocks, 16, h_kv, d]   value pool
 *   block_table int32 [n, max_blocks_per_seq]  physical block of each logical
 *               block; entries past ceil(ctx/16) are never read
 *   ctx_lens    int32 [n]   context length of each sequence (0..max_ctx_len)
 *   o           fp16 [n, h_q, d]   output, fully overwritten; a zero-length
 *               context yields a zero row
 *   scale       multiplies q.k (usually 1/sqrt(d))
 *   workspace   at least attn_decode_workspace_bytes(dims) bytes
 * Position t of sequence b is slot t % 16 of block block_table[b][t / 16].
 * Blocks past ceil(ctx/16) are never read; slots past the context inside the
 * last block may be read but never influence o (even if they hold NaN).
 * Contents of ctx_lens and block_table are not validated (attn_check_paged
 * does that on host copies), but a context outside [0, max_ctx_len] is
 * clamped into it and a table entry outside [0, num_blocks) into that range,
 * so no access leaves the pools or the table rows (o is then undefined).
 * Returns ATTN_ERR_UNSUPPORTED when n_seqs * ceil(max_ctx_len / 16) exceeds
 * 2^30 (the device's block counts are int32).
 */
attn_status attn_decode_paged(const attn_paged_dims* dims, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* block_table,
                              const int32_t* ctx_lens, void* o, float scale, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged_noalloc -- attn_decode_paged for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, results and checks as
 * attn_decode_paged, minus the workspace: the work plan and the partials
 * live in a 32 MiB (33554432-byte) device array that the library holds, one
 * copy per device, from the first call on that device until the process
 * ends. The call itself allocates nothing.
 *   Returns ATTN_ERR_WORKSPACE, enqueuing nothing, when
 *   attn_decode_workspace_bytes(dims) exceeds 33554432 bytes (e.g. more than
 *   about 3500 sequences at h_q = 16, d = 128); ATTN_ERR_HIP if the device
 *   array's address cannot be looked up.
 *   Every call on one device shares that device's array and leaves its
 *   partials there; nothing in it needs to start at zero. Calls that may run
 *   at the same time on one device (different streams, or several host
 *   threads each with its own stream) race on it and give undefined output;
 *   calls on one stream are ordered and safe.
 */
attn_status attn_decode_paged_noalloc(const attn_paged_dims* dims, const void* q,
                                      const void* k_pool, const void* v_pool,
                                      const int32_t* block_table, const int32_t* ctx_lens,
                                      void* o, float scale, void* stream);

/* Shape of a chunked prefill over a paged cache: `paged` describes the
 * pools, the block table and the contexts (ctx_lens count each sequence's
 * context INCLUDING its new tokens; max_ctx_len bounds them); the new tokens
 * are packed by cu_q (int32 [n_seqs + 1], 0 = cu_q[0] <= ... = total_q) with
 * at most max_q_len per sequence (host copies that size the launch). */
typedef struct attn_prefill_dims {
    attn_paged_dims paged;
    int32_t total_q;
    int32_t max_q_len;
} attn_prefill_dims;

/*
 * attn_kv_append -- write the new keys and values of a chunked prefill into
 * the paged pools (the rollout engine's paged key/value cache; pitchhut "Key
 * Features" item 2).
 *   k_new, v_new fp16 [total_q, h_kv, d]  new keys / values packed by cu_q
 *   cu_q        int32 [n_seqs + 1]
 *   block_table int32 [n_seqs, max_blocks_per_seq]
 *   ctx_lens    int32 [n_seqs]   context lengths including the new tokens
 *   k_pool, v_pool fp16 [num_blocks, 16, h_kv, d]  updated in place
 * New token i of sequence b (L_b = cu_q[b+1] - cu_q[b] of them) is context
 * position t = ctx_lens[b] - L_b + i and lands in slot t % 16 of block
 * block_table[b][t / 16]. No other pool slot is written. A sequence whose
 * L_b exceeds its context is skipped (invalid input; attn_check_prefill
 * reports it). Table entries outside [0, num_blocks) and contexts above
 * max_ctx_len are clamped, so no access leaves the pools (the result is then
 * undefined). Each sequence's new positions must map to distinct slots.
 */
attn_status attn_kv_append(const attn_prefill_dims* dims, const void* k_new, const void* v_new,
                           const int32_t* cu_q, const int32_t* block_table,
                           const int32_t* ctx_lens, void* k_pool, void* v_pool, void* stream);

/*
 * attn_prefill_paged -- causal GQA attention of the new query tokens of a
 * chunked prefill against each sequence's whole context in the paged pools
 * (run after attn_kv_append has stored the chunk's keys and values).
 *   q           fp16 [total_q, h_q, d]   new queries packed by cu_q
 *   k_pool, v_pool fp16 [num_blocks, 16, h_kv, d]
 *   block_table, ctx_lens, cu_q   as for attn_kv_append
 *   o           fp16 [total_q, h_q, d]   output, fully overwritten
 *   lse         fp32 [h_q, total_q] natural-log log-sum-exp per row, or
 *               NULL when not needed
 * New token i of sequence b sits at context position
 * p = ctx_lens[b] - L_b + i and attends to positions 0..p (the same S, LSE
 * and O as attn_fwd, whose causal mask is the case ctx_lens[b] = L_b).
 * Positions past a sequence's context are never read. Rounding as attn_fwd;
 * bitwise reproducible. A sequence whose L_b exceeds its context is skipped
 * (its rows are left unwritten). Clamping of bad table entries and contexts
 * as for attn_kv_append.
 */
attn_status attn_prefill_paged(const attn_prefill_dims* dims, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_table,
                               const int32_t* ctx_lens, const int32_t* cu_q, void* o,
                               float* lse, float scale, void* stream);

/*
 * Rotary position embedding (RoPE) -- the rotation of queries and keys that
 * comes right before attention (the mlllm.io article, "What happened", lists
 * RoPE among the hand-written kernels). The pages print no formula; the
 * library uses the rotate-half pairing of Qwen3, the model the pages
 * benchmark: dimension j < d/2 of every head turns together with dimension
 * j + d/2 by the angle pos * theta_j,
 *   x'_j = x_j cos - x_{j+d/2} sin,   x'_{j+d/2} = x_{j+d/2} cos + x_j sin,
 * with cos / sin read from caller-owned fp32 tables [max_pos, d/2] (device
 * pointers, 16-byte aligned; row p holds position p; the library only reads
 * them). The rotations of q and k (attn_rope, attn_kv_append_rope,
 * attn_prefill_paged_rope, attn_decode_paged_rope) are computed in fp64 and
 * rounded once to fp16, so
 * their results are the same bits whichever entry point rotates; the inverse
 * rotation inside attn_bwd_rope works in fp32 (see there).
 * Errors of every RoPE entry point: ATTN_ERR_INVALID_ARG when rope is NULL,
 * a table pointer is NULL or not 16-byte aligned, max_pos < 1, or max_pos
 * does not cover the positions the call can form; all other checks are
 * those of the entry point without RoPE, made before any HIP call.
 */
typedef struct attn_rope_tables {
    const float* cos;
    const float* sin;
    int32_t max_pos;
} attn_rope_tables;

/*
 * attn_rope_tables_init -- fill cos / sin fp32 [max_pos, head_dim/2] with
 * cos(p * base^(-2j/head_dim)) and sin(...), evaluated in fp64 and rounded
 * to fp32. head_dim 64 or 128, base > 1 (Qwen3: 1e6), max_pos >= 1.
 */
attn_status attn_rope_tables_init(int32_t max_pos, int32_t head_dim, double base, float* cos,
                                  float* sin, void* stream);

/*
 * attn_rope -- rotate packed q [total_tokens, h_q, d] and k [total_tokens,
 * h_kv, d] (fp16, in place; either may be NULL) by their positions.
 *   ctx_lens == NULL: token i of a sequence (rows cu_seqlens[b] + i) is at
 *     position i (training over packed sequences; max_pos >= max_seqlen).
 *   ctx_lens != NULL: the tokens are the new chunk of a cached sequence, at
 *     positions ctx_lens[b] - L_b + i (max_ctx_len bounds ctx_lens; max_pos
 *     >= max_ctx_len); a sequence whose L_b exceeds its context is skipped.
 *   inverse != 0 applies the transposed rotation: the backward, which turns
 *     dq and dk of the rotated tensors into those of the unrotated ones.
 * Positions beyond the tables are clamped to max_pos - 1 (only reachable
 * with invalid ctx_lens). Bitwise deterministic.
 */
attn_status attn_rope(const attn_varlen_dims* dims, void* q, void* k, const int32_t* cu_seqlens,
                      const int32_t* ctx_lens, int32_t max_ctx_len, const attn_rope_tables* rope,
                      int32_t inverse, void* stream);

/*
 * attn_bwd_rope -- attn_bwd for attention whose q and k were rotated by
 * attn_rope (ctx_lens = NULL): q and k here are the rotated tensors, and dq
 * and dk are carried back to the unrotated ones by the inverse rotation at
 * their stores (token i of a sequence at position i), computed in fp32 from
 * the fp32 gradient and rounded once to fp16; dv is as attn_bwd's. It
 * replaces attn_bwd followed by attn_rope(..., inverse = 1) on dq and dk,
 * which rounds to fp16 twice (results agree to about one fp16 unit; unlike
 * the forward rotations this one is not bit-exact against a correctly
 * rounded reference). Same workspace as attn_bwd; rope->max_pos >=
 * max_seqlen.
 */
attn_status attn_bwd_rope(const attn_varlen_dims* dims, const void* q, const void* k,
                          const void* v, const void* o, const float* lse, const void* dO,
                          const int32_t* cu_seqlens, const attn_rope_tables* rope, void* dq,
                          void* dk, void* dv, float scale, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged_rope -- attn_decode_paged whose queries are rotated by
 * their positions ctx_lens[b] - 1 (the token being decoded is the last of
 * its context) as they are loaded; q itself is not modified, and the keys
 * in the pool are taken as already rotated (attn_kv_append_rope). O is
 * bitwise that of attn_rope on q (ctx_lens, one token per sequence)
 * followed by attn_decode_paged. rope->max_pos >= max_ctx_len.
 */
attn_status attn_decode_paged_rope(const attn_paged_dims* dims, const void* q,
                                   const void* k_pool, const void* v_pool,
                                   const int32_t* block_table, const int32_t* ctx_lens,
                                   const attn_rope_tables* rope, void* o, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_kv_append_rope -- attn_kv_append that rotates each new key by its
 * context position on its way into the pool (values are copied as they
 * are). The pool then holds the same bits as attn_rope on k_new (with
 * ctx_lens) followed by attn_kv_append. rope->max_pos >= max_ctx_len.
 */
attn_status attn_kv_append_rope(const attn_prefill_dims* dims, const void* k_new,
                                const void* v_new, const int32_t* cu_q,
                                const int32_t* block_table, const int32_t* ctx_lens,
                                const attn_rope_tables* rope, void* k_pool, void* v_pool,
                                void* stream);

/*
 * attn_prefill_paged_rope -- attn_prefill_paged whose queries are rotated by
 * their context positions as they are loaded (q itself is not modified);
 * the keys in the pool are taken as already rotated (attn_kv_append_rope).
 * O and LSE are bitwise those of attn_rope on q followed by
 * attn_prefill_paged. rope->max_pos >= max_ctx_len.
 */
attn_status attn_prefill_paged_rope(const attn_prefill_dims* dims, const void* q,
                                    const void* k_pool, const void* v_pool,
                                    const int32_t* block_table, const int32_t* ctx_lens,
                                    const int32_t* cu_q, const attn_rope_tables* rope, void* o,
                                    float* lse, float scale, void* stream);

/* Shape of an RMSNorm call: `rows` rows of `n` values (n % 8 == 0,
 * 8 <= n <= 2048; rows >= 0). */
typedef struct attn_norm_dims {
    int32_t rows;
    int32_t n;
} attn_norm_dims;

/*
 * attn_rmsnorm_fwd -- RMSNorm, the layer operation next to attention in the
 * Qwen3 stack (pitchhut "Project Highlights"):
 *   r_i = 1 / sqrt(mean_j x_ij^2 + eps),  y_ij = x_ij r_i w_j.
 *   x     fp16 [rows, n]    input rows
 *   w     fp16 [n]          weight
 *   y     fp16 [rows, n]    output, fully overwritten (may not alias x)
 *   rstd  fp32 [rows]       r_i, fully overwritten (attn_rmsnorm_bwd needs it)
 * fp32 sums; y rounded to nearest-even fp16.
 */
attn_status attn_rmsnorm_fwd(const attn_norm_dims* dims, const void* x, const void* w,
                             float eps, void* y, float* rstd, void* stream);

/* Bytes of device workspace attn_rmsnorm_bwd needs (fp32 partial dw rows,
 * one per backward work-group; 0 for rows == 0). */
size_t attn_rmsnorm_bwd_workspace_bytes(const attn_norm_dims* dims);

/*
 * attn_rmsnorm_bwd -- gradients of sum(y * dy) for attn_rmsnorm_fwd:
 *   dx_ij = r_i (w_j dy_ij - xh_ij mean_k(w_k dy_ik xh_ik)),  xh = x r,
 *   dw_j  = sum_i dy_ij xh_ij.
 *   x, w   as given to attn_rmsnorm_fwd;  rstd fp32 [rows] its output
 *   dy     fp16 [rows, n]
 *   dx     fp16 [rows, n]   fully overwritten (may not alias x or dy)
 *   dw     fp32 [n]         fully overwritten (not accumulated into)
 *   workspace  at least attn_rmsnorm_bwd_workspace_bytes(dims) bytes,
 *              256-byte aligned
 * dw sums the rows in a fixed order: bitwise reproducible.
 */
attn_status attn_rmsnorm_bwd(const attn_norm_dims* dims, const void* x, const void* w,
                             const float* rstd, const void* dy, void* dx, float* dw,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Shape of a sampling call: n_rows rows of `vocab` logits. */
typedef struct attn_sample_dims {
    int32_t n_rows;
    int32_t vocab;
} attn_sample_dims;

/*
 * attn_sample -- temperature / top-k / top-p sampling, the rollout engine's
 * step after the LM head (pitchhut "Key Features", item 1), with the random
 * number supplied by the caller (one uniform per row), so the token is a
 * deterministic function of the logits and u:
 *   z = logits / temperature; rank tokens by z descending, ties by index
 *   ascending; keep the first k = min(top_k, vocab); weights
 *   w_j = exp(z_j - z_0) over the kept ranking with cumulative sums c_j;
 *   cut = min{j : c_j >= top_p * c_(k-1)};
 *   token = the one at rank min{j <= cut : c_j > u * c_cut}.
 *   logits fp32 [n_rows, vocab]  finite or -inf, at least one finite per row
 *   u      fp32 [n_rows]         uniforms in [0, 1)
 *   tokens int32 [n_rows]        output
 * Requires temperature > 0 (finite), 1 <= top_k <= 1024, 0 < top_p <= 1.
 * fp32 arithmetic; a u within fp32 rounding of a cumulative boundary may
 * pick the neighbouring rank.
 */
attn_status attn_sample(const attn_sample_dims* dims, const float* logits, const float* u,
                        float temperature, int32_t top_k, float top_p, int32_t* tokens,
                        void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* attn_status_string(attn_status status);

/* The entry points above do not read the contents of the device index
 * arrays on the host (they never synchronize). The two validators below check
 * host copies; the Python binding runs them before every launch when the
 * environment sets ATTN_DEBUG_VALIDATE=1 (a synchronous debug mode).
 *
 * Host-side check of a HOST copy of cu_seqlens against dims: cu[0] == 0,
 * non-decreasing, cu[n] == total_tokens, every length <= max_seqlen.
 * Returns ATTN_OK or ATTN_ERR_INVALID_ARG. Makes no HIP call. */
attn_status attn_check_cu_seqlens(const attn_varlen_dims* dims, const int32_t* cu_host);

/* Host-side check of HOST copies of block_table and ctx_lens against dims:
 * 0 <= ctx <= max_ctx_len, ceil(ctx/16) <= max_blocks_per_seq and every used
 * entry in [0, num_blocks). Returns ATTN_OK or ATTN_ERR_INVALID_ARG. */
attn_status attn_check_paged(const attn_paged_dims* dims, const int32_t* block_table_host,
                             const int32_t* ctx_lens_host);

/* Host-side check of HOST copies of cu_q, block_table and ctx_lens against
 * a prefill's dims: the attn_check_paged conditions, cu_q rising from 0 to
 * total_q with every L_b <= max_q_len, and L_b <= ctx_lens[b]. Returns ATTN_OK
 * or ATTN_ERR_INVALID_ARG. Makes no HIP call. */
attn_status attn_check_prefill(const attn_prefill_dims* dims, const int32_t* cu_q_host,
                               const int32_t* block_table_host, const int32_t* ctx_lens_host);

#ifdef __cplusplus
}
#endif

#endif /* CGQA_ATTN_H */
