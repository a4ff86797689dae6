// attn_api.cpp -- the C ABI declared in include/attn.h: argument checks,
// workspace sizing and the hand-off to the kernel launchers. Host code only;
// the kernels live in the .hip files.
#include "attn.h"

#include <hip/hip_runtime_api.h>

#include "kernels.h"

#include <atomic>

namespace {

// Compute units of the current device (queried once per device; persistent
// kernels launch at most one work-group per unit).
int num_compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

constexpr size_t kWsAlign = 256;

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks shared by forward and backward. Sets *empty for a batch with
// nothing to compute.
attn_status check_varlen(const attn_varlen_dims* d, bool* empty) {
  if (!d) return ATTN_ERR_INVALID_ARG;
  if (d->n_seqs < 0 || d->total_tokens < 0 || d->max_seqlen < 0) return ATTN_ERR_INVALID_ARG;
  if (d->h_q <= 0 || d->h_kv <= 0 || d->head_dim <= 0) return ATTN_ERR_INVALID_ARG;
  if (d->h_q % d->h_kv != 0) return ATTN_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (d->h_q / d->h_kv > 16) return ATTN_ERR_UNSUPPORTED;
  if (d->max_seqlen > d->total_tokens) return ATTN_ERR_INVALID_ARG;
  if (d->n_seqs > 0 && d->total_tokens > 0 && d->max_seqlen == 0) return ATTN_ERR_INVALID_ARG;
  // Element offsets are formed in 64-bit, token indices in 32-bit.
  if ((int64_t)d->total_tokens * d->h_q > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  // Work items (grids and item indices are 32-bit): at most one per (sequence,
  // 32-row query block of the longest sequence, query head).
  if ((int64_t)((d->max_seqlen + 31) / 32) * d->n_seqs * d->h_q > INT32_MAX)
    return ATTN_ERR_UNSUPPORTED;
  *empty = d->n_seqs == 0 || d->total_tokens == 0;
  return ATTN_OK;
}

// Workspace of the backward: two fp32 [h_q, T] row-term arrays, -D =
// -rowsum(dO * O) and LSE * log2(e), each starting on a 256-byte boundary.
size_t bwd_row_bytes(const attn_varlen_dims* d) {
  return align_up((size_t)d->h_q * d->total_tokens * sizeof(float));
}
bool bwd_ds_path(const attn_varlen_dims* d) {
  return cgqa::bwd_use_ds(d->n_seqs, d->total_tokens, d->max_seqlen, d->h_q);
}
size_t bwd_ds_bytes(const attn_varlen_dims* d) {
  return bwd_ds_path(d)
             ? align_up(cgqa::bwd_ds_blocks(d->n_seqs, d->h_q, d->max_seqlen) * cgqa::kDsBlockBytes)
             : 0;
}
size_t bwd_ws_bytes(const attn_varlen_dims* d) { return 2 * bwd_row_bytes(d) + bwd_ds_bytes(d); }

attn_status check_paged(const attn_paged_dims* d, bool* empty) {
  if (!d) return ATTN_ERR_INVALID_ARG;
  if (d->n_seqs < 0 || d->h_q <= 0 || d->h_kv <= 0 || d->head_dim <= 0) return ATTN_ERR_INVALID_ARG;
  if (d->max_blocks_per_seq < 0 || d->num_blocks < 0 || d->max_ctx_len < 0)
    return ATTN_ERR_INVALID_ARG;
  if (d->h_q % d->h_kv != 0) return ATTN_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (d->h_q / d->h_kv > 16) return ATTN_ERR_UNSUPPORTED;
  if (d->block_size != 16) return ATTN_ERR_UNSUPPORTED;
  if (d->n_seqs > 65535 || d->h_kv > 65535) return ATTN_ERR_UNSUPPORTED;  // grid y/z limits
  if ((int64_t)d->max_blocks_per_seq * 16 < d->max_ctx_len) return ATTN_ERR_INVALID_ARG;
  // Block counts and their prefix sums are int32 on the device.
  if ((int64_t)d->n_seqs * (((int64_t)d->max_ctx_len + 15) / 16) > (INT32_MAX >> 1))
    return ATTN_ERR_UNSUPPORTED;
  *empty = d->n_seqs == 0;
  // A non-empty context needs at least one pool block.
  if (!*empty && d->max_ctx_len > 0 && d->num_blocks == 0) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// Workspace of the decode: partial outputs, partial (max, sum) pairs and the
// work plan (block prefix sums and each work-group's first sequence).
size_t decode_ws_parts(const attn_paged_dims* d, size_t* o_bytes, size_t* ml_bytes) {
  const int nwg = cgqa::decode_num_wgs(d->n_seqs, d->max_ctx_len);
  const size_t slots = (size_t)(nwg + d->n_seqs) * d->h_q;
  *o_bytes = align_up(slots * d->head_dim * sizeof(float));
  *ml_bytes = align_up(slots * 2 * sizeof(float));
  return *o_bytes + *ml_bytes + align_up((size_t)(d->n_seqs + 1 + nwg) * sizeof(int32_t));
}

// Shape checks of a chunked prefill: the pool side as for the decode, then
// the packed new tokens. Sets *empty when there is nothing to compute.
attn_status check_prefill(const attn_prefill_dims* d, bool* empty) {
  if (!d) return ATTN_ERR_INVALID_ARG;
  bool no_seqs = false;
  const attn_status st = check_paged(&d->paged, &no_seqs);
  if (st != ATTN_OK) return st;
  if (d->total_q < 0 || d->max_q_len < 0 || d->max_q_len > d->total_q) return ATTN_ERR_INVALID_ARG;
  if (d->max_q_len > d->paged.max_ctx_len) return ATTN_ERR_INVALID_ARG;
  if (no_seqs && d->total_q > 0) return ATTN_ERR_INVALID_ARG;
  if (d->total_q > 0 && d->max_q_len == 0) return ATTN_ERR_INVALID_ARG;
  // 32-bit indices: LSE rows, work items and block-table entries.
  if ((int64_t)d->total_q * d->paged.h_q > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)((d->max_q_len + 31) / 32) * d->paged.n_seqs * d->paged.h_q > INT32_MAX)
    return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)d->paged.n_seqs * d->paged.max_blocks_per_seq > INT32_MAX)
    return ATTN_ERR_UNSUPPORTED;
  *empty = no_seqs || d->total_q == 0;
  return ATTN_OK;
}

attn_status check_norm(const attn_norm_dims* d, bool* empty) {
  if (!d || d->rows < 0 || d->n <= 0) return ATTN_ERR_INVALID_ARG;
  if (d->n % 8 != 0 || d->n > cgqa::kNormMaxCols) return ATTN_ERR_UNSUPPORTED;
  *empty = d->rows == 0;
  return ATTN_OK;
}

size_t norm_ws_bytes(const attn_norm_dims* d) {
  return align_up((size_t)cgqa::rmsnorm_bwd_num_wgs(d->rows, d->n) * d->n * sizeof(float));
}

// RoPE tables of a call: both present, 16-byte aligned, max_pos >= 1 and
// covering every position the call can form (max_positions of them).
attn_status check_rope(const attn_rope_tables* t, int64_t max_positions) {
  if (!t || !t->cos || !t->sin || t->max_pos <= 0) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(t->cos) || !aligned16(t->sin)) return ATTN_ERR_INVALID_ARG;
  if (max_positions > t->max_pos) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
  }
  return "ATTN_UNKNOWN_STATUS";
}

attn_status attn_fwd(const attn_varlen_dims* dims, const void* q, const void* k, const void* v,
                     const int32_t* cu_seqlens, float scale, void* o, float* lse, void* stream) {
  bool empty = false;
  attn_status st = check_varlen(dims, &empty);
  if (st != ATTN_OK) return st;
  if (empty) return ATTN_OK;
  if (!q || !k || !v || !cu_seqlens || !o || !lse) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      ((uintptr_t)cu_seqlens & 3u))
    return ATTN_ERR_INVALID_ARG;
  cgqa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_seqlens = cu_seqlens;
  a.o = o;
  a.lse = lse;
  a.n_seqs = dims->n_seqs;
  a.total_tokens = dims->total_tokens;
  a.max_seqlen = dims->max_seqlen;
  a.h_q = dims->h_q;
  a.h_kv = dims->h_kv;
  a.head_dim = dims->head_dim;
  a.scale = scale;
  a.num_cus = num_compute_units();
  return cgqa::launch_fwd(a, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t attn_bwd_workspace_bytes(const attn_varlen_dims* dims) {
  bool empty = false;
  if (check_varlen(dims, &empty) != ATTN_OK || empty) return 0;
  return bwd_ws_bytes(dims);
}

static attn_status bwd_impl(const attn_varlen_dims* dims, const void* q, const void* k,
                            const void* v, const void* o, const float* lse, const void* dO,
                            const int32_t* cu_seqlens, const attn_rope_tables* rope, void* dq,
                            void* dk, void* dv, float scale, void* workspace,
                            size_t workspace_bytes, void* stream) {
  bool empty = false;
  attn_status st = check_varlen(dims, &empty);
  if (st != ATTN_OK) return st;
  if (rope && (st = check_rope(rope, dims->max_seqlen)) != ATTN_OK) return st;
  if (empty) return ATTN_OK;
  if (!q || !k || !v || !o || !lse || !dO || !cu_seqlens || !dq || !dk || !dv)
    return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dO) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      ((uintptr_t)cu_seqlens & 3u))
    return ATTN_ERR_INVALID_ARG;
  const size_t need = bwd_ws_bytes(dims);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % kWsAlign))
    return ATTN_ERR_WORKSPACE;
  cgqa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dO;
  a.cu_seqlens = cu_seqlens;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.drow = (float*)workspace;
  a.lse2 = (float*)((char*)workspace + bwd_row_bytes(dims));
  a.ds = bwd_ds_path(dims) ? (char*)workspace + 2 * bwd_row_bytes(dims) : nullptr;
  a.n_seqs = dims->n_seqs;
  a.total_tokens = dims->total_tokens;
  a.max_seqlen = dims->max_seqlen;
  a.h_q = dims->h_q;
  a.h_kv = dims->h_kv;
  a.head_dim = dims->head_dim;
  a.scale = scale;
  a.num_cus = num_compute_units();
  if (rope) {
    a.rope_cos = rope->cos;
    a.rope_sin = rope->sin;
    a.rope_max_pos = rope->max_pos;
  }
  return cgqa::launch_bwd(a, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_bwd(const attn_varlen_dims* dims, const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* dO,
                     const int32_t* cu_seqlens, void* dq, void* dk, void* dv, float scale,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(dims, q, k, v, o, lse, dO, cu_seqlens, nullptr, dq, dk, dv, scale, workspace,
                  workspace_bytes, stream);
}

attn_status attn_bwd_rope(const attn_varlen_dims* dims, const void* q, const void* k,
                          const void* v, const void* o, const float* lse, const void* dO,
                          const int32_t* cu_seqlens, const attn_rope_tables* rope, void* dq,
                          void* dk, void* dv, float scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!rope) return ATTN_ERR_INVALID_ARG;
  return bwd_impl(dims, q, k, v, o, lse, dO, cu_seqlens, rope, dq, dk, dv, scale, workspace,
                  workspace_bytes, stream);
}

size_t attn_decode_workspace_bytes(const attn_paged_dims* dims) {
  bool empty = false;
  if (check_paged(dims, &empty) != ATTN_OK || empty) return 0;
  size_t ob, mb;
  return decode_ws_parts(dims, &ob, &mb);
}

// Checks of a decode call's shape, tables and tensor pointers (all but the
// workspace). Sets *empty when there is nothing to compute.
static attn_status decode_check(const attn_paged_dims* dims, const void* q, const void* k_pool,
                                const void* v_pool, const int32_t* block_table,
                                const int32_t* ctx_lens, const attn_rope_tables* rope,
                                const void* o, bool* empty) {
  attn_status st = check_paged(dims, empty);
  if (st != ATTN_OK) return st;
  if (rope && (st = check_rope(rope, dims->max_ctx_len)) != ATTN_OK) return st;
  if (*empty) return ATTN_OK;
  if (!q || !ctx_lens || !o) return ATTN_ERR_INVALID_ARG;
  if (dims->max_ctx_len > 0 && (!k_pool || !v_pool || !block_table)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(o) || !aligned16(k_pool) || !aligned16(v_pool) ||
      ((uintptr_t)block_table & 3u) || ((uintptr_t)ctx_lens & 3u))
    return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

static attn_status decode_impl(const attn_paged_dims* dims, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_table,
                               const int32_t* ctx_lens, const attn_rope_tables* rope, void* o,
                               float scale, void* workspace, size_t workspace_bytes,
                               void* stream) {
  bool empty = false;
  const attn_status st =
      decode_check(dims, q, k_pool, v_pool, block_table, ctx_lens, rope, o, &empty);
  if (st != ATTN_OK || empty) return st;
  size_t ob, mb;
  const size_t need = decode_ws_parts(dims, &ob, &mb);
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace % kWsAlign)))
    return ATTN_ERR_WORKSPACE;
  cgqa::DecodeArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.ctx_lens = ctx_lens;
  a.o = o;
  a.part_o = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + ob);
  a.plan = (int32_t*)((char*)workspace + ob + mb);
  a.n_seqs = dims->n_seqs;
  a.h_q = dims->h_q;
  a.h_kv = dims->h_kv;
  a.head_dim = dims->head_dim;
  a.max_blocks_per_seq = dims->max_blocks_per_seq;
  a.n_wgs = cgqa::decode_num_wgs(dims->n_seqs, dims->max_ctx_len);
  a.num_blocks = dims->num_blocks;
  a.max_ctx_len = dims->max_ctx_len;
  a.scale = scale;
  if (rope) {
    a.rope_cos = rope->cos;
    a.rope_sin = rope->sin;
    a.rope_max_pos = rope->max_pos;
  }
  return cgqa::launch_decode(a, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_decode_paged(const attn_paged_dims* dims, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* block_table,
                              const int32_t* ctx_lens, void* o, float scale, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return decode_impl(dims, q, k_pool, v_pool, block_table, ctx_lens, nullptr, o, scale, workspace,
                     workspace_bytes, stream);
}

attn_status attn_decode_paged_noalloc(const attn_paged_dims* dims, const void* q,
                                      const void* k_pool, const void* v_pool,
                                      const int32_t* block_table, const int32_t* ctx_lens,
                                      void* o, float scale, void* stream) {
  bool empty = false;
  const attn_status st =
      decode_check(dims, q, k_pool, v_pool, block_table, ctx_lens, nullptr, o, &empty);
  if (st != ATTN_OK || empty) return st;
  size_t ob, mb;
  if (decode_ws_parts(dims, &ob, &mb) > cgqa::kDecodeScratchBytes) return ATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  if (cgqa::decode_scratch(&ws) != hipSuccess) return ATTN_ERR_HIP;
  return decode_impl(dims, q, k_pool, v_pool, block_table, ctx_lens, nullptr, o, scale, ws,
                     cgqa::kDecodeScratchBytes, stream);
}

attn_status attn_decode_paged_rope(const attn_paged_dims* dims, const void* q,
                                   const void* k_pool, const void* v_pool,
                                   const int32_t* block_table, const int32_t* ctx_lens,
                                   const attn_rope_tables* rope, void* o, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!rope) return ATTN_ERR_INVALID_ARG;
  return decode_impl(dims, q, k_pool, v_pool, block_table, ctx_lens, rope, o, scale, workspace,
                     workspace_bytes, stream);
}

static attn_status kv_append_impl(const attn_prefill_dims* dims, const void* k_new,
                                  const void* v_new, const int32_t* cu_q,
                                  const int32_t* block_table, const int32_t* ctx_lens,
                                  const attn_rope_tables* rope, void* k_pool, void* v_pool,
                                  void* stream) {
  bool empty = false;
  attn_status st = check_prefill(dims, &empty);
  if (st != ATTN_OK) return st;
  if (rope && (st = check_rope(rope, dims->paged.max_ctx_len)) != ATTN_OK) return st;
  if (empty) return ATTN_OK;
  if (!k_new || !v_new || !cu_q || !block_table || !ctx_lens || !k_pool || !v_pool)
    return ATTN_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool) ||
      ((uintptr_t)cu_q & 3u) || ((uintptr_t)block_table & 3u) || ((uintptr_t)ctx_lens & 3u))
    return ATTN_ERR_INVALID_ARG;
  cgqa::AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.cu_new = cu_q;
  a.block_table = block_table;
  a.ctx_lens = ctx_lens;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.n_seqs = dims->paged.n_seqs;
  a.max_new = dims->max_q_len;
  a.h_kv = dims->paged.h_kv;
  a.head_dim = dims->paged.head_dim;
  a.max_blocks_per_seq = dims->paged.max_blocks_per_seq;
  a.num_blocks = dims->paged.num_blocks;
  a.max_ctx_len = dims->paged.max_ctx_len;
  if (rope) {
    a.rope_cos = rope->cos;
    a.rope_sin = rope->sin;
    a.rope_max_pos = rope->max_pos;
  }
  return cgqa::launch_kv_append(a, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_kv_append(const attn_prefill_dims* dims, const void* k_new, const void* v_new,
                           const int32_t* cu_q, const int32_t* block_table,
                           const int32_t* ctx_lens, void* k_pool, void* v_pool, void* stream) {
  return kv_append_impl(dims, k_new, v_new, cu_q, block_table, ctx_lens, nullptr, k_pool, v_pool,
                        stream);
}

attn_status attn_kv_append_rope(const attn_prefill_dims* dims, const void* k_new,
                                const void* v_new, const int32_t* cu_q,
                                const int32_t* block_table, const int32_t* ctx_lens,
                                const attn_rope_tables* rope, void* k_pool, void* v_pool,
                                void* stream) {
  if (!rope) return ATTN_ERR_INVALID_ARG;
  return kv_append_impl(dims, k_new, v_new, cu_q, block_table, ctx_lens, rope, k_pool, v_pool,
                        stream);
}

static attn_status prefill_impl(const attn_prefill_dims* dims, const void* q, const void* k_pool,
                                const void* v_pool, const int32_t* block_table,
                                const int32_t* ctx_lens, const int32_t* cu_q,
                                const attn_rope_tables* rope, void* o, float* lse, float scale,
                                void* stream) {
  bool empty = false;
  attn_status st = check_prefill(dims, &empty);
  if (st != ATTN_OK) return st;
  if (rope && (st = check_rope(rope, dims->paged.max_ctx_len)) != ATTN_OK) return st;
  if (empty) return ATTN_OK;
  if (!q || !k_pool || !v_pool || !block_table || !ctx_lens || !cu_q || !o)
    return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o) ||
      !aligned16(lse) || ((uintptr_t)cu_q & 3u) || ((uintptr_t)block_table & 3u) ||
      ((uintptr_t)ctx_lens & 3u))
    return ATTN_ERR_INVALID_ARG;
  cgqa::FwdArgs a;
  a.q = q;
  a.k = k_pool;
  a.v = v_pool;
  a.cu_seqlens = cu_q;
  a.o = o;
  a.lse = lse;
  a.block_table = block_table;
  a.ctx_lens = ctx_lens;
  a.max_blocks_per_seq = dims->paged.max_blocks_per_seq;
  a.num_blocks = dims->paged.num_blocks;
  a.max_ctx_len = dims->paged.max_ctx_len;
  if (rope) {
    a.rope_cos = rope->cos;
    a.rope_sin = rope->sin;
    a.rope_max_pos = rope->max_pos;
  }
  a.n_seqs = dims->paged.n_seqs;
  a.total_tokens = dims->total_q;
  a.max_seqlen = dims->max_q_len;
  a.h_q = dims->paged.h_q;
  a.h_kv = dims->paged.h_kv;
  a.head_dim = dims->paged.head_dim;
  a.scale = scale;
  a.num_cus = num_compute_units();
  return cgqa::launch_prefill(a, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_prefill_paged(const attn_prefill_dims* dims, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_table,
                               const int32_t* ctx_lens, const int32_t* cu_q, void* o,
                               float* lse, float scale, void* stream) {
  return prefill_impl(dims, q, k_pool, v_pool, block_table, ctx_lens, cu_q, nullptr, o, lse, scale,
                      stream);
}

attn_status attn_prefill_paged_rope(const attn_prefill_dims* dims, const void* q,
                                    const void* k_pool, const void* v_pool,
                                    const int32_t* block_table, const int32_t* ctx_lens,
                                    const int32_t* cu_q, const attn_rope_tables* rope, void* o,
                                    float* lse, float scale, void* stream) {
  if (!rope) return ATTN_ERR_INVALID_ARG;
  return prefill_impl(dims, q, k_pool, v_pool, block_table, ctx_lens, cu_q, rope, o, lse, scale,
                      stream);
}

attn_status attn_rope_tables_init(int32_t max_pos, int32_t head_dim, double base, float* cos_t,
                                  float* sin_t, void* stream) {
  if (max_pos <= 0 || !(base > 1.0) || !cos_t || !sin_t) return ATTN_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(cos_t) || !aligned16(sin_t)) return ATTN_ERR_INVALID_ARG;
  cgqa::RopeTableArgs a;
  a.cos = cos_t;
  a.sin = sin_t;
  a.max_pos = max_pos;
  a.head_dim = head_dim;
  a.base = base;
  return cgqa::launch_rope_tables(a, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_rope(const attn_varlen_dims* dims, void* q, void* k, const int32_t* cu_seqlens,
                      const int32_t* ctx_lens, int32_t max_ctx_len, const attn_rope_tables* rope,
                      int32_t inverse, void* stream) {
  bool empty = false;
  attn_status st = check_varlen(dims, &empty);
  if (st != ATTN_OK) return st;
  if (dims->n_seqs > 65535) return ATTN_ERR_UNSUPPORTED;  // grid y limit
  if (ctx_lens && max_ctx_len < dims->max_seqlen) return ATTN_ERR_INVALID_ARG;
  if ((st = check_rope(rope, ctx_lens ? max_ctx_len : dims->max_seqlen)) != ATTN_OK) return st;
  if (empty || (!q && !k)) return ATTN_OK;
  if (!cu_seqlens || ((uintptr_t)cu_seqlens & 3u) || ((uintptr_t)ctx_lens & 3u) ||
      !aligned16(q) || !aligned16(k))
    return ATTN_ERR_INVALID_ARG;
  cgqa::RopeArgs a;
  a.q = q;
  a.k = k;
  a.cu_seqlens = cu_seqlens;
  a.ctx_lens = ctx_lens;
  a.cos = rope->cos;
  a.sin = rope->sin;
  a.max_pos = rope->max_pos;
  a.n_seqs = dims->n_seqs;
  a.max_seqlen = dims->max_seqlen;
  a.h_q = dims->h_q;
  a.h_kv = dims->h_kv;
  a.head_dim = dims->head_dim;
  a.inverse = inverse != 0;
  return cgqa::launch_rope(a, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_check_prefill(const attn_prefill_dims* dims, const int32_t* cu,
                               const int32_t* table, const int32_t* ctx) {
  bool empty = false;
  if (check_prefill(dims, &empty) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  const int32_t n = dims->paged.n_seqs;
  if (!cu || (n > 0 && !ctx)) return ATTN_ERR_INVALID_ARG;
  if (n > 0 && attn_check_paged(&dims->paged, table, ctx) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  if (cu[0] != 0 || cu[n] != dims->total_q) return ATTN_ERR_INVALID_ARG;
  for (int32_t b = 0; b < n; ++b) {
    const int32_t len = cu[b + 1] - cu[b];
    if (len < 0 || len > dims->max_q_len || len > ctx[b]) return ATTN_ERR_INVALID_ARG;
  }
  return ATTN_OK;
}

attn_status attn_rmsnorm_fwd(const attn_norm_dims* dims, const void* x, const void* w,
                             float eps, void* y, float* rstd, void* stream) {
  bool empty = false;
  attn_status st = check_norm(dims, &empty);
  if (st != ATTN_OK) return st;
  if (!(eps >= 0.f)) return ATTN_ERR_INVALID_ARG;
  if (empty) return ATTN_OK;
  if (!x || !w || !y || !rstd) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || ((uintptr_t)rstd & 3u))
    return ATTN_ERR_INVALID_ARG;
  cgqa::NormArgs a;
  a.x = x;
  a.w = w;
  a.y = y;
  a.rstd = rstd;
  a.rows = dims->rows;
  a.n = dims->n;
  a.eps = eps;
  return cgqa::launch_rmsnorm_fwd(a, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t attn_rmsnorm_bwd_workspace_bytes(const attn_norm_dims* dims) {
  bool empty = false;
  if (check_norm(dims, &empty) != ATTN_OK || empty) return 0;
  return norm_ws_bytes(dims);
}

attn_status attn_rmsnorm_bwd(const attn_norm_dims* dims, const void* x, const void* w,
                             const float* rstd, const void* dy, void* dx, float* dw,
                             void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  attn_status st = check_norm(dims, &empty);
  if (st != ATTN_OK) return st;
  if (empty) return ATTN_OK;
  if (!x || !w || !rstd || !dy || !dx || !dw) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w) || !aligned16(dy) || !aligned16(dx) ||
      ((uintptr_t)rstd & 3u) || ((uintptr_t)dw & 3u))
    return ATTN_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < norm_ws_bytes(dims) || ((uintptr_t)workspace % kWsAlign))
    return ATTN_ERR_WORKSPACE;
  cgqa::NormArgs a;
  a.x = x;
  a.w = w;
  a.dy = dy;
  a.dx = dx;
  a.rstd = const_cast<float*>(rstd);
  a.part = (float*)workspace;
  a.dw = dw;
  a.rows = dims->rows;
  a.n = dims->n;
  a.eps = 0.f;
  return cgqa::launch_rmsnorm_bwd(a, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_sample(const attn_sample_dims* dims, const float* logits, const float* u,
                        float temperature, int32_t top_k, float top_p, int32_t* tokens,
                        void* stream) {
  if (!dims || dims->n_rows < 0 || dims->vocab < 1) return ATTN_ERR_INVALID_ARG;
  if (!(temperature > 0.f) || temperature > 3.0e38f) return ATTN_ERR_INVALID_ARG;
  if (!(top_p > 0.f && top_p <= 1.f)) return ATTN_ERR_INVALID_ARG;
  if (top_k < 1) return ATTN_ERR_INVALID_ARG;
  if (top_k > cgqa::kMaxTopK) return ATTN_ERR_UNSUPPORTED;
  if (dims->n_rows == 0) return ATTN_OK;
  if (!logits || !u || !tokens) return ATTN_ERR_INVALID_ARG;
  if (((uintptr_t)logits & 3u) || ((uintptr_t)u & 3u) || ((uintptr_t)tokens & 3u))
    return ATTN_ERR_INVALID_ARG;
  cgqa::SampleArgs a;
  a.logits = logits;
  a.u = u;
  a.tokens = tokens;
  a.n_rows = dims->n_rows;
  a.vocab = dims->vocab;
  a.top_k = top_k;
  a.temperature = temperature;
  a.top_p = top_p;
  return cgqa::launch_sample(a, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_check_cu_seqlens(const attn_varlen_dims* dims, const int32_t* cu) {
  if (!dims || !cu || dims->n_seqs < 0) return ATTN_ERR_INVALID_ARG;
  if (cu[0] != 0) return ATTN_ERR_INVALID_ARG;
  int32_t mx = 0;
  for (int32_t b = 0; b < dims->n_seqs; ++b) {
    const int32_t len = cu[b + 1] - cu[b];
    if (cu[b + 1] < cu[b]) return ATTN_ERR_INVALID_ARG;
    if (len > mx) mx = len;
  }
  if (cu[dims->n_seqs] != dims->total_tokens) return ATTN_ERR_INVALID_ARG;
  if (mx > dims->max_seqlen) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

attn_status attn_check_paged(const attn_paged_dims* dims, const int32_t* table,
                             const int32_t* ctx) {
  if (!dims || !ctx || dims->n_seqs < 0 || dims->block_size <= 0) return ATTN_ERR_INVALID_ARG;
  for (int32_t b = 0; b < dims->n_seqs; ++b) {
    const int32_t c = ctx[b];
    if (c < 0 || c > dims->max_ctx_len) return ATTN_ERR_INVALID_ARG;
    const int32_t nb = (c + dims->block_size - 1) / dims->block_size;
    if (nb > dims->max_blocks_per_seq) return ATTN_ERR_INVALID_ARG;
    if (nb > 0 && !table) return ATTN_ERR_INVALID_ARG;
    for (int32_t j = 0; j < nb; ++j) {
      const int32_t e = table[(size_t)b * dims->max_blocks_per_seq + j];
      if (e < 0 || e >= dims->num_blocks) return ATTN_ERR_INVALID_ARG;
    }
  }
  return ATTN_OK;
}

}  // extern "C"
