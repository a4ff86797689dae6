// kernels.h -- launch arguments and launchers shared by the C ABI layer
// (attn_api.cpp) and the HIP kernel files. Host-side only declarations.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace cgqa {

// Forward and paged prefill. For the prefill, k and v are the paged pools,
// cu_seqlens packs the new query tokens (total_tokens of them, at most
// max_seqlen per sequence), ctx_lens holds each sequence's context length
// (new tokens included) and lse may be null.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_seqlens;
  void* o;
  float* lse;
  const int32_t* block_table = nullptr;
  const int32_t* ctx_lens = nullptr;
  int max_blocks_per_seq = 0, num_blocks = 0, max_ctx_len = 0;
  // Paged prefill only: RoPE tables [rope_max_pos, head_dim / 2] to rotate the
  // queries with as they are loaded, or null.
  const float* rope_cos = nullptr;
  const float* rope_sin = nullptr;
  int rope_max_pos = 0;
  int n_seqs, total_tokens, max_seqlen, h_q, h_kv, head_dim;
  float scale;
  int num_cus = 256;  // compute units of the device (persistent grid size)
};

// New keys and values of a chunked prefill, written into the paged pools.
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int32_t* cu_new;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  void* k_pool;
  void* v_pool;
  // RoPE tables [rope_max_pos, head_dim / 2] to rotate the keys with on their
  // way into the pool, or null.
  const float* rope_cos = nullptr;
  const float* rope_sin = nullptr;
  int rope_max_pos = 0;
  int n_seqs, max_new, h_kv, head_dim, max_blocks_per_seq, num_blocks, max_ctx_len;
};

// RoPE tables: cos / sin fp32 [max_pos, head_dim / 2].
struct RopeTableArgs {
  float* cos;
  float* sin;
  int max_pos, head_dim;
  double base;
};

// In-place RoPE of packed q [T, h_q, d] and k [T, h_kv, d] (either may be
// null). Positions: index within the sequence, or ctx_lens[b] - L_b + i.
struct RopeArgs {
  void* q;
  void* k;
  const int32_t* cu_seqlens;
  const int32_t* ctx_lens;  // may be null
  const float* cos;
  const float* sin;
  int max_pos;
  int n_seqs, max_seqlen, h_q, h_kv, head_dim;
  bool inverse;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  const int32_t* cu_seqlens;
  void* dq;
  void* dk;
  void* dv;
  float* drow;    // workspace: fp32 [h_q, T], -rowsum(dO * O)
  float* lse2;    // workspace: fp32 [h_q, T], LSE * log2(e)
  void* ds = nullptr;  // workspace: fp16 dS blocks (the dS path), or null
  // RoPE tables [rope_max_pos, head_dim / 2] to rotate dq and dk back with at
  // their stores (q and k are the rotated tensors), or null.
  const float* rope_cos = nullptr;
  const float* rope_sin = nullptr;
  int rope_max_pos = 0;
  int n_seqs, total_tokens, max_seqlen, h_q, h_kv, head_dim;
  int num_cus;    // compute units of the device (persistent dq grid)
  float scale;
};

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  void* o;
  float* part_o;   // workspace: fp32 [n_wgs + n, h_q, d] partial outputs
  float* part_ml;  // workspace: fp32 [n_wgs + n, h_q, 2] partial (max, sum)
  int32_t* plan;   // workspace: int32 [n + 1] block prefix sums, [n_wgs] first sequences
  int n_seqs, h_q, h_kv, head_dim, max_blocks_per_seq, n_wgs;
  // Pool blocks and the largest context (<= 16 * max_blocks_per_seq): the
  // kernels clamp contexts into [0, max_ctx_len] and table entries into
  // [0, num_blocks).
  int num_blocks = 0, max_ctx_len = 0;
  float scale;
  // RoPE tables [rope_max_pos, head_dim / 2] to rotate each query by its
  // position ctx - 1 as it is loaded, or null.
  const float* rope_cos = nullptr;
  const float* rope_sin = nullptr;
  int rope_max_pos = 0;
};

// Work-groups of the paged-decode gather: the flattened (sequence, block)
// space is cut into n_wgs equal contiguous ranges. Bounded by the number of
// blocks any batch with these dims can hold.
constexpr int kDecodeMaxWGs = 512;
inline int decode_num_wgs(int n_seqs, int max_ctx_len) {
  const long long bound = (long long)n_seqs * ((max_ctx_len + 15) / 16);
  return bound < 1 ? 1 : (bound < kDecodeMaxWGs ? (int)bound : kDecodeMaxWGs);
}

// Workspace of the allocation-free decode: a device array of this many bytes
// (one per device, held until the process ends). decode_scratch returns the
// current device's copy, looked up on the first call on that device.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t decode_scratch(void** ptr);

// Query-stationary work-groups have `waves` waves (dQ: kQWaves; the forward:
// kQWaves or 4, by sequence length); each wave owns 32 query rows of one
// head. A work-group covers hpw heads of a KV group (hpw = the largest power
// of two <= min(G, waves)) and 32 * waves / hpw query positions; a group of
// G heads needs ceil(G / hpw) head chunks.
constexpr int kQWaves = 8;
struct QTileLayout {
  int hpw, nqb, n_chunks;
};
inline QTileLayout qtile_layout(int G, int waves = kQWaves) {
  int hpw = 1;
  while (hpw * 2 <= G && hpw * 2 <= waves) hpw *= 2;
  return QTileLayout{hpw, waves / hpw, (G + hpw - 1) / hpw};
}

// RMSNorm over rows of n fp16 values (n % 8 == 0, 8 <= n <= kNormMaxCols).
// The backward writes one fp32 partial dw row per work-group (at most
// kNormMaxWGs of them) into `part`, then sums them into dw.
constexpr int kNormMaxCols = 2048;
constexpr int kNormMaxWGs = 256;
struct NormArgs {
  const void* x;
  const void* w;
  const void* dy = nullptr;
  void* y = nullptr;
  void* dx = nullptr;
  float* rstd;
  float* part = nullptr;
  float* dw = nullptr;
  int rows, n;
  float eps;
};
int rmsnorm_bwd_num_wgs(int rows, int n);
hipError_t launch_rmsnorm_fwd(const NormArgs& a, hipStream_t stream);
hipError_t launch_rmsnorm_bwd(const NormArgs& a, hipStream_t stream);

// Sampling over logits: one work-group of kMaxTopK threads per row.
constexpr int kMaxTopK = 1024;
struct SampleArgs {
  const float* logits;  // [n_rows, vocab]
  const float* u;       // [n_rows] uniforms in [0, 1)
  int32_t* tokens;      // [n_rows]
  int n_rows, vocab, top_k;
  float temperature, top_p;
};
hipError_t launch_sample(const SampleArgs& a, hipStream_t stream);

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
hipError_t launch_prefill(const FwdArgs& a, hipStream_t stream);
hipError_t launch_rope_tables(const RopeTableArgs& a, hipStream_t stream);
hipError_t launch_rope(const RopeArgs& a, hipStream_t stream);
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);
// dS blocks of the backward's dS path: one 32 x 32 fp16 block (2 KiB) per
// (sequence, query head, 32-row query block, 32-key block), indexed with the
// longest sequence's block count on both block axes.
inline size_t bwd_ds_blocks(int n_seqs, int h_q, int max_seqlen) {
  const size_t nb = (size_t)((max_seqlen + 31) / 32);
  return (size_t)n_seqs * h_q * nb * nb;
}
constexpr size_t kDsBlockBytes = 32 * 32 * 2;
constexpr size_t kDsMaxBytes = (size_t)4 << 30;
// The dS path is taken for batches whose sequences are very unequal (the
// padded size n_seqs * max_seqlen is at least 1.25 T), when its blocks fit
// in kDsMaxBytes. Measured: 10% faster backward on a GRPO group batch, equal
// on batches of equal lengths (which keep the recompute path).
inline bool bwd_use_ds(int n_seqs, int total_tokens, int max_seqlen, int h_q) {
  if (n_seqs < 2) return false;
  if ((long long)n_seqs * max_seqlen * 4 < (long long)total_tokens * 5) return false;
  return bwd_ds_blocks(n_seqs, h_q, max_seqlen) * kDsBlockBytes <= kDsMaxBytes;
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace cgqa
