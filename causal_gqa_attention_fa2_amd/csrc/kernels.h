// kernels.h -- launch arguments and launchers shared by the C ABI layer
// (attn_api.cpp) and the HIP kernel files. Host-side only declarations.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace cgqa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_seqlens;
  void* o;
  float* lse;
  int n_seqs, total_tokens, max_seqlen, h_q, h_kv, head_dim;
  float scale;
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
  float* dq_acc;  // workspace: fp32 [T, h_q, d]
  float* drow;    // workspace: fp32 [h_q, T], rowsum(dO * O)
  int n_seqs, total_tokens, max_seqlen, h_q, h_kv, head_dim;
  float scale;
};

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  void* o;
  float* part_o;   // workspace: fp32 [n, h_q, max_splits, d]
  float* part_ml;  // workspace: fp32 [n, h_q, max_splits, 2] (max, sum)
  int n_seqs, h_q, h_kv, head_dim, max_blocks_per_seq, max_splits;
  float scale;
};

// Tokens of context handled by one decode work-group (a multiple of 16).
constexpr int kDecodeSplit = 512;

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace cgqa
