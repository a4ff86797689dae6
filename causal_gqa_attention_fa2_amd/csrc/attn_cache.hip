// attn_cache.hip -- key/value cache append for the chunked prefill over a
// paged cache (the rollout engine's "paged key-value caching"; pitchhut "Key
// Features", item 2).
//
// New token i of sequence b (row cu[b] + i of k_new / v_new) is the context
// position t = ctx[b] - L_b + i (L_b = cu[b+1] - cu[b], the sequence's new
// tokens are the last L_b of its ctx[b] positions) and goes to slot t % 16
// of pool block bt[b][t / 16]. Pure data movement, bound by HBM: each
// work-group moves 16 tokens of one sequence in 16-byte pieces, every byte
// read once and written once. The variant with RoPE tables rotates each key
// by its position t on the way (rope_pair in cdna4.h: the same bits as the
// standalone RoPE pass); a thread then holds the two 16-byte pieces whose
// dimensions pair up (8p .. 8p+7 and d/2 + 8p ..).
#include "cdna4.h"
#include "kernels.h"

namespace cgqa {
namespace {

constexpr int kTokPerWG = 16;
constexpr int kAppendThreads = 256;

struct AppendParams {
  const uint4* __restrict__ k_new;
  const uint4* __restrict__ v_new;
  const int32_t* __restrict__ cu;
  const int32_t* __restrict__ bt;
  const int32_t* __restrict__ ctx;
  uint4* __restrict__ k_pool;
  uint4* __restrict__ v_pool;
  const float* __restrict__ cos_t;  // RoPE tables [max_pos, d / 2] (ROPE only)
  const float* __restrict__ sin_t;
  int max_pos;
  int cpt;  // 16-byte pieces per token row (h_kv * d / 8)
  int max_blocks, num_blocks, max_ctx;
};

template <int D, bool ROPE>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(AppendParams p) {
  const int b = blockIdx.y;
  const int s0 = p.cu[b];
  const int L = p.cu[b + 1] - s0;
  const int c = min(p.ctx[b], p.max_ctx);  // a context past the table is clamped
  const int i0 = blockIdx.x * kTokPerWG;
  if (i0 >= L || c < L) return;  // nothing here, or an invalid batch
  const int off = c - L;
  const int ntok = min(kTokPerWG, L - i0);
  // Pool row of each of the work-group's tokens, looked up once.
  __shared__ size_t dst_row[kTokPerWG];
  if (threadIdx.x < ntok) {
    const int t = off + i0 + threadIdx.x;
    const int lb = min(t >> 4, p.max_blocks - 1);
    const int phys = min(max(p.bt[(size_t)b * p.max_blocks + lb], 0), p.num_blocks - 1);
    dst_row[threadIdx.x] = ((size_t)phys * 16 + (t & 15)) * p.cpt;
  }
  __syncthreads();
  const int n = ntok * p.cpt;
  const size_t src0 = (size_t)(s0 + i0) * p.cpt;  // the tokens' rows are contiguous
  if constexpr (ROPE) {
    constexpr int PP = D / 16;  // pieces per half head
    const int per_tok = p.cpt / 2;  // pairs of pieces per token
    for (int e = threadIdx.x; e < ntok * per_tok; e += kAppendThreads) {
      const int tok = e / per_tok;
      const int r = e - tok * per_tok;
      const int h = r / PP;
      const int pc = r - h * PP;
      const int pos = min(off + i0 + tok, p.max_pos - 1);
      const int piece = tok * p.cpt + h * 2 * PP + pc;  // low piece; high one PP further
      f16x8 lo = __builtin_bit_cast(f16x8, p.k_new[src0 + piece]);
      f16x8 hi = __builtin_bit_cast(f16x8, p.k_new[src0 + piece + PP]);
      rope_rotate8(lo, hi, p.cos_t + (size_t)pos * (D / 2) + 8 * pc,
                   p.sin_t + (size_t)pos * (D / 2) + 8 * pc, 1.f);
      const size_t dst = dst_row[tok] + (piece - tok * p.cpt);
      p.k_pool[dst] = __builtin_bit_cast(uint4, lo);
      p.k_pool[dst + PP] = __builtin_bit_cast(uint4, hi);
    }
    for (int e = threadIdx.x; e < n; e += kAppendThreads) {
      const int tok = e / p.cpt;
      p.v_pool[dst_row[tok] + (e - tok * p.cpt)] = p.v_new[src0 + e];
    }
  } else {
    for (int e = threadIdx.x; e < n; e += kAppendThreads) {
      const int tok = e / p.cpt;
      const size_t dst = dst_row[tok] + (e - tok * p.cpt);
      p.k_pool[dst] = p.k_new[src0 + e];
      p.v_pool[dst] = p.v_new[src0 + e];
    }
  }
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
  AppendParams p;
  p.k_new = (const uint4*)a.k_new;
  p.v_new = (const uint4*)a.v_new;
  p.cu = a.cu_new;
  p.bt = a.block_table;
  p.ctx = a.ctx_lens;
  p.k_pool = (uint4*)a.k_pool;
  p.v_pool = (uint4*)a.v_pool;
  p.cos_t = a.rope_cos;
  p.sin_t = a.rope_sin;
  p.max_pos = a.rope_max_pos;
  p.cpt = a.h_kv * a.head_dim / 8;
  p.max_blocks = a.max_blocks_per_seq;
  p.num_blocks = a.num_blocks;
  p.max_ctx = a.max_ctx_len;
  const dim3 grid((a.max_new + kTokPerWG - 1) / kTokPerWG, a.n_seqs);
  if (a.rope_cos == nullptr)
    hipLaunchKernelGGL((kv_append_kernel<128, false>), grid, dim3(kAppendThreads), 0, stream, p);
  else if (a.head_dim == 128)
    hipLaunchKernelGGL((kv_append_kernel<128, true>), grid, dim3(kAppendThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((kv_append_kernel<64, true>), grid, dim3(kAppendThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace cgqa
