// attn_rope.hip -- rotary position embedding (RoPE) of queries and keys, the
// step right before attention (the mlllm.io article, "What happened", lists
// RoPE among the stack's hand-written kernels).
//
// Pairing: dimension j < d/2 of a head turns together with dimension j + d/2
// by the angle pos * base^(-2j/d) (the rotate-half layout of Qwen3). The
// kernels read the cosines and sines from fp32 tables [max_pos, d/2] and
// rotate in fp64 with one correct rounding to fp16 (rope_pair in cdna4.h), so
// the result does not depend on which kernel rotates: this standalone pass,
// the key/value append or the paged prefill's query loads.
//
//   rope_tables_kernel  cos / sin of pos * base^(-2j/d), evaluated in fp64
//                       and rounded to fp32.
//   rope_kernel         in-place rotation of packed q [T, h_q, d] and k
//                       [T, h_kv, d] (either may be absent); positions are
//                       the token's index within its sequence, or for a
//                       chunked prefill ctx[b] - L_b + i. The inverse rotation
//                       (the transpose) carries dq and dk back. Bound by HBM:
//                       every element is read and written once; the table
//                       rows are shared by the heads of a token.
#include "cdna4.h"
#include "kernels.h"

namespace cgqa {
namespace {

constexpr int kRopeTok = 16;  // tokens of one sequence per work-group
constexpr int kRopeThreads = 256;
constexpr int kRopeUnroll = 4;  // work items in flight per thread

__global__ __launch_bounds__(kRopeThreads) void rope_tables_kernel(float* __restrict__ cos_t,
                                                                   float* __restrict__ sin_t,
                                                                   int max_pos, int half,
                                                                   double base) {
  const size_t n = (size_t)max_pos * half;
  for (size_t e = (size_t)blockIdx.x * kRopeThreads + threadIdx.x; e < n;
       e += (size_t)gridDim.x * kRopeThreads) {
    const int pos = (int)(e / half);
    const int j = (int)(e - (size_t)pos * half);
    const double f = pow(base, -2.0 * j / (2.0 * half));
    const double a = (double)pos * f;
    cos_t[e] = (float)cos(a);
    sin_t[e] = (float)sin(a);
  }
}

struct RopeParams {
  f16* __restrict__ x[2];  // q, k (a null one is skipped)
  int heads[2];            // h_q, h_kv
  const int32_t* __restrict__ cu;
  const int32_t* __restrict__ ctx;  // null: positions from 0 in each sequence
  const float* __restrict__ cos_t;
  const float* __restrict__ sin_t;
  int max_pos;
  float sign;  // +1 rotate, -1 inverse
};

// One work-group: kRopeTok tokens of sequence blockIdx.y in tensor
// blockIdx.z. Work item = (token, head, piece p < d/16): the 8 pairs of
// dimensions 8p .. 8p+7 and d/2 + 8p .. d/2 + 8p + 7, two 16-byte loads and
// stores; the 8 cosines and sines are two 16-byte table loads each.
template <int D>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(RopeParams p) {
  constexpr int PP = D / 16;  // pieces per half head
  const int z = blockIdx.z;
  f16* __restrict__ x = p.x[z];
  if (x == nullptr) return;
  const int H = p.heads[z];
  const int b = blockIdx.y;
  const int s0 = p.cu[b];
  const int L = p.cu[b + 1] - s0;
  const int i0 = blockIdx.x * kRopeTok;
  if (i0 >= L) return;
  int off = 0;
  if (p.ctx != nullptr) {
    const int c = p.ctx[b];
    if (c < L) return;  // invalid batch (a chunk longer than its context)
    off = c - L;
  }
  const int ntok = min(kRopeTok, L - i0);
  const int per_tok = H * PP;
  const int n = ntok * per_tok;
  // kRopeUnroll items per thread per pass: all their loads (data and table)
  // are issued before the first rotation. Items past n repeat item `base`
  // (always valid) and are not stored.
  for (int base = threadIdx.x; base < n; base += kRopeThreads * kRopeUnroll) {
    f16* row[kRopeUnroll];
    f16x8 lo[kRopeUnroll], hi[kRopeUnroll];
    f32x4 c0[kRopeUnroll], c1[kRopeUnroll], sn0[kRopeUnroll], sn1[kRopeUnroll];
#pragma unroll
    for (int u = 0; u < kRopeUnroll; ++u) {
      const int e0 = base + u * kRopeThreads;
      const int e = e0 < n ? e0 : base;
      const int tok = e / per_tok;
      const int r = e - tok * per_tok;
      const int h = r / PP;
      const int pc = r - h * PP;
      const int pos = min(off + i0 + tok, p.max_pos - 1);
      row[u] = x + ((size_t)(s0 + i0 + tok) * H + h) * D + 8 * pc;
      lo[u] = *(const f16x8*)row[u];
      hi[u] = *(const f16x8*)(row[u] + D / 2);
      const f32x4* ct = (const f32x4*)(p.cos_t + (size_t)pos * (D / 2) + 8 * pc);
      const f32x4* st = (const f32x4*)(p.sin_t + (size_t)pos * (D / 2) + 8 * pc);
      c0[u] = ct[0];
      c1[u] = ct[1];
      sn0[u] = st[0];
      sn1[u] = st[1];
    }
#pragma unroll
    for (int u = 0; u < kRopeUnroll; ++u) {
      rope_rotate8(lo[u], hi[u], c0[u], c1[u], sn0[u], sn1[u], p.sign);
      if (base + u * kRopeThreads < n) {
        *(f16x8*)row[u] = lo[u];
        *(f16x8*)(row[u] + D / 2) = hi[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_rope_tables(const RopeTableArgs& a, hipStream_t stream) {
  const size_t n = (size_t)a.max_pos * (a.head_dim / 2);
  const size_t wgs = (n + kRopeThreads - 1) / kRopeThreads;
  const dim3 grid((unsigned)(wgs < 4096 ? wgs : 4096));
  hipLaunchKernelGGL(rope_tables_kernel, grid, dim3(kRopeThreads), 0, stream, a.cos, a.sin,
                     a.max_pos, a.head_dim / 2, a.base);
  return hipGetLastError();
}

hipError_t launch_rope(const RopeArgs& a, hipStream_t stream) {
  RopeParams p;
  p.x[0] = (f16*)a.q;
  p.x[1] = (f16*)a.k;
  p.heads[0] = a.h_q;
  p.heads[1] = a.h_kv;
  p.cu = a.cu_seqlens;
  p.ctx = a.ctx_lens;
  p.cos_t = a.cos;
  p.sin_t = a.sin;
  p.max_pos = a.max_pos;
  p.sign = a.inverse ? -1.f : 1.f;
  const dim3 grid((a.max_seqlen + kRopeTok - 1) / kRopeTok, a.n_seqs, 2);
  if (a.head_dim == 128)
    hipLaunchKernelGGL(rope_kernel<128>, grid, dim3(kRopeThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(rope_kernel<64>, grid, dim3(kRopeThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace cgqa
