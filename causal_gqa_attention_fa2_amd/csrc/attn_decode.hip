// attn_decode.hip -- single-token decode attention over a paged KV cache for
// gfx950 (the rollout engine's paged key-value caching; pitchhut "Key
// Features" item 2, mlllm.io "What happened").
//
// Every sequence has one query token per head; its context lives in 16-token
// blocks of a shared pool, addressed through the sequence's block table. The
// work is a gather-and-reduce that reads every context key and value once,
// so it is bound by HBM bandwidth; it runs on the vector ALUs, not on MFMA.
//
// Split-context scheme (two launches):
//   1. split:   one work-group (4 waves) per (sequence, KV head, 512-token
//               split). A wave takes every 4th block of the split; in a wave
//               each token row of a block is held by D/8 lanes with 16 bytes
//               each, so one load instruction gathers 64 / (D/8) rows. The G
//               query heads of the KV head share every loaded block.
//               Each lane keeps an online-softmax state (max, sum, 8 output
//               columns) per query head; the states are merged across the
//               lanes' token rows, across waves through LDS, and written as
//               the split's partial (unnormalised output, max, sum).
//   2. combine: per (sequence, query head), merge the splits' partials by
//               their maxima and write fp16 output.
#include "cdna4.h"
#include "kernels.h"

namespace cgqa {
namespace {

constexpr int kMaxG = 16;

struct DecParams {
  const f16* __restrict__ q;
  const f16* __restrict__ kp;
  const f16* __restrict__ vp;
  const int32_t* __restrict__ bt;
  const int32_t* __restrict__ ctx;
  f16* __restrict__ o;
  float* __restrict__ part_o;
  float* __restrict__ part_ml;
  int n, h_q, h_kv, G, max_blocks, max_splits;
  float scale_log2;
};

struct SoftState {
  float m, l;
  float a[8];
};

__device__ __forceinline__ void merge_state(SoftState& s, float m2, float l2, const float* a2) {
  const float M = fmaxf(s.m, m2);
  const float c1 = fast_exp2(s.m - M);
  const float c2 = fast_exp2(m2 - M);
  s.l = s.l * c1 + l2 * c2;
#pragma unroll
  for (int e = 0; e < 8; ++e) s.a[e] = s.a[e] * c1 + a2[e] * c2;
  s.m = M;
}

template <int D, int G>
__global__ __launch_bounds__(256) void decode_split_kernel(DecParams p) {
  constexpr int LPR = D / 8;      // lanes per token row
  constexpr int TPI = 64 / LPR;   // token rows per load instruction
  constexpr int NLD = 16 / TPI;   // load instructions per 16-token block
  __shared__ float xch[4][G][LPR][10];

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int ctx = p.ctx[b];
  const int t_begin = split * kDecodeSplit;
  if (t_begin >= ctx) return;
  const int t_end = min(ctx, t_begin + kDecodeSplit);
  const int blk_begin = t_begin / 16;
  const int blk_end = (t_end + 15) / 16;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int rg = lane / LPR;  // token row within a load instruction
  const int dc = lane % LPR;  // 8-column chunk of the head dimension

  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const f16x8 x = *(const f16x8*)(p.q + ((size_t)b * p.h_q + g * G + h) * D + dc * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[h][e] = (float)x[e] * p.scale_log2;
  }
  SoftState st[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st[h].m = kMaxInit;
    st[h].l = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st[h].a[e] = 0.f;
  }

  const int32_t* table = p.bt + (size_t)b * p.max_blocks;
  const size_t row_stride = (size_t)p.h_kv * D;  // halves between token rows
  for (int blk = blk_begin + wave; blk < blk_end; blk += 4) {
    const int phys = table[blk];
    const f16* kb = p.kp + ((size_t)phys * 16) * row_stride + (size_t)g * D + dc * 8;
    const f16* vb = p.vp + ((size_t)phys * 16) * row_stride + (size_t)g * D + dc * 8;
    f16x8 kr[NLD], vr[NLD];
    bool ok[NLD];
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int tok = j * TPI + rg;
      ok[j] = blk * 16 + tok < t_end;
      kr[j] = zero_f16x8();
      vr[j] = zero_f16x8();
      if (ok[j]) {
        kr[j] = *(const f16x8*)(kb + (size_t)tok * row_stride);
        vr[j] = *(const f16x8*)(vb + (size_t)tok * row_stride);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s[NLD];
      float mx = kMaxInit;
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += qv[h][e] * (float)kr[j][e];
#pragma unroll
        for (int w = LPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, LPR);
        s[j] = ok[j] ? acc : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      const float m_new = fmaxf(st[h].m, mx);
      const float alpha = fast_exp2(st[h].m - m_new);
      st[h].m = m_new;
      st[h].l *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) st[h].a[e] *= alpha;
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const float pj = fast_exp2(s[j] - m_new);
        st[h].l += pj;
#pragma unroll
        for (int e = 0; e < 8; ++e) st[h].a[e] += pj * (float)vr[j][e];
      }
    }
  }

  // Merge the TPI token rows of the wave (lanes dc, dc + LPR, ...).
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int w = LPR; w < 64; w <<= 1) {
      float a2[8];
      const float m2 = __shfl_xor(st[h].m, w);
      const float l2 = __shfl_xor(st[h].l, w);
#pragma unroll
      for (int e = 0; e < 8; ++e) a2[e] = __shfl_xor(st[h].a[e], w);
      merge_state(st[h], m2, l2, a2);
    }
    if (rg == 0) {
      xch[wave][h][dc][0] = st[h].m;
      xch[wave][h][dc][1] = st[h].l;
#pragma unroll
      for (int e = 0; e < 8; ++e) xch[wave][h][dc][2 + e] = st[h].a[e];
    }
  }
  __syncthreads();
  // Threads (h, dc) of the first G * LPR merge the four waves.
  if (tid < G * LPR) {
    const int h = tid / LPR;
    const int c = tid % LPR;
    SoftState s;
    s.m = xch[0][h][c][0];
    s.l = xch[0][h][c][1];
#pragma unroll
    for (int e = 0; e < 8; ++e) s.a[e] = xch[0][h][c][2 + e];
#pragma unroll
    for (int w = 1; w < 4; ++w) merge_state(s, xch[w][h][c][0], xch[w][h][c][1], &xch[w][h][c][2]);
    const size_t slot = ((size_t)b * p.h_q + g * G + h) * p.max_splits + split;
    float* po = p.part_o + slot * D + c * 8;
    *(f32x4*)po = f32x4{s.a[0], s.a[1], s.a[2], s.a[3]};
    *(f32x4*)(po + 4) = f32x4{s.a[4], s.a[5], s.a[6], s.a[7]};
    if (c == 0) {
      p.part_ml[2 * slot] = s.m;
      p.part_ml[2 * slot + 1] = s.l;
    }
  }
}

// One wave per (sequence, query head): merge the splits, normalise, store.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecParams p) {
  constexpr int PER = D / 64;  // output columns per lane
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= p.n * p.h_q) return;
  const int b = row / p.h_q;
  const int ctx = p.ctx[b];
  const int ns = (ctx + kDecodeSplit - 1) / kDecodeSplit;
  f16* out = p.o + (size_t)row * D + lane * PER;
  if (ns == 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = (f16)0.f;
    return;
  }
  const float* ml = p.part_ml + (size_t)row * p.max_splits * 2;
  float M = kMaxInit;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
  float l = 0.f, acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float c = fast_exp2(ml[2 * s] - M);
    l += ml[2 * s + 1] * c;
    const float* po = p.part_o + ((size_t)row * p.max_splits + s) * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] += po[e] * c;
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[e] = (f16)(acc[e] * inv);
}

template <int D>
hipError_t launch_d(const DecParams& p, int G, hipStream_t stream) {
  const dim3 grid(p.max_splits, p.h_kv, p.n);
  // With every context empty there is nothing to gather; combine writes zeros.
  if (p.max_splits > 0) switch (G) {
#define CGQA_G(GG) \
  case GG: hipLaunchKernelGGL((decode_split_kernel<D, GG>), grid, dim3(256), 0, stream, p); break;
    CGQA_G(1) CGQA_G(2) CGQA_G(3) CGQA_G(4) CGQA_G(5) CGQA_G(6) CGQA_G(7) CGQA_G(8)
    CGQA_G(9) CGQA_G(10) CGQA_G(11) CGQA_G(12) CGQA_G(13) CGQA_G(14) CGQA_G(15) CGQA_G(16)
#undef CGQA_G
    default: return hipErrorInvalidValue;
  }
  const int rows = p.n * p.h_q;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3((rows + 3) / 4), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  DecParams p;
  p.q = (const f16*)a.q;
  p.kp = (const f16*)a.k_pool;
  p.vp = (const f16*)a.v_pool;
  p.bt = a.block_table;
  p.ctx = a.ctx_lens;
  p.o = (f16*)a.o;
  p.part_o = a.part_o;
  p.part_ml = a.part_ml;
  p.n = a.n_seqs;
  p.h_q = a.h_q;
  p.h_kv = a.h_kv;
  p.G = a.h_q / a.h_kv;
  p.max_blocks = a.max_blocks_per_seq;
  p.max_splits = a.max_splits;
  p.scale_log2 = a.scale * kLog2e;
  if (p.G > kMaxG) return hipErrorInvalidValue;
  return a.head_dim == 128 ? launch_d<128>(p, p.G, stream) : launch_d<64>(p, p.G, stream);
}

}  // namespace cgqa
