// attn_fwd.hip -- causal GQA attention forward (FlashAttention-2 style) for
// gfx950.
//
// Method (FlashAttention-2 forward as named on the RL.cu pages, pitchhut
// "Project Highlights"): keys and values stream through LDS tile by tile;
// each query row keeps a running maximum m, a running sum l of
// exp(score - m) and an unnormalised output accumulator, rescaled whenever m
// grows (online softmax); the end divides by l and saves
// LSE = m + ln l for the backward pass. FP16 inputs, FP32 accumulation
// (pitchhut "Key Features", item 1).
//
// Work decomposition. One work-group of at most four waves per (sequence,
// query tile, KV head, head chunk). A chunk holds hpw = min(G, 4) of the
// G = h_q / h_kv query heads of the KV head and the query tile
// BR = 32 * nqb positions (nqb = 4 / hpw), one 64-lane wave per (head, 32
// positions). For G <= 4 there is one chunk, so every K/V tile is read from
// HBM once per KV head and shared by all G heads through LDS
// (grouped-query sharing).
//
// Per wave and 64-key tile, everything stays in registers:
//   S^T = K Q^T      32x32x16 MFMA; K from LDS (rows = keys), Q^T from
//                    registers. In the accumulator layout lane l owns query
//                    column l % 32, so a row's max and sum are an in-lane
//                    reduction plus one permlane32 exchange.
//   P^T = exp2(S^T * scale * log2(e) - m)        (fp32, then fp16)
//   O^T += V^T P^T   32x32x16 MFMA; P^T feeds the B operand straight from
//                    the S^T accumulators; V^T is read from the row-major V
//                    tile with ds_read_b64_tr_b16.
#include "cdna4.h"
#include "kernels.h"

namespace cgqa {
namespace {

constexpr int kBC = 64;  // keys per tile

struct FwdParams {
  const f16* __restrict__ q;
  const f16* __restrict__ k;
  const f16* __restrict__ v;
  const int32_t* __restrict__ cu;
  f16* __restrict__ o;
  float* __restrict__ lse;
  int n_seqs, T, h_q, h_kv, G, hpw, nqb, n_chunks, n_qtiles;
  float scale_log2;  // scale * log2(e)
};

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdParams p) {
  constexpr int KP = D + 8;   // K tile row pitch (halves): natural 16-byte reads
  constexpr int VP = D + 16;  // V tile row pitch (halves): transpose reads
  constexpr int NT = D / 16;  // MFMA k-steps over the head dimension
  constexpr int ND = D / 32;  // 32-wide output blocks over the head dimension
  __shared__ __attribute__((aligned(16))) f16 Ks[kBC * KP];
  __shared__ __attribute__((aligned(16))) f16 Vs[kBC * VP];

  const int BR = 32 * p.nqb;
  // Heaviest query tiles (the last ones of the longest sequences) first.
  const int per = p.n_seqs * p.h_kv * p.n_chunks;
  const int qt = p.n_qtiles - 1 - (int)blockIdx.x / per;
  int rem = (int)blockIdx.x % per;
  const int chunk = rem % p.n_chunks;
  rem /= p.n_chunks;
  const int g = rem % p.h_kv;
  const int b = rem / p.h_kv;
  const int s0 = p.cu[b];
  const int L = p.cu[b + 1] - s0;
  const int q_wg0 = qt * BR;
  if (q_wg0 >= L) return;  // uniform over the work-group
  const int n_kt = (min(L, q_wg0 + BR) + kBC - 1) / kBC;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int grp = lane >> 4;
  const int j16 = lane & 15;
  const int hig = chunk * p.hpw + wave / p.nqb;  // head within the group
  const int head = g * p.G + hig;
  const int q0 = q_wg0 + (wave % p.nqb) * 32;
  const int qpos = q0 + l32;
  const bool qvalid = qpos < L && hig < p.G;

  // Q^T as the B operand: lane holds Q[qpos][16t + 8hi .. +7].
  f16x8 qf[NT];
  {
    const f16* qrow = p.q + ((size_t)(s0 + qpos) * p.h_q + head) * D + 8 * hi;
#pragma unroll
    for (int t = 0; t < NT; ++t) qf[t] = zero_f16x8();
    if (qvalid) {
#pragma unroll
      for (int t = 0; t < NT; ++t) qf[t] = *(const f16x8*)(qrow + 16 * t);
    }
  }

  f32x16 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = zero_f32x16();
  float m_run = kMaxInit;
  float l_run = 0.f;  // this half-wave's share of the row sum

  const int nthreads = blockDim.x;
  constexpr int CH = D / 8;  // 16-byte chunks per row
  const bool wave_has_rows = q0 < L && hig < p.G;

  for (int kt = 0; kt < n_kt; ++kt) {
    __syncthreads();  // previous tile fully consumed
    for (int c = tid; c < kBC * CH; c += nthreads) {
      const int r = c / CH;
      const int cc = c - r * CH;
      const int key = kt * kBC + r;
      f16x8 kv = zero_f16x8(), vv = zero_f16x8();
      if (key < L) {
        const size_t off = ((size_t)(s0 + key) * p.h_kv + g) * D + cc * 8;
        kv = *(const f16x8*)(p.k + off);
        vv = *(const f16x8*)(p.v + off);
      }
      *(f16x8*)(Ks + r * KP + cc * 8) = kv;
      *(f16x8*)(Vs + r * VP + cc * 8) = vv;
    }
    __syncthreads();
    if (!wave_has_rows || kt * kBC > q0 + 31) continue;  // tile fully masked for this wave

    // S^T for the two 32-key halves of the tile.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero_f32x16();
      const f16* krow = Ks + (kb * 32 + l32) * KP + 8 * hi;
#pragma unroll
      for (int t = 0; t < NT; ++t) s[kb] = mfma32x32x16(*(const f16x8*)(krow + 16 * t), qf[t], s[kb]);
    }

    // Scale into log2 units, causal mask, tile maximum.
    const bool need_mask = kt * kBC + kBC - 1 > q0;
    float mx = kMaxInit;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[kb][i] * p.scale_log2;
        if (need_mask) {
          const int key = kt * kBC + kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
          if (key > qpos) x = -INFINITY;
        }
        s[kb][i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = half_swap_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;

    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(s[kb][i] - m_new);
        s[kb][i] = e;
        rs += e;
      }
    }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }

    // P^T as B operands: k-step u covers tile keys 16u..16u+15; slot s of
    // half hi holds key 16u + 8(s/4) + 4hi + s%4.
    f16x8 pf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[u][e] = (f16)s[u >> 1][8 * (u & 1) + e];
    }

    // O^T += V^T P^T. A operand slot s of half hi must hold V[key(s)][d]
    // for the same keys: two transpose reads of 4 rows each.
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int dcol = 32 * db + 16 * (grp & 1) + 4 * (j16 & 3);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int krow = 16 * u + 4 * hi + (j16 >> 2);
        const f16x4 lo = lds_read_tr(Vs + krow * VP + dcol);
        const f16x4 up = lds_read_tr(Vs + (krow + 8) * VP + dcol);
        oacc[db] = mfma32x32x16(cat4(lo, up), pf[u], oacc[db]);
      }
    }
  }

  const float l_tot = half_swap_sum(l_run);  // all lanes take part in the exchange
  if (!qvalid) return;
  const float inv = 1.f / l_tot;
  f16* orow = p.o + ((size_t)(s0 + qpos) * p.h_q + head) * D;
#pragma unroll
  for (int db = 0; db < ND; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (f16)(oacc[db][4 * r4 + e] * inv);
      *(f16x4*)(orow + 32 * db + 8 * r4 + 4 * hi) = w;
    }
  }
  if (hi == 0) p.lse[(size_t)head * p.T + s0 + qpos] = m_run * kLn2 + logf(l_tot);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  FwdParams p;
  p.q = (const f16*)a.q;
  p.k = (const f16*)a.k;
  p.v = (const f16*)a.v;
  p.cu = a.cu_seqlens;
  p.o = (f16*)a.o;
  p.lse = a.lse;
  p.n_seqs = a.n_seqs;
  p.T = a.total_tokens;
  p.h_q = a.h_q;
  p.h_kv = a.h_kv;
  p.G = a.h_q / a.h_kv;
  p.hpw = p.G < 4 ? p.G : 4;
  p.nqb = 4 / p.hpw;
  p.n_chunks = (p.G + p.hpw - 1) / p.hpw;
  const int BR = 32 * p.nqb;
  p.n_qtiles = (a.max_seqlen + BR - 1) / BR;
  p.scale_log2 = a.scale * kLog2e;
  const dim3 grid(p.n_qtiles * a.n_seqs * a.h_kv * p.n_chunks);
  const dim3 block(64 * p.hpw * p.nqb);
  if (a.head_dim == 128)
    hipLaunchKernelGGL(fwd_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(fwd_kernel<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace cgqa
