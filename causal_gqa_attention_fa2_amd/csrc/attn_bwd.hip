// attn_bwd.hip -- causal GQA attention backward (FlashAttention-2 style) for
// gfx950: dQ, dK, dV by recomputing the softmax from the saved log-sum-exp
// (RL.cu pages: FlashAttention-2 "for both forward and backward passes",
// pitchhut "Project Highlights"; gradient checkpointing, "Key Features" 3).
//
// With P = exp(S - LSE) rebuilt per tile, the backward of O = P V,
// P = softmax(S), S = scale Q K^T is
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Two kernels on one stream, no atomics, bitwise reproducible:
//   1. dq:   query-stationary, shaped like the forward. One work-group per
//            (sequence, query tile, KV head, head chunk); per wave 32 query
//            rows of one head. The wave first forms its rows' D from dO and
//            O (and stores it for kernel 2), then streams K/V tiles through a
//            double-buffered LDS ring: S^T = K Q^T and dP^T = V dO^T (lane =
//            query column, so LSE and D are per-lane scalars), dS^T, and
//            dQ^T += K^T dS^T with K^T taken by transpose reads of the same
//            K tile. dq is written once, in fp16.
//   2. dkdv: key-stationary. One work-group per (sequence, 128-key tile, KV
//            head), four waves of 32 keys; K and V of the wave stay in
//            registers while the (G query heads) x (32-row query blocks at or
//            after the keys) stream through a double-buffered LDS ring:
//            S = Q K^T, dP = dO V^T (lane = key), P and dS, then
//            dV^T += dO^T P and dK^T += Q^T dS with dO^T / Q^T by transpose
//            reads. The G heads of the group add into the same registers.
// Compared with a single key-stationary kernel that adds dQ with fp32
// atomics, this recomputes S and dP once more (7 instead of 5 GEMMs of the
// tile size) but drops the fp32 dQ accumulator, its zeroing, its conversion
// pass and all atomic traffic.
//
// LDS tiles read both row-wise and by transpose reads use the chunk swizzle of
// cdna4.h; a tile read only row-wise is padded by 8 halves per row.
#include "cdna4.h"
#include "kernels.h"

namespace cgqa {
namespace {

constexpr int kBC = 64;               // keys per tile (dq kernel)
constexpr int kWavesK = 4;            // waves per dkdv work-group, 32 keys each
constexpr int kBK = 32 * kWavesK;     // keys per dkdv work-group

struct BwdParams {
  const f16* __restrict__ q;
  const f16* __restrict__ k;
  const f16* __restrict__ v;
  const f16* __restrict__ o;
  const float* __restrict__ lse;
  const f16* __restrict__ dout;
  const int32_t* __restrict__ cu;
  float* __restrict__ drow;  // workspace: fp32 [h_q, T], rowsum(dO * O)
  f16* __restrict__ dq;
  f16* __restrict__ dk;
  f16* __restrict__ dv;
  int n_seqs, T, h_q, h_kv, G, hpw, nqb, n_chunks, n_qtiles, n_ktiles;
  float scale, scale_log2;
};

template <int D, int NTH>
__global__ __launch_bounds__(NTH, 2) void dq_kernel(BwdParams p) {
  constexpr int NT = D / 16;  // MFMA k-steps over the head dimension
  constexpr int ND = D / 32;  // 32-wide output blocks over the head dimension
  constexpr int CH = D / 8;   // 16-byte chunks per row
  constexpr int VP = D + 8;   // V tile pitch (row reads only)
  constexpr int CPT = (kBC * CH + NTH - 1) / NTH;
  __shared__ __attribute__((aligned(16))) f16 Ks[2][kBC * D];  // swizzled
  __shared__ __attribute__((aligned(16))) f16 Vs[2][kBC * VP];

  const int BR = 32 * p.nqb;
  const int per = p.n_seqs * p.h_kv * p.n_chunks;
  const int qt = p.n_qtiles - 1 - (int)blockIdx.x / per;  // heaviest tiles first
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
  const int hig = chunk * p.hpw + wave / p.nqb;
  const int head = g * p.G + min(hig, p.G - 1);
  const int q0 = q_wg0 + (wave % p.nqb) * 32;
  const int qpos = q0 + l32;
  const bool wave_has_rows = q0 < L && hig < p.G;
  const bool qvalid = qpos < L && hig < p.G;
  const int qrow = s0 + min(qpos, L - 1);  // rows past the end read the last row

  // Q^T and dO^T as B operands: lane holds row qpos, columns 16t + 8hi .. +7.
  f16x8 qf[NT], dof[NT];
  float dsum = 0.f;
  {
    const size_t off = ((size_t)qrow * p.h_q + head) * D + 8 * hi;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      qf[t] = *(const f16x8*)(p.q + off + 16 * t);
      dof[t] = *(const f16x8*)(p.dout + off + 16 * t);
      const f16x8 ot = *(const f16x8*)(p.o + off + 16 * t);
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum += (float)dof[t][e] * (float)ot[e];
    }
  }
  dsum = half_swap_sum(dsum);  // D = rowsum(dO * O) over both halves of the row
  const float lse2 = p.lse[(size_t)head * p.T + qrow] * kLog2e;
  if (qvalid && hi == 0) p.drow[(size_t)head * p.T + s0 + qpos] = dsum;

  f16x8 kst[CPT], vst[CPT];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = min(tid + i * NTH, kBC * CH - 1);
      const int r = c / CH;
      const int key = min(kt * kBC + r, L - 1);
      const size_t off = ((size_t)(s0 + key) * p.h_kv + g) * D + (c - r * CH) * 8;
      kst[i] = *(const f16x8*)(p.k + off);
      vst[i] = *(const f16x8*)(p.v + off);
    }
  };
  // Keys past the end become zero rows (their scores are masked and their
  // dS is zero, so only finiteness matters).
  auto store_tile = [&](int kt, int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NTH;
      if (c < kBC * CH) {
        const int r = c / CH;
        const int cc = c - r * CH;
        const bool ok = kt * kBC + r < L;
        *(f16x8*)(Ks[buf] + r * D + swz<D>(r, cc * 8)) = ok ? kst[i] : zero_f16x8();
        *(f16x8*)(Vs[buf] + r * VP + cc * 8) = ok ? vst[i] : zero_f16x8();
      }
    }
  };

  f32x16 dq_acc[ND];  // dQ^T: rows = head dim, cols = queries
#pragma unroll
  for (int db = 0; db < ND; ++db) dq_acc[db] = zero_f32x16();

  load_tile(0);
  store_tile(0, 0);
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < n_kt;
    if (more) load_tile(kt + 1);

    if (wave_has_rows && kt * kBC <= q0 + 31) {
      const f16* Kb = Ks[buf];
      const f16* Vb = Vs[buf];
      const bool diag = kt * kBC + kBC - 1 > q0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // S^T = K Q^T and dP^T = V dO^T for 32 keys (accumulator element i:
        // key kt*64 + 32kb + 8(i/4) + 4hi + i%4, query qpos).
        f32x16 s = zero_f32x16(), dp = zero_f32x16();
        const int kr = kb * 32 + l32;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          s = mfma32x32x16(*(const f16x8*)(Kb + kr * D + swz<D>(kr, 16 * t + 8 * hi)), qf[t], s);
          dp = mfma32x32x16(*(const f16x8*)(Vb + kr * VP + 16 * t + 8 * hi), dof[t], dp);
        }
        f16x8 dsf[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pv = fast_exp2(fmaf(s[i], p.scale_log2, -lse2));
          if (diag) {
            const int key = kt * kBC + kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
            if (key > qpos) pv = 0.f;
          }
          dsf[i >> 3][i & 7] = (f16)(pv * (dp[i] - dsum));
        }
        // dQ^T += K^T dS^T over these 32 keys; K^T by transpose reads of the
        // K tile (A slot e of half hi <-> key 16u + 8(e/4) + 4hi + e%4).
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const int col = 32 * db + 16 * (grp & 1) + 4 * (j16 & 3);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int r0 = kb * 32 + 16 * u + 4 * hi + (j16 >> 2);
            const int r1 = r0 + 8;
            const f16x8 a = cat4(lds_read_tr(Kb + r0 * D + swz<D>(r0, col)),
                                 lds_read_tr(Kb + r1 * D + swz<D>(r1, col)));
            dq_acc[db] = mfma32x32x16(a, dsf[u], dq_acc[db]);
          }
        }
      }
    }

    if (more) store_tile(kt + 1, buf ^ 1);
    __syncthreads();
  }

  if (!qvalid) return;
  f16* dqrow = p.dq + ((size_t)(s0 + qpos) * p.h_q + head) * D;
#pragma unroll
  for (int db = 0; db < ND; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (f16)(dq_acc[db][4 * r4 + e] * p.scale);
      *(f16x4*)(dqrow + 32 * db + 8 * r4 + 4 * hi) = w;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void dkdv_kernel(BwdParams p) {
  constexpr int NT = D / 16;
  constexpr int ND = D / 32;
  constexpr int CH = D / 8;
  constexpr int CPT = (32 * CH + 255) / 256;  // chunks per thread of a Q (or dO) block
  __shared__ __attribute__((aligned(16))) f16 Qs[2][32 * D];   // swizzled
  __shared__ __attribute__((aligned(16))) f16 dOs[2][32 * D];  // swizzled
  __shared__ __attribute__((aligned(16))) float lse_s[2][32];
  __shared__ __attribute__((aligned(16))) float drow_s[2][32];

  // Key tile 0 of every (sequence, KV head) sees the most query rows: first.
  const int per = p.n_seqs * p.h_kv;
  const int kt = (int)blockIdx.x / per;
  const int rem = (int)blockIdx.x % per;
  const int g = rem % p.h_kv;
  const int b = rem / p.h_kv;
  const int s0 = p.cu[b];
  const int L = p.cu[b + 1] - s0;
  const int k_wg0 = kt * kBK;
  if (k_wg0 >= L) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int grp = lane >> 4;
  const int j16 = lane & 15;
  const int kw0 = k_wg0 + 32 * wave;  // first key of this wave
  const int key = kw0 + l32;
  const bool kvalid = key < L;

  // K^T and V^T B operands of this wave: lane holds row `key` (rows past the
  // end read the last row: their scores are masked), columns 16t + 8hi .. +7.
  f16x8 kf[NT], vf[NT];
  {
    const size_t off = ((size_t)(s0 + min(key, L - 1)) * p.h_kv + g) * D + 8 * hi;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      kf[t] = *(const f16x8*)(p.k + off + 16 * t);
      vf[t] = *(const f16x8*)(p.v + off + 16 * t);
    }
  }

  // Query blocks at or after the key tile, for each head of the group.
  const int qb_begin = k_wg0 / 32;
  const int n_qb = (L + 31) / 32 - qb_begin;
  const int n_it = p.G * n_qb;

  f16x8 qst[CPT], dst[CPT];
  float aux = 0.f;  // lse (threads 0..31) or D (threads 32..63) of the staged block
  auto load_blk = [&](int it) {
    const int head = g * p.G + it / n_qb;
    const int q0 = (qb_begin + it % n_qb) * 32;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = min(tid + i * 256, 32 * CH - 1);
      const int r = c / CH;
      const size_t off =
          ((size_t)(s0 + min(q0 + r, L - 1)) * p.h_q + head) * D + (c - r * CH) * 8;
      qst[i] = *(const f16x8*)(p.q + off);
      dst[i] = *(const f16x8*)(p.dout + off);
    }
    if (tid < 64) {
      const size_t ix = (size_t)head * p.T + s0 + min(q0 + (tid & 31), L - 1);
      aux = tid < 32 ? p.lse[ix] : p.drow[ix];
    }
  };
  auto store_blk = [&](int it, int buf) {
    const int q0 = (qb_begin + it % n_qb) * 32;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * 256;
      if (c < 32 * CH) {
        const int r = c / CH;
        const int cc = c - r * CH;
        *(f16x8*)(Qs[buf] + r * D + swz<D>(r, cc * 8)) = qst[i];
        *(f16x8*)(dOs[buf] + r * D + swz<D>(r, cc * 8)) = dst[i];
      }
    }
    if (tid < 64) {
      const bool ok = q0 + (tid & 31) < L;  // rows past the end: P = 0
      if (tid < 32) lse_s[buf][tid] = ok ? aux * kLog2e : INFINITY;
      else drow_s[buf][tid - 32] = ok ? aux : 0.f;
    }
  };

  f32x16 dk_acc[ND], dv_acc[ND];  // dK^T, dV^T: rows = head dim, cols = keys
#pragma unroll
  for (int db = 0; db < ND; ++db) {
    dk_acc[db] = zero_f32x16();
    dv_acc[db] = zero_f32x16();
  }

  load_blk(0);
  store_blk(0, 0);
  __syncthreads();
  for (int it = 0; it < n_it; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < n_it;
    if (more) load_blk(it + 1);
    const int q0 = (qb_begin + it % n_qb) * 32;

    // Waves whose keys all lie after the block's last query see only masked pairs.
    if (kw0 <= q0 + 31 && kw0 < L) {
      const f16* Qb = Qs[buf];
      const f16* dOb = dOs[buf];
      f32x16 s = zero_f32x16(), dp = zero_f32x16();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int col = swz<D>(l32, 16 * t + 8 * hi);
        s = mfma32x32x16(*(const f16x8*)(Qb + l32 * D + col), kf[t], s);
        dp = mfma32x32x16(*(const f16x8*)(dOb + l32 * D + col), vf[t], dp);
      }
      // Accumulator element i: query row q0 + 8(i/4) + 4hi + i%4, key `key`.
      const bool need_mask = kw0 + 31 > q0;
      f16x8 pf[2], dsf[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qr = 8 * (i >> 2) + 4 * hi + (i & 3);
        float pv = fast_exp2(fmaf(s[i], p.scale_log2, -lse_s[buf][qr]));
        if (need_mask && key > q0 + qr) pv = 0.f;
        pf[i >> 3][i & 7] = (f16)pv;
        dsf[i >> 3][i & 7] = (f16)(pv * (dp[i] - drow_s[buf][qr]));
      }
      // dV^T += dO^T P and dK^T += Q^T dS; A-operand slot e of half hi holds
      // query row 16u + 8(e/4) + 4hi + e%4, matching the B slots.
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const int col = 32 * db + 16 * (grp & 1) + 4 * (j16 & 3);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r0 = 16 * u + 4 * hi + (j16 >> 2);
          const int r1 = r0 + 8;
          const int c0 = swz<D>(r0, col), c1 = swz<D>(r1, col);
          const f16x8 a_do = cat4(lds_read_tr(dOb + r0 * D + c0), lds_read_tr(dOb + r1 * D + c1));
          dv_acc[db] = mfma32x32x16(a_do, pf[u], dv_acc[db]);
          const f16x8 a_q = cat4(lds_read_tr(Qb + r0 * D + c0), lds_read_tr(Qb + r1 * D + c1));
          dk_acc[db] = mfma32x32x16(a_q, dsf[u], dk_acc[db]);
        }
      }
    }

    if (more) store_blk(it + 1, buf ^ 1);
    __syncthreads();
  }

  if (!kvalid) return;
  const size_t off = ((size_t)(s0 + key) * p.h_kv + g) * D;
#pragma unroll
  for (int db = 0; db < ND; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f16x4 wk, wv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wk[e] = (f16)(dk_acc[db][4 * r4 + e] * p.scale);
        wv[e] = (f16)dv_acc[db][4 * r4 + e];
      }
      const int d = 32 * db + 8 * r4 + 4 * hi;
      *(f16x4*)(p.dk + off + d) = wk;
      *(f16x4*)(p.dv + off + d) = wv;
    }
  }
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  BwdParams p;
  p.q = (const f16*)a.q;
  p.k = (const f16*)a.k;
  p.v = (const f16*)a.v;
  p.o = (const f16*)a.o;
  p.lse = a.lse;
  p.dout = (const f16*)a.dout;
  p.cu = a.cu_seqlens;
  p.drow = a.drow;
  p.dq = (f16*)a.dq;
  p.dk = (f16*)a.dk;
  p.dv = (f16*)a.dv;
  p.n_seqs = a.n_seqs;
  p.T = a.total_tokens;
  p.h_q = a.h_q;
  p.h_kv = a.h_kv;
  p.G = a.h_q / a.h_kv;
  p.hpw = p.G < 4 ? p.G : 4;
  p.nqb = 4 / p.hpw;
  p.n_chunks = (p.G + p.hpw - 1) / p.hpw;
  p.n_qtiles = (a.max_seqlen + 32 * p.nqb - 1) / (32 * p.nqb);
  p.n_ktiles = (a.max_seqlen + kBK - 1) / kBK;
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  const dim3 gq(p.n_qtiles * a.n_seqs * a.h_kv * p.n_chunks);
  const dim3 gk(p.n_ktiles * a.n_seqs * a.h_kv);
  const int nth = 64 * p.hpw * p.nqb;  // 256, or 192 when G == 3
  if (a.head_dim == 128) {
    if (nth == 256) hipLaunchKernelGGL((dq_kernel<128, 256>), gq, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((dq_kernel<128, 192>), gq, dim3(192), 0, stream, p);
    hipLaunchKernelGGL(dkdv_kernel<128>, gk, dim3(256), 0, stream, p);
  } else {
    if (nth == 256) hipLaunchKernelGGL((dq_kernel<64, 256>), gq, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((dq_kernel<64, 192>), gq, dim3(192), 0, stream, p);
    hipLaunchKernelGGL(dkdv_kernel<64>, gk, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace cgqa
