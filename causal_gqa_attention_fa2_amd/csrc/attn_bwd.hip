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
// Three launches on one stream:
//   1. prep:    D[h, t] = rowsum(dO * O) in fp32 and dQ_acc = 0.
//   2. main:    one work-group per (sequence, 128-key tile, KV head), four
//               waves of 32 keys. K and V of the wave stay in registers; the
//               loop runs over the G query heads of the KV head and over the
//               32-row query blocks at or after the key tile (causal).
//               dK and dV accumulate in registers across the whole loop (GQA:
//               the G heads add into the same accumulators). dS^T goes
//               through LDS so the work-group can form dQ_blk = dS K over its
//               128 keys, which is added into the fp32 dQ_acc with atomics.
//   3. convert: dq = fp16(scale * dQ_acc).
//
// MFMA shapes (32x32x16, accumulators C[row][col], lane owns column l % 32):
//   S  = Q K^T   : A = Q rows from LDS, B = K^T from registers -> lane = key
//   dP = dO V^T  : A = dO rows from LDS, B = V^T from registers
//   dV^T += dO^T P   and   dK^T += Q^T dS : B = P / dS straight from the
//                  S / dP accumulators, A = dO^T / Q^T by transpose reads
//   dQ_blk = dS K: A = dS via transpose reads of dS^T, B = K via transpose
//                  reads of the K tile.
#include "cdna4.h"
#include "kernels.h"

namespace cgqa {
namespace {

constexpr int kWavesK = 4;            // waves per work-group, 32 keys each
constexpr int kBK = 32 * kWavesK;     // keys per work-group
constexpr int kDSP = 32 + 16;         // dS^T tile pitch (halves)

struct BwdParams {
  const f16* __restrict__ q;
  const f16* __restrict__ k;
  const f16* __restrict__ v;
  const f16* __restrict__ o;
  const float* __restrict__ lse;
  const f16* __restrict__ dout;
  const int32_t* __restrict__ cu;
  float* __restrict__ dq_acc;
  float* __restrict__ drow;
  f16* __restrict__ dq;
  f16* __restrict__ dk;
  f16* __restrict__ dv;
  int n_seqs, T, h_q, h_kv, G, n_ktiles;
  float scale, scale_log2;
};

// D[h, t] = sum_d dO[t, h, d] * O[t, h, d]; zero dQ_acc. One row per
// D/8 lanes, 16 bytes per lane.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
  constexpr int LPR = D / 8;
  const int rows = p.T * p.h_q;
  const int row = blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + c * 8;
    const f16x8 a = *(const f16x8*)(p.dout + off);
    const f16x8 b = *(const f16x8*)(p.o + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *(f32x4*)(p.dq_acc + off) = z;
    *(f32x4*)(p.dq_acc + off + 4) = z;
  }
#pragma unroll
  for (int w = LPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, LPR);
  if (row < rows && c == 0) {
    const int t = row / p.h_q;
    const int h = row - t * p.h_q;
    p.drow[(size_t)h * p.T + t] = acc;
  }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_main_kernel(BwdParams p) {
  constexpr int NT = D / 16;
  constexpr int ND = D / 32;
  constexpr int KP = D + 16;  // K tile pitch (transpose reads)
  constexpr int QP = D + 16;  // Q / dO block pitch
  __shared__ __attribute__((aligned(16))) f16 Ks[kBK * KP];
  __shared__ __attribute__((aligned(16))) f16 Qs[32 * QP];
  __shared__ __attribute__((aligned(16))) f16 dOs[32 * QP];
  __shared__ __attribute__((aligned(16))) f16 dSs[kBK * kDSP];
  __shared__ float lse_s[32];
  __shared__ float drow_s[32];

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

  // K tile -> LDS (zero past the sequence end).
  constexpr int CH = D / 8;
  for (int c = tid; c < kBK * CH; c += 256) {
    const int r = c / CH;
    const int cc = c - r * CH;
    f16x8 kv = zero_f16x8();
    if (k_wg0 + r < L) kv = *(const f16x8*)(p.k + ((size_t)(s0 + k_wg0 + r) * p.h_kv + g) * D + cc * 8);
    *(f16x8*)(Ks + r * KP + cc * 8) = kv;
  }
  // K^T and V^T B operands of this wave: lane holds row `key`, columns
  // 16t + 8hi .. +7.
  f16x8 kf[NT], vf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    kf[t] = zero_f16x8();
    vf[t] = zero_f16x8();
  }
  if (kvalid) {
    const size_t off = ((size_t)(s0 + key) * p.h_kv + g) * D + 8 * hi;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      kf[t] = *(const f16x8*)(p.k + off + 16 * t);
      vf[t] = *(const f16x8*)(p.v + off + 16 * t);
    }
  }

  f32x16 dk_acc[ND], dv_acc[ND];  // dK^T, dV^T: rows = head dim, cols = keys
#pragma unroll
  for (int db = 0; db < ND; ++db) {
    dk_acc[db] = zero_f32x16();
    dv_acc[db] = zero_f32x16();
  }

  const int qb_begin = k_wg0 / 32;
  const int qb_end = (L + 31) / 32;
  for (int hh = 0; hh < p.G; ++hh) {
    const int head = g * p.G + hh;
    for (int qb = qb_begin; qb < qb_end; ++qb) {
      const int q0 = qb * 32;
      __syncthreads();  // LDS of the previous block fully consumed
      for (int c = tid; c < 32 * CH; c += 256) {
        const int r = c / CH;
        const int cc = c - r * CH;
        f16x8 qv = zero_f16x8(), dov = zero_f16x8();
        if (q0 + r < L) {
          const size_t off = ((size_t)(s0 + q0 + r) * p.h_q + head) * D + cc * 8;
          qv = *(const f16x8*)(p.q + off);
          dov = *(const f16x8*)(p.dout + off);
        }
        *(f16x8*)(Qs + r * QP + cc * 8) = qv;
        *(f16x8*)(dOs + r * QP + cc * 8) = dov;
      }
      if (tid < 32) {
        float lv = INFINITY, dv = 0.f;  // rows past the end: P = 0
        if (q0 + tid < L) {
          const size_t ix = (size_t)head * p.T + s0 + q0 + tid;
          lv = p.lse[ix] * kLog2e;
          dv = p.drow[ix];
        }
        lse_s[tid] = lv;
        drow_s[tid] = dv;
      }
      __syncthreads();

      // Waves whose keys all lie after the block's last query see only masked
      // pairs; they contribute zero dS rows.
      const bool active = kw0 <= q0 + 31 && kw0 < L;
      f16* ds_row = dSs + (32 * wave + l32) * kDSP;
      if (active) {
        f32x16 s = zero_f32x16(), dp = zero_f32x16();
        const f16* qrow = Qs + l32 * QP + 8 * hi;
        const f16* dorow = dOs + l32 * QP + 8 * hi;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          s = mfma32x32x16(*(const f16x8*)(qrow + 16 * t), kf[t], s);
          dp = mfma32x32x16(*(const f16x8*)(dorow + 16 * t), vf[t], dp);
        }
        // Accumulator element i: query row 8(i/4) + 4hi + i%4, key `key`.
        const bool need_mask = kw0 + 31 > q0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qr = 8 * (i >> 2) + 4 * hi + (i & 3);
          float pv = fast_exp2(s[i] * p.scale_log2 - lse_s[qr]);
          if (need_mask && key > q0 + qr) pv = 0.f;
          s[i] = pv;
          dp[i] = pv * (dp[i] - drow_s[qr]);
        }
        f16x8 pf[2], dsf[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pf[u][e] = (f16)s[8 * u + e];
            dsf[u][e] = (f16)dp[8 * u + e];
          }
        }
        // dV^T += dO^T P and dK^T += Q^T dS. A-operand slot s of half hi
        // holds query row 16u + 8(s/4) + 4hi + s%4, matching the B slots.
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const int dcol = 32 * db + 16 * (grp & 1) + 4 * (j16 & 3);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int r = 16 * u + 4 * hi + (j16 >> 2);
            const f16x8 a_do = cat4(lds_read_tr(dOs + r * QP + dcol), lds_read_tr(dOs + (r + 8) * QP + dcol));
            dv_acc[db] = mfma32x32x16(a_do, pf[u], dv_acc[db]);
            const f16x8 a_q = cat4(lds_read_tr(Qs + r * QP + dcol), lds_read_tr(Qs + (r + 8) * QP + dcol));
            dk_acc[db] = mfma32x32x16(a_q, dsf[u], dk_acc[db]);
          }
        }
        // dS^T row `key`: query columns 8(i/4) + 4hi + 0..3.
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (f16)dp[4 * r4 + e];
          *(f16x4*)(ds_row + 8 * r4 + 4 * hi) = w;
        }
      } else {
        const f16x4 z = {0, 0, 0, 0};
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) *(f16x4*)(ds_row + 8 * r4 + 4 * hi) = z;
      }
      __syncthreads();

      // dQ_blk[q][d] = sum over the active keys of dS[q][key] K[key][d].
      const int last_q = min(q0 + 31, L - 1);
      const int n_active = min(kWavesK, (last_q - k_wg0) / 32 + 1);
      for (int db = wave; db < ND; db += kWavesK) {
        f32x16 acc = zero_f32x16();
        for (int u = 0; u < 2 * n_active; ++u) {
          // A = dS (rows = queries, k = keys 16u + 8hi + s) from dS^T.
          const int kr = 16 * u + 8 * hi + (j16 >> 2);
          const int qc = 16 * (grp & 1) + 4 * (j16 & 3);
          const f16x8 a = cat4(lds_read_tr(dSs + kr * kDSP + qc), lds_read_tr(dSs + (kr + 4) * kDSP + qc));
          // B = K (k = keys, cols = head dim) from the K tile.
          const int dc = 32 * db + 16 * (grp & 1) + 4 * (j16 & 3);
          const f16x8 bk = cat4(lds_read_tr(Ks + kr * KP + dc), lds_read_tr(Ks + (kr + 4) * KP + dc));
          acc = mfma32x32x16(a, bk, acc);
        }
        // acc element i: query row 8(i/4) + 4hi + i%4, head-dim column
        // 32db + l32.
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qr = q0 + 8 * (i >> 2) + 4 * hi + (i & 3);
          if (qr < L)
            unsafeAtomicAdd(p.dq_acc + ((size_t)(s0 + qr) * p.h_q + head) * D + 32 * db + l32, acc[i]);
        }
      }
    }
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

// dq = fp16(scale * dQ_acc), 8 elements per thread.
__global__ __launch_bounds__(256) void bwd_convert_kernel(const float* __restrict__ acc,
                                                          f16* __restrict__ dq, size_t n8,
                                                          float scale) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *(const f32x4*)(acc + 8 * i);
  const f32x4 b = *(const f32x4*)(acc + 8 * i + 4);
  f16x8 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w[e] = (f16)(a[e] * scale);
    w[4 + e] = (f16)(b[e] * scale);
  }
  *(f16x8*)(dq + 8 * i) = w;
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
  p.dq_acc = a.dq_acc;
  p.drow = a.drow;
  p.dq = (f16*)a.dq;
  p.dk = (f16*)a.dk;
  p.dv = (f16*)a.dv;
  p.n_seqs = a.n_seqs;
  p.T = a.total_tokens;
  p.h_q = a.h_q;
  p.h_kv = a.h_kv;
  p.G = a.h_q / a.h_kv;
  p.n_ktiles = (a.max_seqlen + kBK - 1) / kBK;
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  const int D = a.head_dim;
  const int rows = a.total_tokens * a.h_q;
  const int rows_per_block = 256 / (D / 8);
  const dim3 gprep((rows + rows_per_block - 1) / rows_per_block);
  const dim3 gmain(p.n_ktiles * a.n_seqs * a.h_kv);
  const size_t n8 = (size_t)rows * D / 8;
  const dim3 gconv((unsigned)((n8 + 255) / 256));
  if (D == 128) {
    hipLaunchKernelGGL(bwd_prep_kernel<128>, gprep, dim3(256), 0, stream, p);
    hipLaunchKernelGGL(bwd_main_kernel<128>, gmain, dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(bwd_prep_kernel<64>, gprep, dim3(256), 0, stream, p);
    hipLaunchKernelGGL(bwd_main_kernel<64>, gmain, dim3(256), 0, stream, p);
  }
  hipLaunchKernelGGL(bwd_convert_kernel, gconv, dim3(256), 0, stream, (const float*)p.dq_acc,
                     p.dq, n8, p.scale);
  return hipGetLastError();
}

}  // namespace cgqa
