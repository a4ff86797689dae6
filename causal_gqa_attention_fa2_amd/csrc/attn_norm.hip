// attn_norm.hip -- RMSNorm forward and backward for gfx950, the layer
// operation next to attention in the Qwen3 stack of the RL.cu pages
// (pitchhut "Project Highlights"; mlllm.io "What happened").
//
//   r = 1 / sqrt(mean_j x_j^2 + eps),   y_j = x_j r w_j
//   dx_j = r (w_j dy_j - x_hat_j mean_k(w_k dy_k x_hat_k)),  x_hat = x r
//   dw_j = sum over rows of dy_j x_hat_j
//
// Both passes are bound by HBM: every row is read once (x, and dy in the
// backward) and written once, in 16-byte pieces. A group of LPR lanes (LPR =
// the largest power of two <= min(64, n / 8)) owns one row; lane i of the
// group holds pieces i, i + LPR, ... of the row in registers, so the row's
// sums are an in-register sum plus a butterfly over the group. Sums are fp32.
// dw is deterministic: each backward work-group adds its rows' terms in a
// fixed order into a partial row of the workspace, and a second kernel adds
// the partial rows in work-group order.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace cgqa {
namespace {

typedef _Float16 h16;
typedef h16 h16x8 __attribute__((ext_vector_type(8)));

constexpr int kNormThreads = 256;
constexpr int kNormBwdThreads = 1024;  // 16 waves: four per SIMD keep more rows in flight

// Pieces a lane may hold: a row of n / 8 pieces uses LPR = 64 lanes when it
// has at least 64 pieces (then at most kNormMaxCols / 512 per lane), else the
// largest power of two LPR <= n / 8, which leaves fewer than 2 LPR pieces.
template <int LPR>
constexpr int pieces_per_lane() {
  return LPR == 64 ? kNormMaxCols / 512 : 2;
}

struct NormParams {
  const h16x8* __restrict__ x;
  const h16x8* __restrict__ w;
  const h16x8* __restrict__ dy;
  const float* __restrict__ rstd_in;
  h16x8* __restrict__ y;  // y (forward) or dx (backward)
  float* __restrict__ rstd_out;
  float* __restrict__ part;  // backward: [n_wgs, n] fp32 partial dw rows
  float* __restrict__ dw;
  int rows, pieces;  // pieces = n / 8
  float eps, inv_n;
};

// Butterfly sum over the LPR lanes of a group (LPR a power of two <= 64).
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <int LPR>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_fwd_kernel(NormParams p) {
  constexpr int RPW = 64 / LPR;  // rows per wave
  constexpr int PPL = pieces_per_lane<LPR>();
  const int lane = threadIdx.x & 63;
  const int gl = lane % LPR;
  const int row = (blockIdx.x * (kNormThreads / 64) + threadIdx.x / 64) * RPW + lane / LPR;
  if (row >= p.rows) return;  // whole groups leave together; no cross-group exchange follows
  const h16x8* xr = p.x + (size_t)row * p.pieces;
  // w goes out with x, so its latency hides under the row's.
  h16x8 xv[PPL], wv[PPL];
#pragma unroll
  for (int k = 0; k < PPL; ++k) {
    const int c = gl + k * LPR;
    if (c < p.pieces) {
      xv[k] = xr[c];
      wv[k] = p.w[c];
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < PPL; ++k) {
    const int c = gl + k * LPR;
    if (c < p.pieces) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += (float)xv[k][e] * (float)xv[k][e];
    }
  }
  ss = group_sum<LPR>(ss);
  const float r = 1.f / sqrtf(ss * p.inv_n + p.eps);
  h16x8* yr = p.y + (size_t)row * p.pieces;
#pragma unroll
  for (int k = 0; k < PPL; ++k) {
    const int c = gl + k * LPR;
    if (c < p.pieces) {
      h16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (h16)((float)xv[k][e] * r * (float)wv[k][e]);
      yr[c] = o;
    }
  }
  if (gl == 0) p.rstd_out[row] = r;
}

// Backward, one pass over the rows with 1024-thread work-groups (GPW row
// groups, four waves per SIMD): dx per row, and this work-group's share of
// dw. Row group grp of work-group g takes rows g GPW + grp + i n_wgs GPW
// (grid stride); for rows of 512 to 1024 values, the loads of a group's next
// row go out before the current row's arithmetic, so two rows' latencies
// overlap. Every lane keeps fp32 dw
// sums for its pieces, then the work-group adds its groups' sums through LDS
// in group order and writes one partial row.
template <int LPR, int PPL>
__global__ __launch_bounds__(kNormBwdThreads) void rmsnorm_bwd_kernel(NormParams p) {
  constexpr int GPW = kNormBwdThreads / LPR;  // row groups per work-group
  // One row of dw terms per group: GPW * n floats, at most 16 * 2048 (LPR =
  // 64 serves n >= 512) or GPW * 16 LPR (below that n < 16 LPR) = 64 KiB.
  constexpr int kRed = LPR == 64 ? 16 * kNormMaxCols : GPW * 16 * LPR;
  __shared__ float red[kRed];
  const int lane = threadIdx.x & 63;
  const int gl = lane % LPR;
  const int grp = threadIdx.x / LPR;  // 0 .. GPW - 1
  float acc[PPL][8];
#pragma unroll
  for (int k = 0; k < PPL; ++k) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
  }
  const int stride = gridDim.x * GPW;
  // dx of one row from its x, dy, w pieces and r; adds the row's dw terms.
  auto row_grads = [&](int row, const h16x8(&xv)[PPL], const h16x8(&gv)[PPL],
                       const h16x8(&wv)[PPL], float r) __attribute__((always_inline)) {
    float dot = 0.f;
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      const int c = gl + k * LPR;
      if (c < p.pieces) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          dot += (float)gv[k][e] * (float)wv[k][e] * ((float)xv[k][e] * r);
      }
    }
    const float proj = group_sum<LPR>(dot) * p.inv_n;
    h16x8* dxr = p.y + (size_t)row * p.pieces;
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      const int c = gl + k * LPR;
      if (c < p.pieces) {
        h16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xh = (float)xv[k][e] * r;
          const float g = (float)gv[k][e];
          o[e] = (h16)(r * (g * (float)wv[k][e] - xh * proj));
          acc[k][e] += g * xh;
        }
        dxr[c] = o;
      }
    }
  };
  auto load_row = [&](int row, h16x8(&xs)[PPL], h16x8(&gs)[PPL], float& rs)
                      __attribute__((always_inline)) {
    const h16x8* xr = p.x + (size_t)row * p.pieces;
    const h16x8* gr = p.dy + (size_t)row * p.pieces;
    rs = p.rstd_in[row];
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      const int c = gl + k * LPR;
      if (c < p.pieces) {
        xs[k] = xr[c];
        gs[k] = gr[c];
      }
    }
  };
  int row = blockIdx.x * GPW + grp;
  if constexpr (LPR == 64 && PPL == 2) {
    // Rows of 512 to 1024 values: w stays in registers, and the loads of a
    // group's next row go out before the current row's arithmetic.
    h16x8 wv[PPL];
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      const int c = gl + k * LPR;
      if (c < p.pieces) wv[k] = p.w[c];
    }
    h16x8 xv[PPL], gv[PPL];
    float r = 0.f;
    if (row < p.rows) load_row(row, xv, gv, r);
    for (; row < p.rows; row += stride) {
      h16x8 xn[PPL], gn[PPL];
      float rn = 0.f;
      if (row + stride < p.rows) load_row(row + stride, xn, gn, rn);
      row_grads(row, xv, gv, wv, r);
#pragma unroll
      for (int k = 0; k < PPL; ++k) {
        xv[k] = xn[k];
        gv[k] = gn[k];
      }
      r = rn;
    }
  } else {
    // Rows are loaded in turn, with the arithmetic written out here (through
    // row_grads it spills at four pieces per lane). Four pieces per lane
    // (n > 1024) leave no registers for a second row; for narrow rows (LPR <
    // 64, several rows per wave) loading ahead measured slower.
    for (; row < p.rows; row += stride) {
      const h16x8* xr = p.x + (size_t)row * p.pieces;
      const h16x8* gr = p.dy + (size_t)row * p.pieces;
      const float r = p.rstd_in[row];
      h16x8 xv[PPL], gv[PPL], wv[PPL];
      float dot = 0.f;
#pragma unroll
      for (int k = 0; k < PPL; ++k) {
        const int c = gl + k * LPR;
        if (c < p.pieces) {
          xv[k] = xr[c];
          gv[k] = gr[c];
          wv[k] = p.w[c];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            dot += (float)gv[k][e] * (float)wv[k][e] * ((float)xv[k][e] * r);
        }
      }
      const float proj = group_sum<LPR>(dot) * p.inv_n;
      h16x8* dxr = p.y + (size_t)row * p.pieces;
#pragma unroll
      for (int k = 0; k < PPL; ++k) {
        const int c = gl + k * LPR;
        if (c < p.pieces) {
          h16x8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float xh = (float)xv[k][e] * r;
            const float g = (float)gv[k][e];
            o[e] = (h16)(r * (g * (float)wv[k][e] - xh * proj));
            acc[k][e] += g * xh;
          }
          dxr[c] = o;
        }
      }
    }
  }
  // Sum the GPW groups' dw terms in group order: every group stores its row
  // of terms in LDS, then each column is added up over the groups in order
  // (the same sequence of fp32 additions as adding the groups one by one,
  // with two barriers instead of one per group).
  const int n = p.pieces * 8;
#pragma unroll
  for (int k = 0; k < PPL; ++k) {
    const int c = gl + k * LPR;
    if (c < p.pieces) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red[grp * n + c * 8 + e] = acc[k][e];
    }
  }
  __syncthreads();
  float* prow = p.part + (size_t)blockIdx.x * n;
  for (int j = threadIdx.x; j < n; j += kNormBwdThreads) {
    float t = 0.f;
    for (int g = 0; g < GPW; ++g) t += red[g * n + j];
    prow[j] = t;
  }
}

// dw_j = sum of the partial rows. A work-group owns 64 columns; its 16
// waves sum the partial rows g = wave, wave + 16, ... (independent loads, all
// in flight at once for up to 256 rows), then wave 0 adds the 16 wave sums in
// wave order, so the result does not depend on timing.
constexpr int kNormDwThreads = 1024;
__global__ __launch_bounds__(kNormDwThreads) void rmsnorm_dw_kernel(const float* __restrict__ part,
                                                                    float* __restrict__ dw,
                                                                    int n, int n_rows) {
  constexpr int kWaves = kNormDwThreads / 64;
  __shared__ float sums[kNormDwThreads];
  const int wave = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + (threadIdx.x & 63);
  float s = 0.f;
  if (j < n) {
#pragma unroll 16
    for (int g = wave; g < n_rows; g += kWaves) s += part[(size_t)g * n + j];
  }
  sums[threadIdx.x] = s;
  __syncthreads();
  if (wave == 0 && j < n) {
    float t = sums[threadIdx.x];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t += sums[threadIdx.x + 64 * w];
    dw[j] = t;
  }
}

int lanes_per_row(int n) {
  const int pieces = n / 8;
  int lpr = 8;
  while (lpr * 2 <= pieces && lpr * 2 <= 64) lpr *= 2;
  return lpr;
}

template <int LPR>
hipError_t launch_fwd_lpr(const NormParams& p, hipStream_t stream) {
  const int rows_per_wg = (kNormThreads / 64) * (64 / LPR);
  const dim3 grid((p.rows + rows_per_wg - 1) / rows_per_wg);
  hipLaunchKernelGGL(rmsnorm_fwd_kernel<LPR>, grid, dim3(kNormThreads), 0, stream, p);
  return hipGetLastError();
}

template <int LPR>
hipError_t launch_bwd_lpr(const NormParams& p, int n_wgs, hipStream_t stream) {
  // A lane holds at most ceil(pieces / LPR) pieces: two below LPR = 64 (see
  // pieces_per_lane), and with LPR = 64 two up to n = 1024, four above.
  if (LPR < 64 || p.pieces <= 2 * LPR)
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<LPR, 2>), dim3(n_wgs), dim3(kNormBwdThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<LPR, pieces_per_lane<LPR>()>), dim3(n_wgs),
                       dim3(kNormBwdThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int rmsnorm_bwd_num_wgs(int rows, int n) {
  const int groups = kNormBwdThreads / lanes_per_row(n);
  const int need = (rows + groups - 1) / groups;
  return need < 1 ? 1 : (need < kNormMaxWGs ? need : kNormMaxWGs);
}

hipError_t launch_rmsnorm_fwd(const NormArgs& a, hipStream_t stream) {
  NormParams p{};
  p.x = (const h16x8*)a.x;
  p.w = (const h16x8*)a.w;
  p.y = (h16x8*)a.y;
  p.rstd_out = a.rstd;
  p.rows = a.rows;
  p.pieces = a.n / 8;
  p.eps = a.eps;
  p.inv_n = 1.f / (float)a.n;
  switch (lanes_per_row(a.n)) {
    case 8: return launch_fwd_lpr<8>(p, stream);
    case 16: return launch_fwd_lpr<16>(p, stream);
    case 32: return launch_fwd_lpr<32>(p, stream);
    default: return launch_fwd_lpr<64>(p, stream);
  }
}

hipError_t launch_rmsnorm_bwd(const NormArgs& a, hipStream_t stream) {
  NormParams p{};
  p.x = (const h16x8*)a.x;
  p.w = (const h16x8*)a.w;
  p.dy = (const h16x8*)a.dy;
  p.rstd_in = a.rstd;
  p.y = (h16x8*)a.dx;
  p.part = a.part;
  p.dw = a.dw;
  p.rows = a.rows;
  p.pieces = a.n / 8;
  p.eps = a.eps;
  p.inv_n = 1.f / (float)a.n;
  const int n_wgs = rmsnorm_bwd_num_wgs(a.rows, a.n);
  hipError_t e;
  switch (lanes_per_row(a.n)) {
    case 8: e = launch_bwd_lpr<8>(p, n_wgs, stream); break;
    case 16: e = launch_bwd_lpr<16>(p, n_wgs, stream); break;
    case 32: e = launch_bwd_lpr<32>(p, n_wgs, stream); break;
    default: e = launch_bwd_lpr<64>(p, n_wgs, stream); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rmsnorm_dw_kernel, dim3((a.n + 63) / 64), dim3(kNormDwThreads), 0, stream,
                     (const float*)a.part, a.dw, a.n, n_wgs);
  return hipGetLastError();
}

}  // namespace cgqa
