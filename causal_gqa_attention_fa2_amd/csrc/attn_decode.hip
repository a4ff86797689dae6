// attn_decode.hip -- single-token decode attention over a paged KV cache for
// gfx950 (the rollout engine's paged key-value caching; pitchhut "Key
// Features" item 2, mlllm.io "What happened").
//
// Every sequence has one query token per head; its context lives in 16-token
// blocks of a shared pool, addressed through the sequence's block table. The
// work is a gather-and-reduce that reads every context key and value once,
// so it is bound by HBM bandwidth; it runs on the vector ALUs, not on MFMA.
//
// Balanced split-context scheme (three launches):
//   1. plan:    one work-group prefix-sums the block counts ceil(ctx/16) of
//               the sequences (wave shuffle scans) and records, for each
//               gather work-group, the sequence its range starts in.
//   2. gather:  the flattened (sequence, block) space is cut into n_wgs equal
//               contiguous ranges, one per work-group, whatever the mix of
//               context lengths (ranges may span several sequences). A
//               work-group has one wave per KV head (up to 8); its waves walk
//               the same blocks together, so the KV heads of each token row
//               (one contiguous run of h_kv * d halves) are fetched at the
//               same time. In a wave each token row of a block is held by D/8
//               lanes with 16 bytes each; one load instruction gathers
//               64 / (D/8) rows and two blocks are in flight per wave. The G
//               query heads of the KV head share every loaded block. q.k and
//               the P.V sums use v_dot2_f32_f16 (fp16 products, fp32 sums);
//               row sums of q.k use DPP lane moves. Each lane keeps an
//               online-softmax state (max, sum, 8 output columns) per query
//               head; at the end of each sequence segment the lanes' states
//               are merged and stored as a partial in slot (work-group +
//               sequence), which is unique because the ranges are ordered.
//   3. combine: per (sequence, query head), merge the partials of the
//               work-groups that covered the sequence and write fp16 output.
#include "cdna4.h"
#include "kernels.h"

#include <mutex>

namespace cgqa {
namespace {

constexpr int kMaxG = 16;
constexpr int kDecodeWaves = 8;  // KV heads (waves) per gather work-group
constexpr int kPlanThreads = 256;

struct DecParams {
  const f16* __restrict__ q;
  const f16* __restrict__ kp;
  const f16* __restrict__ vp;
  const int32_t* __restrict__ bt;
  const int32_t* __restrict__ ctx;
  f16* __restrict__ o;
  float* __restrict__ part_o;
  float* __restrict__ part_ml;
  int32_t* __restrict__ blk_start;  // [n + 1]
  int32_t* __restrict__ wg_first;   // [n_wgs]
  int n, h_q, h_kv, G, max_blocks, n_wgs;
  // Pool size and the largest context the table rows can address: every
  // context length is clamped into [0, max_ctx] and every table entry into
  // [0, num_blocks), so no access leaves the pools or the table rows.
  int num_blocks, max_ctx;
  float scale_log2;
  // RoPE tables [max_pos, D / 2] to rotate each query by its position
  // ctx - 1 as it is loaded, or null.
  const float* __restrict__ cos_t;
  const float* __restrict__ sin_t;
  int max_pos;
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

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Context length of sequence b as every kernel of the decode uses it: the
// caller's value clamped into [0, max_ctx] (max_ctx <= 16 * max_blocks, so
// ceil(ctx / 16) table entries of the row exist). The plan, the gather and
// the combine all see the same value, so the block ranges agree.
__device__ __forceinline__ int ctx_of(const DecParams& p, int b) {
  return min(max(p.ctx[b], 0), p.max_ctx);
}

// Two fp16 values (lo from a, hi from b) taken from the same half of two words.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float fdot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                false);
}

// Exclusive prefix sum of the sequences' block counts into blk_start[0..n]
// and, for every gather work-group whose range starts in sequence b,
// wg_first[w] = b. One work-group of kPlanThreads threads: chunks of
// kPlanThreads sequences, wave scans by lane shuffles, one LDS exchange of the
// wave totals per chunk.
__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(DecParams p) {
  constexpr int NW = kPlanThreads / 64;
  __shared__ int wsum[NW];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int carry = 0;
  for (int base = 0; base < p.n; base += kPlanThreads) {
    const int b = base + tid;
    const int nb = b < p.n ? ceil_div(ctx_of(p, b), 16) : 0;
    int x = nb;  // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = carry, chunk_total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      before += w < wave ? wsum[w] : 0;
      chunk_total += wsum[w];
    }
    if (b < p.n) p.blk_start[b] = before + x - nb;
    carry += chunk_total;
    __syncthreads();  // wsum is rewritten by the next chunk
  }
  if (tid == 0) p.blk_start[p.n] = carry;
  const int total = carry;
  const int chunk = max(1, ceil_div(total, p.n_wgs));
  // Second pass (this thread's own sequences, so its own writes): the
  // work-groups whose range starts inside sequence b.
  for (int b = tid; b < p.n; b += kPlanThreads) {
    const int start = p.blk_start[b];
    const int nb = ceil_div(ctx_of(p, b), 16);
    for (int w = ceil_div(start, chunk); w * chunk < start + nb; ++w) p.wg_first[w] = b;
  }
}

// One wave: online softmax of the G query heads of KV head g of sequence b
// over its logical blocks [j0, j1); the merged state goes to partial slot
// `slot`.
template <int D, int G>
__device__ __forceinline__ void gather_segment(const DecParams& p, int b, int g, int j0, int j1,
                                               int slot, int lane) {
  constexpr int LPR = D / 8;      // lanes per token row
  constexpr int TPI = 64 / LPR;   // token rows per load instruction
  constexpr int NLD = 16 / TPI;   // load instructions per 16-token block
  constexpr int NB = 2;           // blocks in flight per wave
  constexpr int NTOK = NB * NLD;  // tokens per lane per iteration
  const int rg = lane / LPR;      // token row within a load instruction
  const int dc = lane % LPR;      // 8-column chunk of the head dimension
  const int t_end = ctx_of(p, b);

  u32x4 qh[G];  // q chunk of each head as fp16 pairs
#pragma unroll
  for (int h = 0; h < G; ++h)
    qh[h] = *(const u32x4*)(p.q + ((size_t)b * p.h_q + g * G + h) * D + dc * 8);
  if (p.cos_t != nullptr) {
    // RoPE of the query at position ctx - 1: chunk dc pairs with chunk
    // dc ^ (LPR / 2) (dimensions D/2 apart), which lane ^ (LPR / 2) holds.
    // Both lanes rotate the pair (rope_pair, exact) and keep their half.
    const int pos = min(max(t_end - 1, 0), p.max_pos - 1);
    const bool low = dc < LPR / 2;
    const int j0c = 8 * (dc % (LPR / 2));
    const float* ct = p.cos_t + (size_t)pos * (D / 2) + j0c;
    const float* st = p.sin_t + (size_t)pos * (D / 2) + j0c;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      u32x4 other;
#pragma unroll
      for (int e = 0; e < 4; ++e) other[e] = (uint32_t)__shfl_xor((int)qh[h][e], LPR / 2, 64);
      const f16x8 mine = __builtin_bit_cast(f16x8, qh[h]);
      const f16x8 part = __builtin_bit_cast(f16x8, other);
      f16x8 lo = low ? mine : part, hi = low ? part : mine;
      rope_rotate8(lo, hi, ct, st, 1.f);
      qh[h] = __builtin_bit_cast(u32x4, low ? lo : hi);
    }
  }
  SoftState st[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st[h].m = kMaxInit;
    st[h].l = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st[h].a[e] = 0.f;
  }

  const size_t row_stride = (size_t)p.h_kv * D;  // halves between token rows
  const f16* kbase = p.kp + (size_t)g * D + dc * 8;
  const f16* vbase = p.vp + (size_t)g * D + dc * 8;
  const int32_t* table = p.bt + (size_t)b * p.max_blocks;
  for (int win = j0; win < j1; win += 64) {
    // Table entries of the next (up to) 64 blocks, one per lane.
    const int cnt = min(64, j1 - win);
    int my_phys = 0;
    // win + lane < j1 <= ceil(t_end / 16) <= max_blocks: inside the row.
    if (lane < cnt) my_phys = min(max(table[win + lane], 0), p.num_blocks - 1);
    for (int i0 = 0; i0 < cnt; i0 += NB) {
      // Loads are unconditional (a guarded load lets the compiler reuse its
      // destination register and wait on it before issuing the next one):
      // rows past the context read the block's unused slots and are masked
      // below; a missing second block re-reads the first.
      u32x4 kr[NTOK], vr[NTOK];
      bool ok[NTOK];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const int i = i0 + bb;
        const int phys = __builtin_amdgcn_readlane(my_phys, i < cnt ? i : i0);
        const size_t base = (size_t)phys * 16 * row_stride;
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
          const int tok = j * TPI + rg;
          const int t = bb * NLD + j;
          ok[t] = i < cnt && (win + i) * 16 + tok < t_end;
          // Non-temporal: every pool row is read exactly once per call, so
          // it should not displace anything in the caches (measured ~10%
          // faster on gfx950 for a pool larger than the last-level cache).
          kr[t] = __builtin_nontemporal_load((const u32x4*)(kbase + base + (size_t)tok * row_stride));
          vr[t] = __builtin_nontemporal_load((const u32x4*)(vbase + base + (size_t)tok * row_stride));
        }
      }
      // Keep every load of the iteration ahead of the arithmetic that uses it.
      __builtin_amdgcn_sched_barrier(0);
      // Masked rows may hold anything (even NaN): zero their values.
#pragma unroll
      for (int t = 0; t < NTOK; ++t) {
#pragma unroll
        for (int c = 0; c < 4; ++c) vr[t][c] = ok[t] ? vr[t][c] : 0u;
      }
      // Values of token pairs (2u, 2u+1) interleaved per column for v_dot2.
      u32x4 vlo[NTOK / 2], vhi[NTOK / 2];
#pragma unroll
      for (int u = 0; u < NTOK / 2; ++u) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          vlo[u][c] = pair_lo(vr[2 * u][c], vr[2 * u + 1][c]);
          vhi[u][c] = pair_hi(vr[2 * u][c], vr[2 * u + 1][c]);
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s[NTOK];
        float mx = kMaxInit;
#pragma unroll
        for (int t = 0; t < NTOK; ++t) {
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < 4; ++c) acc = fdot2(kr[t][c], qh[h][c], acc);
          acc = group_sum<LPR>(acc) * p.scale_log2;
          s[t] = ok[t] ? acc : -INFINITY;
          mx = fmaxf(mx, s[t]);
        }
        const float m_new = fmaxf(st[h].m, mx);
        const float alpha = fast_exp2(st[h].m - m_new);
        st[h].m = m_new;
        float lsum = 0.f;
        uint32_t pp[NTOK / 2];
#pragma unroll
        for (int u = 0; u < NTOK / 2; ++u) {
          const f16 p0 = (f16)fast_exp2(s[2 * u] - m_new);
          const f16 p1 = (f16)fast_exp2(s[2 * u + 1] - m_new);
          lsum += (float)p0 + (float)p1;
          pp[u] = __builtin_bit_cast(uint32_t, f16x2{p0, p1});
        }
        st[h].l = st[h].l * alpha + lsum;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float a0 = st[h].a[2 * c] * alpha;
          float a1 = st[h].a[2 * c + 1] * alpha;
#pragma unroll
          for (int u = 0; u < NTOK / 2; ++u) {
            a0 = fdot2(vlo[u][c], pp[u], a0);
            a1 = fdot2(vhi[u][c], pp[u], a1);
          }
          st[h].a[2 * c] = a0;
          st[h].a[2 * c + 1] = a1;
        }
      }
    }
  }

  // Merge the TPI token rows of the wave (lanes dc, dc + LPR, ...) and store
  // the partial from the lanes of row group 0.
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
      const size_t row = (size_t)slot * p.h_q + g * G + h;
      float* po = p.part_o + row * D + dc * 8;
      *(f32x4*)po = f32x4{st[h].a[0], st[h].a[1], st[h].a[2], st[h].a[3]};
      *(f32x4*)(po + 4) = f32x4{st[h].a[4], st[h].a[5], st[h].a[6], st[h].a[7]};
      if (dc == 0) {
        p.part_ml[2 * row] = st[h].m;
        p.part_ml[2 * row + 1] = st[h].l;
      }
    }
  }
}

template <int D, int G>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_gather_kernel(DecParams p) {
  const int w = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.y * kDecodeWaves + wave;  // KV head of this wave
  const int total = p.blk_start[p.n];
  const int chunk = max(1, ceil_div(total, p.n_wgs));
  int c = w * chunk;
  const int c_end = min(total, c + chunk);
  if (c >= c_end || g >= p.h_kv) return;  // no barrier follows: waves may leave
  int b = p.wg_first[w];
  while (c < c_end) {
    const int sb = p.blk_start[b];
    const int seg_end = min(c_end, p.blk_start[b + 1]);
    if (seg_end > c) gather_segment<D, G>(p, b, g, c - sb, seg_end - sb, w + b, lane);
    c = max(c, seg_end);
    ++b;
  }
}

// One wave per (sequence, query head): merge the partials of the work-groups
// that covered the sequence, normalise, store fp16. Partials are read in
// batches of kBatch with every load of a batch issued before any use, so a
// sequence costs one memory round trip per batch (usually one).
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecParams p) {
  constexpr int PER = D / 64;  // output columns per lane
  constexpr int kBatch = 4;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= p.n * p.h_q) return;
  const int b = row / p.h_q;
  const int head = row - b * p.h_q;
  f16* out = p.o + (size_t)row * D + lane * PER;
  const int sb = p.blk_start[b];
  const int eb = p.blk_start[b + 1];
  if (eb == sb) {  // empty context
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = (f16)0.f;
    return;
  }
  const int chunk = max(1, ceil_div(p.blk_start[p.n], p.n_wgs));
  const int w0 = sb / chunk;
  const int w1 = (eb - 1) / chunk;
  float M = kMaxInit, l = 0.f, acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int wb = w0; wb <= w1; wb += kBatch) {
    float m2[kBatch], l2[kBatch], o2[kBatch][PER];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      // Slots past w1 re-read slot w1 (in bounds) and are dropped below.
      const size_t srow = (size_t)(min(wb + i, w1) + b) * p.h_q + head;
      m2[i] = p.part_ml[2 * srow];
      l2[i] = p.part_ml[2 * srow + 1];
      const float* po = p.part_o + srow * D + lane * PER;
#pragma unroll
      for (int e = 0; e < PER; ++e) o2[i][e] = po[e];
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (wb + i <= w1) Mb = fmaxf(Mb, m2[i]);
    const float cs = fast_exp2(M - Mb);
    l *= cs;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] *= cs;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const float c = wb + i <= w1 ? fast_exp2(m2[i] - Mb) : 0.f;
      l += l2[i] * c;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += o2[i][e] * c;
    }
    M = Mb;
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[e] = (f16)(acc[e] * inv);
}

template <int D>
hipError_t launch_d(const DecParams& p, int G, hipStream_t stream) {
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  const int waves = p.h_kv < kDecodeWaves ? p.h_kv : kDecodeWaves;
  const dim3 grid(p.n_wgs, (p.h_kv + kDecodeWaves - 1) / kDecodeWaves);
  const dim3 block(64 * waves);
  switch (G) {
#define CGQA_G(GG) \
  case GG: hipLaunchKernelGGL((decode_gather_kernel<D, GG>), grid, block, 0, stream, p); break;
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
}  // namespace cgqa

// Device array that stands in for the workspace of the allocation-free
// decode. Host code never uses this name as an address: the runtime gives
// each device's copy its own device address (decode_scratch below).
static __device__ __align__(256) unsigned char scratch[cgqa::kDecodeScratchBytes];

namespace cgqa {

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

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
  p.blk_start = a.plan;
  p.wg_first = a.plan + a.n_seqs + 1;
  p.n = a.n_seqs;
  p.h_q = a.h_q;
  p.h_kv = a.h_kv;
  p.G = a.h_q / a.h_kv;
  p.max_blocks = a.max_blocks_per_seq;
  p.n_wgs = a.n_wgs;
  p.num_blocks = a.num_blocks;
  p.max_ctx = a.max_ctx_len;
  p.scale_log2 = a.scale * kLog2e;
  p.cos_t = a.rope_cos;
  p.sin_t = a.rope_sin;
  p.max_pos = a.rope_max_pos;
  if (p.G > kMaxG) return hipErrorInvalidValue;
  return a.head_dim == 128 ? launch_d<128>(p, p.G, stream) : launch_d<64>(p, p.G, stream);
}

}  // namespace cgqa
