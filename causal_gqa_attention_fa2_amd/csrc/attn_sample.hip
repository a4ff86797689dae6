// attn_sample.hip -- temperature / top-k / top-p sampling over logits for
// gfx950, the rollout engine's step after the decode and the LM head
// (pitchhut "Key Features", item 1).
//
// One work-group of 1024 threads per row:
//  1. radix select (11 + 11 + 10 bits of an order-preserving key of the fp32
//     logit, one LDS histogram per pass) finds K*, the k-th largest key. A
//     first read of the row bounds the first digit from below through the
//     threads' maxima; a second copies the keys from that digit up to LDS
//     (when they fit), and all three digits are selected on that copy, so
//     the row is read twice and no pass adds every key into one histogram;
//  2. the keys above K* are gathered (with the keys equal to K* when all of
//     them are kept, the usual case; otherwise the lowest-index keys equal
//     to K* follow, in tiles of 1024 in index order with ranks from wave
//     ballots), so the kept set is the first k of the ranking "logit
//     descending, index ascending"; the row is streamed with 16-byte loads;
//  3. a bitonic sort in LDS puts the k candidates in ranking order;
//  4. weights w_j = exp((v_j - v_0) / T); the cumulative sums c_j in
//     ranking order (a wave scan for k <= 64, else one thread), ranks
//     0..cut kept with cut = min{j : c_j >= top_p c_last}, and the token at
//     rank min{j <= cut : c_j > u c_cut} for the row's uniform u.
// Scaling by 1/T > 0 keeps the order, so the selection runs on raw logits.
// The result is a deterministic function of the logits and u.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace cgqa {
namespace {

constexpr int kSampleThreads = 1024;
constexpr int kWaves = kSampleThreads / 64;
constexpr int kCandidates = 4096;  // LDS copy of the keys past the first radix digit
constexpr int kHead = 16384;       // least number of logits behind the first bound

struct SampleParams {
  const float* __restrict__ logits;
  const float* __restrict__ u;
  int32_t* __restrict__ tokens;
  int vocab, k;
  float inv_t, top_p;
};

// Larger float -> larger key (sign flipped for positives, all bits for
// negatives); -inf maps below every finite value.
__device__ __forceinline__ uint32_t fkey(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Ranking order: a before b when its logit is larger, or equal with a
// smaller index.
__device__ __forceinline__ bool before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Calls fn(value, index) for every logit of the row: 16-byte loads, four in
// flight per thread, when the row is 16-byte aligned; the rest one by one.
template <typename F>
__device__ __forceinline__ void for_each_logit(const float* row, int V, int tid, F&& fn) {
  int done = 0;
  if (((uintptr_t)row & 15u) == 0) {
    const int v4 = V >> 2;
    const float4* r4 = (const float4*)row;
    constexpr int kU = 4;
    for (int i0 = tid; i0 < v4; i0 += kU * kSampleThreads) {
      float4 x[kU];
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const int i = i0 + k * kSampleThreads;
        if (i < v4) x[k] = r4[i];
      }
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const int i = i0 + k * kSampleThreads;
        if (i < v4) {
          fn(x[k].x, 4 * i);
          fn(x[k].y, 4 * i + 1);
          fn(x[k].z, 4 * i + 2);
          fn(x[k].w, 4 * i + 3);
        }
      }
    }
    done = v4 << 2;
  }
  for (int i = done + tid; i < V; i += kSampleThreads) fn(row[i], i);
}

__device__ __forceinline__ float key_to_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

__global__ __launch_bounds__(kSampleThreads) void sample_kernel(SampleParams p) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t suf[kSampleThreads];
  __shared__ float cval[kMaxTopK];
  __shared__ int cidx[kMaxTopK];
  __shared__ float cum[kMaxTopK];
  __shared__ uint32_t bkey[kCandidates];  // keys whose top digit reaches the k-th's
  __shared__ int bidx[kCandidates];
  __shared__ uint32_t s_digit, s_above, s_eq, s_count, s_taken, s_nb, s_wave[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int V = p.vocab;
  const float* row = p.logits + (size_t)blockIdx.x * V;

  // Digit of the histogram where the count of larger digits first reaches
  // `need`: suffix sums over digit pairs (2t, 2t + 1), then the pair's digit.
  // Sets s_digit, s_above (keys with larger digits) and s_eq (keys with
  // this digit).
  auto find_digit = [&](uint32_t need) {
    // Suffix sums over the pairs: within each wave by lane shuffles, then
    // the totals of the waves above.
    uint32_t v = hist[2 * tid] + hist[2 * tid + 1];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_down(v, off, 64);
      if (lane + off < 64) v += o;
    }
    if (lane == 0) s_wave[wave] = v;
    __syncthreads();
    for (int w = wave + 1; w < kWaves; ++w) v += s_wave[w];
    suf[tid] = v;
    __syncthreads();
    const uint32_t above_pair = tid + 1 < kSampleThreads ? suf[tid + 1] : 0u;
    if (suf[tid] >= need && above_pair < need) {
      const uint32_t h1 = hist[2 * tid + 1];
      if (above_pair + h1 >= need) {
        s_digit = 2 * tid + 1;
        s_above = above_pair;
        s_eq = h1;
      } else {
        s_digit = 2 * tid;
        s_above = above_pair + h1;
        s_eq = hist[2 * tid];
      }
    }
    __syncthreads();
  };
  auto clear_hist = [&]() {
    hist[2 * tid] = 0;
    hist[2 * tid + 1] = 0;
    __syncthreads();
  };

  // 1. Radix select of the k-th largest key: digits of 11, 11 and 10 bits
  // from the top; `need` is the rank of K* among the keys matching the
  // digits chosen so far. The first digit streams the row; when the keys
  // whose first digit reaches the chosen one fit in LDS (kCandidates), one
  // more pass copies them there and the other digits (and the gather) work
  // on that copy instead of re-reading the row.
  //
  // A lower bound of the first digit comes without an LDS atomic per key:
  // each thread's largest key over its share of the row, then the digit at
  // which these 1024 maxima reach k. k threads hold a key in that digit or
  // above, so the row's k-th largest key is there too. Every key from that
  // digit up is then copied to LDS (a few hundred on language-model
  // logits), and the first digit proper is counted on the copy, whose
  // histogram above the bound is the row's.
  // The maxima are taken over the row's first V0 logits only (about a
  // sixteenth, and at least kHead or the whole row): the k-th largest key of
  // a part of the row is a lower bound for the whole row's as well. The copy
  // then reads the rest of the row and the first part again (just read, so
  // mostly from cache): the row crosses HBM about once.
  const int V0 = V <= kHead ? V : max(kHead, (V / 16 + 3) & ~3);
  uint32_t tmax = 0;  // below every key: threads without logits count nothing
  for_each_logit(row, V0, tid, [&](float x, int) { tmax = max(tmax, fkey(x)); });
  clear_hist();
  atomicAdd(&hist[tmax >> 21], 1u);
  __syncthreads();
  find_digit((uint32_t)p.k);
  const uint32_t d0 = s_digit;
  if (tid == 0) s_nb = 0;
  __syncthreads();
  auto copy_from = [&](int i0, int n) {
    for_each_logit(row + i0, n, tid, [&](float x, int i) {
      const uint32_t key = fkey(x);
      if ((key >> 21) >= d0) {
        const uint32_t slot = atomicAdd(&s_nb, 1u);
        if (slot < (uint32_t)kCandidates) {
          bkey[slot] = key;
          bidx[slot] = i0 + i;
        }
      }
    });
  };
  copy_from(V0, V - V0);
  copy_from(0, V0);
  __syncthreads();
  const bool buffered = s_nb <= (uint32_t)kCandidates;  // uniform
  const int nb = buffered ? (int)s_nb : 0;
  clear_hist();
  if (buffered) {
    for (int j = tid; j < nb; j += kSampleThreads) atomicAdd(&hist[bkey[j] >> 21], 1u);
  } else {
    // More keys reach the bound than the copy holds: count the whole row.
    for_each_logit(row, V, tid, [&](float x, int) { atomicAdd(&hist[fkey(x) >> 21], 1u); });
  }
  __syncthreads();
  find_digit((uint32_t)p.k);
  uint32_t prefix = s_digit << 21;
  uint32_t need = (uint32_t)p.k - s_above;
  __syncthreads();
#pragma unroll 1
  for (int pass = 1; pass < 3; ++pass) {
    const int shift = pass == 1 ? 10 : 0;
    const int bits = pass == 2 ? 10 : 11;
    const uint32_t hi_mask = 0xFFFFFFFFu << (shift + bits);
    clear_hist();
    auto count = [&](uint32_t key) {
      if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & ((1u << bits) - 1u)], 1u);
    };
    if (buffered) {
      for (int j = tid; j < nb; j += kSampleThreads) count(bkey[j]);
    } else {
      for_each_logit(row, V, tid, [&](float x, int) { count(fkey(x)); });
    }
    __syncthreads();
    find_digit(need);
    prefix |= s_digit << shift;
    need -= s_above;
    __syncthreads();
  }
  const uint32_t kstar = prefix;
  const int n_gt = p.k - (int)need;  // keys above K*; `need` ties are taken
  // s_eq now counts the keys equal to K*. When they all fit next to the keys
  // above K*, every one joins the gather and the sort keeps the lowest
  // indices (the usual case); otherwise the `need` lowest-index ties are
  // taken in index order below.
  const bool all_ties = n_gt + s_eq <= (uint32_t)kMaxTopK;

  // 2. Gather.
  if (tid == 0) {
    s_count = 0;
    s_taken = 0;
  }
  __syncthreads();
  auto take = [&](uint32_t key, int i) {
    if (key > kstar || (all_ties && key == kstar)) {
      const uint32_t slot = atomicAdd(&s_count, 1u);
      cval[slot] = key_to_float(key);
      cidx[slot] = i;
    }
  };
  if (buffered) {
    for (int j = tid; j < nb; j += kSampleThreads) take(bkey[j], bidx[j]);
  } else {
    for_each_logit(row, V, tid, [&](float x, int i) { take(fkey(x), i); });
  }
  __syncthreads();
  for (int base = 0; !all_ties && base < V; base += kSampleThreads) {
    const uint32_t taken = s_taken;
    if (taken >= need) break;  // uniform: read after the barrier below
    const int i = base + tid;
    const float v = i < V ? row[i] : 0.f;
    const bool eq = i < V && fkey(v) == kstar;
    const uint64_t ball = __ballot(eq);
    if (lane == 0) s_wave[wave] = (uint32_t)__popcll(ball);
    __syncthreads();
    uint32_t rank = taken;
    for (int w = 0; w < wave; ++w) rank += s_wave[w];
    rank += (uint32_t)__popcll(ball & ((1ull << lane) - 1ull));
    if (eq && rank < need) {
      cval[n_gt + rank] = v;
      cidx[n_gt + rank] = i;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t tot = 0;
      for (int w = 0; w < kWaves; ++w) tot += s_wave[w];
      s_taken = taken + tot;
    }
    __syncthreads();
  }
  // Unused slots sort last (with every tie gathered there can be more than
  // k filled slots; the sort puts the first k of the ranking in front).
  const int filled = all_ties ? (int)s_count : p.k;
  if (tid >= filled) {
    cval[tid] = -INFINITY;
    cidx[tid] = 0x7FFFFFFF;
  }
  __syncthreads();

  // 3. Bitonic sort into ranking order: of the first 64 slots by one wave
  // (lane shuffles, no barriers) when at most 64 are filled, else of all
  // 1024 slots.
  if (filled <= 64) {
    if (wave == 0) {
      float v = cval[lane];
      int ix = cidx[lane];
#pragma unroll
      for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          const float vo = __shfl_xor(v, stride, 64);
          const int io = __shfl_xor(ix, stride, 64);
          // The lower lane of a pair keeps the earlier element when the
          // block sorts ascending in ranking order (lane & size == 0).
          const bool lower = (lane & stride) == 0;
          const bool up = (lane & size) == 0;
          const bool mine_first = before(v, ix, vo, io);
          if (mine_first != (lower == up)) {
            v = vo;
            ix = io;
          }
        }
      }
      cval[lane] = v;
      cidx[lane] = ix;
    }
    __syncthreads();
  }
  for (int size = 2; filled > 64 && size <= kSampleThreads; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int partner = tid ^ stride;
      if (partner > tid) {
        const float va = cval[tid], vb = cval[partner];
        const int ia = cidx[tid], ib = cidx[partner];
        const bool up = (tid & size) == 0;
        if (up != before(va, ia, vb, ib)) {
          cval[tid] = vb;
          cidx[tid] = ib;
          cval[partner] = va;
          cidx[partner] = ia;
        }
      }
      __syncthreads();
    }
  }

  // 4. Weights, then the cumulative sums and the draw in ranking order.
  if (tid < p.k) cum[tid] = expf((cval[tid] - cval[0]) * p.inv_t);
  __syncthreads();
  if (p.k <= 64) {
    // One wave: inclusive scan of the weights across lanes, then the cut and
    // the draw as the first lane (rank) whose sum passes each threshold.
    if (wave == 0) {
      float c = lane < p.k ? cum[lane] : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(c, off, 64);
        if (lane >= off) c += o;
      }
      const float total = __shfl(c, p.k - 1, 64);
      const uint64_t in_k = p.k == 64 ? ~0ull : ((1ull << p.k) - 1ull);
      const uint64_t over_p = __ballot(c >= p.top_p * total) & in_k;
      const int cut = over_p ? __builtin_ctzll(over_p) : p.k - 1;
      const float target = p.u[blockIdx.x] * __shfl(c, cut, 64);
      const uint64_t upto_cut = cut == 63 ? ~0ull : ((1ull << (cut + 1)) - 1ull);
      const uint64_t over_u = __ballot(c > target) & upto_cut;
      const int pick = over_u ? __builtin_ctzll(over_u) : cut;
      if (lane == 0) p.tokens[blockIdx.x] = cidx[pick];
    }
  } else if (tid == 0) {
    float c = 0.f;
    for (int j = 0; j < p.k; ++j) {
      c += cum[j];
      cum[j] = c;
    }
    const float thr = p.top_p * c;
    int cut = p.k - 1;
    for (int j = 0; j < p.k; ++j) {
      if (cum[j] >= thr) {
        cut = j;
        break;
      }
    }
    const float target = p.u[blockIdx.x] * cum[cut];
    int pick = cut;
    for (int j = 0; j <= cut; ++j) {
      if (cum[j] > target) {
        pick = j;
        break;
      }
    }
    p.tokens[blockIdx.x] = cidx[pick];
  }
}

}  // namespace

hipError_t launch_sample(const SampleArgs& a, hipStream_t stream) {
  SampleParams p;
  p.logits = a.logits;
  p.u = a.u;
  p.tokens = a.tokens;
  p.vocab = a.vocab;
  p.k = a.top_k < a.vocab ? a.top_k : a.vocab;
  p.inv_t = 1.f / a.temperature;
  p.top_p = a.top_p;
  hipLaunchKernelGGL(sample_kernel, dim3(a.n_rows), dim3(kSampleThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace cgqa
