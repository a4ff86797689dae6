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
//   1. dq:   query-stationary, shaped like the forward. Persistent
//            work-groups of eight waves walk work items (sequence, query
//            tile, KV head, head chunk); each wave owns one (head, 32-row
//            query block) slot of the item. A wave forms its rows' D from dO
//            and O (and stores D and LSE * log2(e) for kernel 2), then for
//            every 32-key K/V tile computes S^T = K Q^T and dP^T = V dO^T
//            (lane = query column, so LSE and D are per-lane scalars), dS^T,
//            and dQ^T += K^T dS^T with K^T taken by transpose reads of the
//            same K tile. Each wave holds its rows' whole dQ^T, so no wave
//            reduction follows; dq is written once, in fp16.
//   2. dkdv: key-stationary. One work-group of eight waves per (sequence,
//            128-key tile, KV head); waves w and w + 4 own the same 32 keys.
//            The (G query heads) x (32-row query blocks at or after the keys)
//            stream through an LDS ring. Wave w (K in registers) forms
//            S = Q K^T and P, hands P to wave w + 4 through LDS and adds
//            dV^T += dO^T P; wave w + 4 (V in registers) works one block
//            behind: dP = dO V^T, dS = P * (dP - D), dK^T += Q^T dS. Each
//            wave keeps one 32 x d accumulator, so two waves fit per SIMD and
//            one's matrix work overlaps the other's softmax arithmetic.
// Compared with a single key-stationary kernel that adds dQ with fp32
// atomics, this recomputes S and dP once more (7 instead of 5 GEMMs of the
// tile size) but drops the fp32 dQ accumulator, its zeroing, its conversion
// pass and all atomic traffic.
//
// Batches of very unequal sequence lengths take a second path (chosen by
// the host from the batch shape, with a larger workspace): a row-term
// kernel, then dK/dV that also stores each fp16 dS block, then a dQ kernel
// that reads those blocks instead of recomputing S and dP (5 GEMMs of the
// tile size plus the dS traffic). There the short work items make the
// recomputing dq kernel's per-item costs dominate.
//
// Tiles reach LDS through direct global-to-LDS copies issued two tiles ahead
// (cdna4.h dma16/dma4), one barrier per tile. Every tile uses the chunk
// swizzle of cdna4.h, so row reads and transpose reads are free of bank
// conflicts; all LDS operand addresses are per-lane offsets fixed for the
// whole loop.
#include "cdna4.h"
#include "kernels.h"

#include <algorithm>

#include <type_traits>

namespace cgqa {
namespace {

constexpr int kDqBC = 32;       // keys per K/V tile (dq kernel)
constexpr int kDqStages = 3;    // K/V ring depth (dq kernel)
constexpr int kKvStages = 4;    // Q/dO ring depth (dkdv kernel)
constexpr int kBK = 128;        // keys per dkdv work-group (4 x 32)
// Accumulator chains of dkdv's first product. One dependent chain measured
// faster than two interleaved ones (which need 16 adds to merge): the other
// wave of the SIMD keeps the matrix core busy between the chain's products.
constexpr int kDkdvChains = 1;
constexpr int kBwdThreads = 512;
constexpr int kKMapChunks = 4;  // ragged-batch lists: up to 256 sequences

struct BwdParams {
  const f16* __restrict__ q;
  const f16* __restrict__ k;
  const f16* __restrict__ v;
  const f16* __restrict__ o;
  const float* __restrict__ lse;
  const f16* __restrict__ dout;
  const int32_t* __restrict__ cu;
  float* __restrict__ drow;  // workspace: fp32 [h_q, T], -D = -rowsum(dO * O)
  float* __restrict__ lse2;  // workspace: fp32 [h_q, T], LSE * log2(e)
  f16* __restrict__ dq;
  f16* __restrict__ dk;
  f16* __restrict__ dv;
  f16* __restrict__ ds;      // workspace: fp16 dS blocks (32 x 32, lane-major)
  int nbmax;                 // 32-row blocks of the longest sequence
  // RoPE tables [max_pos, D / 2] when dq and dk are rotated back at their
  // stores (the ROPE kernels), else null.
  const float* __restrict__ cos_t;
  const float* __restrict__ sin_t;
  int max_pos;
  int n_seqs, T, h_q, h_kv, G, hpw, nqb, n_chunks, n_qtiles, n_ktiles;
  // Ragged batches: 1 when dK/dV work-groups walk the list of non-empty key
  // tiles sorted by work (dkdv_item) instead of every (key tile, sequence)
  // slot; max_qb bounds a key tile's query blocks.
  int kmapped, max_qb;
  // Ragged batches: 1 when the dq kernels walk the list of non-empty query
  // tiles (dq_item, at most q_items entries) instead of every slot.
  int qmapped, q_items;
  float scale, scale_log2;
};

// Stores one lane's half of an fp32 accumulator row (element i of block db is
// dimension 32 db + 8 (i / 4) + 4 hi + i % 4) as fp16, scaled by sc. ROPE:
// the row is a gradient with respect to rotated q or k, and is carried back
// to the unrotated tensor by the inverse rotation at position pos (dimension
// j pairs with j + D/2, which is block db + D/64 of the same lane), in fp32
// and rounded to fp16 once (rope_pair_f32).
template <int D, bool ROPE>
__device__ __forceinline__ void store_acc_row(f16* row, const f32x16* acc, float sc, int hi,
                                              const BwdParams& p, int pos) {
  constexpr int ND = D / 32;
  if constexpr (ROPE) {
    const int pp = min(pos, p.max_pos - 1);
    const float* ct = p.cos_t + (size_t)pp * (D / 2) + 4 * hi;
    const float* st = p.sin_t + (size_t)pp * (D / 2) + 4 * hi;
    // All values first, then the stores back to back in address order (as
    // the plain path issues them), so that each row's lines are completed
    // while they are still in L2.
    f16x4 w[ND][4];
#pragma unroll
    for (int db = 0; db < ND / 2; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 c = *(const f32x4*)(ct + 32 * db + 8 * r4);
        const f32x4 s = *(const f32x4*)(st + 32 * db + 8 * r4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f16 a, b;
          rope_pair_f32(acc[db][4 * r4 + e] * sc, acc[db + ND / 2][4 * r4 + e] * sc, c[e], -s[e],
                        a, b);
          w[db][r4][e] = a;
          w[db + ND / 2][r4][e] = b;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < ND; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) *(f16x4*)(row + 32 * db + 8 * r4 + 4 * hi) = w[db][r4];
    }
  } else {
#pragma unroll
    for (int db = 0; db < ND; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (f16)(acc[db][4 * r4 + e] * sc);
        *(f16x4*)(row + 32 * db + 8 * r4 + 4 * hi) = w;
      }
    }
  }
}

// dS = P * (dP - D) in fp16 for the 16 accumulator elements of a lane (dpd
// holds dP - D), each product rounded once (v_fma_mix*_f16): elements
// 8u .. 8u + 7 go to f[u].
__device__ __forceinline__ void ds_pack(const float* pv, const f32x16& dpd, f16x8* f) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 8 * u + 2 * e;
      const f16x2 r = {(f16)__builtin_fmaf(pv[i], dpd[i], 0.f),
                       (f16)__builtin_fmaf(pv[i + 1], dpd[i + 1], 0.f)};
      w[e] = __builtin_bit_cast(uint32_t, r);
    }
    f[u] = __builtin_bit_cast(f16x8, w);
  }
}

// The list of a ragged batch's query tiles of BR rows, heaviest first: the
// pairs (sequence b, query tile qt) with qt * BR < L_b, ordered by qt
// descending (the tiles with the most keys first), then by b; nt_b =
// ceil(L_b / BR) (at most n_qtiles) of the sequences lane + 64c are loaded
// once per work-group. A(t) = sum_b max(nt_b - t, 0) counts the items with
// tile index >= t, so item k has the largest qt with A(qt) > k, and is the
// (k - A(qt + 1))-th sequence, by b, with nt_b > qt. Returns false past the
// end of the list.
__device__ __forceinline__ void dq_counts(const BwdParams& p, int lane, int BR,
                                          int (&nt)[kKMapChunks]) {
#pragma unroll
  for (int c = 0; c < kKMapChunks; ++c) {
    const int bb = lane + 64 * c;
    nt[c] = bb < p.n_seqs ? min((p.cu[bb + 1] - p.cu[bb] + BR - 1) / BR, p.n_qtiles) : 0;
  }
}

__device__ __forceinline__ bool dq_item(const BwdParams& p, const int (&nt)[kKMapChunks], int k,
                                        int lane, int& qt, int& b) {
  int cnt = 0;     // tiles t with A(t) > k
  int a_next = 0;  // A(cnt), found below
  const int nj = (p.n_qtiles + 63) >> 6;
  for (int j = 0; j < nj; ++j) {
    const int t = lane + 64 * j;
    int a = 0;
#pragma unroll
    for (int c = 0; c < kKMapChunks; ++c) {
      if (64 * c >= p.n_seqs) break;  // uniform
      const int nb = min(p.n_seqs - 64 * c, 64);
      for (int i = 0; i < nb; ++i) a += max(__builtin_amdgcn_readlane(nt[c], i) - t, 0);
    }
    cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(t < p.n_qtiles && a > k));
    const uint64_t m = __builtin_amdgcn_ballot_w64(t == cnt);
    if (m) a_next = __builtin_amdgcn_readlane(a, __builtin_ctzll(m));
  }
  if (cnt == 0) return false;
  qt = cnt - 1;
  int r = k - (cnt < p.n_qtiles ? a_next : 0);
#pragma unroll
  for (int c = 0; c < kKMapChunks; ++c) {
    const bool has = nt[c] > qt;
    const uint64_t m = __builtin_amdgcn_ballot_w64(has);
    const int n = __builtin_popcountll(m);
    if (r < n) {
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      b = 64 * c + __builtin_ctzll(__builtin_amdgcn_ballot_w64(has && below == r));
      return true;
    }
    r -= n;
  }
  return false;
}

template <int D, bool ROPE = false>
__global__ __launch_bounds__(kBwdThreads, 1) void dq_kernel(BwdParams p) {
  constexpr int NT = D / 16;   // MFMA k-steps over the head dimension
  constexpr int ND = D / 32;   // 32-wide output blocks over the head dimension
  constexpr int CH = D / 8;    // 16-byte chunks per row
  constexpr int RPI = 64 / CH; // tile rows per copy instruction
  constexpr int NI = kDqBC * CH / 64;  // copy instructions per tensor and tile
  constexpr int CPW = 2 * NI / 8;       // copy instructions per wave and tile (K and V)
  static_assert(CPW >= 1 && 2 * NI == 8 * CPW, "tile must split over the waves");
  constexpr int TILE = kDqBC * D;
  // Ring stage st holds the K tile at smem + 2 st TILE and the V tile right
  // after it (chunk swizzle, unpadded so the copies fill them in lane order).
  __shared__ __attribute__((aligned(16))) f16 smem[2 * kDqStages * TILE];
  static_assert(kDqStages == 3, "the ring below has three stages");

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int grp = lane >> 4;
  const int j16 = lane & 15;

  // Persistent work-groups: item i is query tile n_qtiles - 1 - i / per of
  // (sequence, KV head, head chunk) i % per, so items run heaviest first.
  // Work-groups are dealt to the 8 XCDs round-robin (w % 8), each with its
  // own L2: work-group w takes only items i = x + 8 j with x = w % 8, so the
  // query tiles of one (sequence, KV head) share an L2 as they did with one
  // work-group per item. Within class x the nwx groups of that XCD take
  // j = r nwx + wx (r even) or r nwx + nwx - 1 - wx (r odd) in rounds r
  // (snake order keeps the per-group sums even). Staying resident lets a
  // group overlap the start of its next item (first K/V copies, row loads)
  // with the end of the current one.
  constexpr int kXcds = 8;
  const int BR = 32 * p.nqb;
  const int per = p.n_seqs * p.h_kv * p.n_chunks;
  const int n_items = p.n_qtiles * per;
  const int NW = (int)gridDim.x;
  const int w = (int)blockIdx.x;
  const int xcd = w % kXcds;
  const int wx = w / kXcds;
  const int nwx = (NW - xcd + kXcds - 1) / kXcds;  // groups on this XCD
  auto item_of = [&](int r) {
    const int j = r * nwx + ((r & 1) ? nwx - 1 - wx : wx);
    return xcd + kXcds * j;
  };
  struct Item {
    int b, g, chunk, s0, L, q_wg0, n_kt;
  };
  auto decode = [&](int i) {
    Item it;
    const int qt = p.n_qtiles - 1 - i / per;
    int rem = i % per;
    it.chunk = rem % p.n_chunks;
    rem /= p.n_chunks;
    it.g = rem % p.h_kv;
    it.b = rem / p.h_kv;
    it.s0 = load_uniform(p.cu, it.b);
    it.L = load_uniform(p.cu, it.b + 1) - it.s0;
    it.q_wg0 = qt * BR;
    it.n_kt = it.q_wg0 < it.L ? (min(it.L, it.q_wg0 + BR) + kDqBC - 1) / kDqBC : 0;
    return it;
  };
  // Next non-empty item from round r on (n_items if none).
  auto next_item = [&](int& r) {
    for (;; ++r) {
      const int i = item_of(r);
      if (i >= n_items) return n_items;
      if (decode(i).n_kt > 0) return i;
    }
  };

  // Copy of K/V tile kt of item `it` into ring stage st: instruction i (of
  // 2 NI) fills rows (i % NI) * RPI + lane / CH of K (i < NI) or V; lane l
  // lands in chunk slot l % CH of its row and fetches the global chunk the
  // swizzle maps there. Keys past the sequence fetch its last row (their
  // scores are masked).
  // The tile's first row is a wave-uniform base in SGPRs; each lane adds a
  // 32-bit byte offset fixed for the kernel, recomputed with the clamp only
  // on the sequence's last tile.
  // With RoPE (whose epilogue needs registers) the lane id is rebuilt at each
  // issue, so the compiler cannot keep the offsets live through the loop;
  // without, the offsets stay in registers (cheaper per tile).
  const int tsel = (wave * CPW) / NI;  // K (waves 0-3) or V (4-7)
  auto copy_off = [&](int c, int last) {
    const int ln = ROPE ? lane_id_fresh() : lane;
    const int r = ((wave * CPW) % NI + c) * RPI + ln / CH;
    return (uint32_t)(min(r, last) * p.h_kv * D + swz<D>(r, (ln % CH) * 8)) * 2u;
  };
  const uint32_t smem_lds = lds_addr(smem);
  auto issue_tile = [&](const Item& it, int kt, int st) {
    const int k0 = kt * kDqBC;
    const f16* base = (tsel ? p.v : p.k) + ((size_t)(it.s0 + k0) * p.h_kv + it.g) * D;
    const bool tail = k0 + kDqBC > it.L;  // wave-uniform
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int ii = (wave * CPW) % NI + c;
      dma16s_at(base, copy_off(c, tail ? it.L - 1 - k0 : 31),
                smem_lds + (uint32_t)((2 * st + tsel) * TILE + ii * 512) * 2u);
    }
  };
  // This wave's rows of item `it`: head hig of the group's chunk, 32 query
  // positions from q0.
  struct Rows {
    int head, q0, qpos, qrow;
    bool has_rows, valid;
  };
  auto rows_of = [&](const Item& it) {
    Rows rw;
    const int hig = it.chunk * p.hpw + wave / p.nqb;
    rw.head = it.g * p.G + min(hig, p.G - 1);
    rw.q0 = it.q_wg0 + (wave % p.nqb) * 32;
    rw.qpos = rw.q0 + l32;
    rw.has_rows = rw.q0 < it.L && hig < p.G;
    rw.valid = rw.qpos < it.L && hig < p.G;
    rw.qrow = it.s0 + min(rw.qpos, it.L - 1);  // rows past the end read the last row
    return rw;
  };
  // Q^T and dO^T as B operands (lane holds row qpos, columns 16t + 8hi .. +7),
  // O for the row terms, and the row's LSE.
  f16x8 qf[NT], dof[NT], of[NT];
  float lse_row;
  auto load_rows = [&](const Rows& rw) {
    const size_t off = ((size_t)rw.qrow * p.h_q + rw.head) * D + 8 * hi;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      qf[t] = *(const f16x8*)(p.q + off + 16 * t);
      dof[t] = *(const f16x8*)(p.dout + off + 16 * t);
      of[t] = *(const f16x8*)(p.o + off + 16 * t);
    }
    lse_row = p.lse[(size_t)rw.head * p.T + rw.qrow];
  };

  // Per-lane LDS offsets (halves), fixed for the kernel; the swizzle depends
  // on the row only through row % 16.
  int koff[NT];  // K / V row l32, columns 16t + 8hi
#pragma unroll
  for (int t = 0; t < NT; ++t) koff[t] = l32 * D + swz<D>(l32, 16 * t + 8 * hi);
  // K^T transpose reads: rows 16u + 4hi + j16/4 (and 8 further), columns
  // 32db + 16(grp&1) + 4(j16&3); A slot e of half hi <-> key
  // 16u + 8(e/4) + 4hi + e%4 of the tile, as in the dS^T B operand.
  int ktr0[ND], ktr1[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) {
    const int col = 32 * db + 16 * (grp & 1) + 4 * (j16 & 3);
    const int r0 = 4 * hi + (j16 >> 2);
    const int r1 = r0 + 8;
    ktr0[db] = r0 * D + swz<D>(r0, col);
    ktr1[db] = r1 * D + swz<D>(r1, col);
  }

  int round = 0;
  int cur = next_item(round);
  if (cur >= n_items) return;  // uniform over the work-group
  Item it = decode(cur);
  Rows rw = rows_of(it);
  // The first tile's copies go out before the row loads, so the two
  // latencies overlap instead of adding up.
  issue_tile(it, 0, 0);
  load_rows(rw);

  for (;;) {
    float dsum = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum += (float)dof[t][e] * (float)of[t][e];
    }
    dsum = half_swap_sum(dsum);  // D = rowsum(dO * O) over both halves of the row
    const float lse2 = lse_row * kLog2e;

    f32x16 acc[ND];  // dQ^T: rows = head dim, cols = queries
#pragma unroll
    for (int db = 0; db < ND; ++db) acc[db] = zero_f32x16();

    // Everything in flight (tile 0's copies, the row loads, the previous
    // item's stores) is waited for here, so the compiler places no wait of
    // its own inside the loop; tile 1's copies go out after the wait.
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    const int n_kt = it.n_kt;
    if (n_kt > 1) issue_tile(it, 1, 1);
    // One tile step on ring stage S = kt % 3 (a compile-time constant, so
    // every LDS operand address is a per-lane offset plus an immediate); the
    // copies of tile kt + 2 go to stage (S + 2) % 3, which held tile kt - 1.
    auto step = [&](int kt, auto S) __attribute__((always_inline)) {
      constexpr int st = decltype(S)::value;
      // Tile kt has landed for every wave, and every wave is done with kt - 1.
      if (kt + 1 < n_kt) wait_vm_barrier<CPW>();
      else wait_vm_barrier<0>();
      if (kt + 2 < n_kt) issue_tile(it, kt + 2, (st + 2) % kDqStages);
      const int k0 = kt * kDqBC;
      if (!rw.has_rows || k0 > rw.q0 + 31) return;  // fully masked for this wave
      const f16* Kb = smem + st * 2 * TILE;
      const f16* Vb = Kb + TILE;
      // S^T and dP^T for the tile's 32 keys (accumulator element i: key
      // k0 + 8(i/4) + 4hi + i%4, query qpos), two interleaved chains.
      // dP^T starts from -D, so the chain yields dP^T - D.
      f32x16 sv = zero_f32x16(), dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) dp[i] = -dsum;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        sv = mfma32x32x16(*(const f16x8*)(Kb + koff[t]), qf[t], sv);
        dp = mfma32x32x16(*(const f16x8*)(Vb + koff[t]), dof[t], dp);
      }
      // K^T fragments of the dQ product, read while the softmax terms below
      // are computed.
      f16x8 ktf[2][ND];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int db = 0; db < ND; ++db)
          ktf[u][db] = cat4(lds_read_tr(Kb + ktr0[db] + 16 * u * D),
                            lds_read_tr(Kb + ktr1[db] + 16 * u * D));
      }
      __builtin_amdgcn_sched_barrier(0);
      f16x8 dsf[2];
      if (k0 + 31 > rw.q0) {
        // Diagonal tile: keep P where key <= qpos, i.e. the constant part
        // 8(i/4) + i%4 of the key is <= qpos - k0 - 4hi.
        const int lim = rw.qpos - k0 - 4 * hi;
        float pv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pv[i] = fast_exp2(fmaf(sv[i], p.scale_log2, -lse2));
          if (8 * (i >> 2) + (i & 3) > lim) pv[i] = 0.f;
        }
        ds_pack(pv, dp, dsf);
      } else {
        // Every other tile takes this unmasked copy (two copies, so the
        // compiler does not evaluate the mask everywhere).
        float pv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) pv[i] = fast_exp2(fmaf(sv[i], p.scale_log2, -lse2));
        ds_pack(pv, dp, dsf);
      }
      // dQ^T += K^T dS^T over the 32 keys (K^T by transpose reads).
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int db = 0; db < ND; ++db) acc[db] = mfma32x32x16(ktf[u][db], dsf[u], acc[db]);
      }
    };
    for (int kt = 0; kt < n_kt; kt += kDqStages) {
      step(kt, std::integral_constant<int, 0>{});
      if (kt + 1 < n_kt) step(kt + 1, std::integral_constant<int, 1>{});
      if (kt + 2 < n_kt) step(kt + 2, std::integral_constant<int, 2>{});
    }

    // This wave's dq rows, scaled, in fp16; D and LSE * log2(e) for the
    // dK/dV kernel. The stores go out before the next item's copies and row
    // loads, so they drain first.
    if (rw.valid) {
      f16* dqrow = p.dq + ((size_t)rw.qrow * p.h_q + rw.head) * D;
      store_acc_row<D, ROPE>(dqrow, acc, p.scale, hi, p, rw.qpos);
      if (hi == 0) {
        p.drow[(size_t)rw.head * p.T + rw.qrow] = -dsum;
        p.lse2[(size_t)rw.head * p.T + rw.qrow] = lse2;
      }
    }
    // Every wave is done with the ring (an LDS-only barrier: the stores stay
    // in flight). The next item's first tile goes to stage 0 and its row
    // loads go out.
    lds_barrier();
    ++round;
    const int nxt = next_item(round);
    if (nxt >= n_items) break;
    it = decode(nxt);
    rw = rows_of(it);
    issue_tile(it, 0, 0);
    load_rows(rw);
  }
}

// Item k of the list of a ragged batch's non-empty key tiles, heaviest
// first: the pairs (sequence b, key tile kt) with kt < nk_b = ceil(L_b / 128),
// ordered by their work w = c_b - 4 kt descending (c_b = ceil(L_b / 32) query
// blocks; the tile sees the blocks from 4 kt on), then by b. With the
// work-groups dispatched in this order, the longest tiles start first and
// the shortest fill the end. Every wave computes the same answer from
// cu_seqlens; lane l holds the sequences l + 64c. Returns false past the end.
//   A(v) = sum_b #{kt < nk_b : c_b - 4 kt >= v} = sum_b min(nk_b, (c_b - v) / 4 + 1)
//   (0 when c_b < v) counts the items of work >= v, so item k has the largest
//   work v* with A(v*) > k, and is the (k - A(v* + 1))-th sequence, by b, with
//   a tile of work exactly v*: (c_b - v*) % 4 == 0 and (c_b - v*) / 4 < nk_b.
__device__ __forceinline__ bool dkdv_item(const BwdParams& p, int k, int lane, int& b, int& kt) {
  int cq[kKMapChunks], nk[kKMapChunks];
#pragma unroll
  for (int c = 0; c < kKMapChunks; ++c) {
    const int bb = lane + 64 * c;
    const int len = bb < p.n_seqs ? p.cu[bb + 1] - p.cu[bb] : 0;
    cq[c] = (len + 31) / 32;
    nk[c] = (len + kBK - 1) / kBK;
  }
  int cnt = 0;     // works v in 1 .. max_qb with A(v) > k
  int a_next = 0;  // A(cnt + 1), found below
  const int nj = (p.max_qb + 63) >> 6;
  for (int j = 0; j < nj; ++j) {
    const int v = 1 + lane + 64 * j;
    int a = 0;
#pragma unroll
    for (int c = 0; c < kKMapChunks; ++c) {
      if (64 * c >= p.n_seqs) break;  // uniform
      const int nb = min(p.n_seqs - 64 * c, 64);
      for (int i = 0; i < nb; ++i) {
        const int cb = __builtin_amdgcn_readlane(cq[c], i);
        const int kb = __builtin_amdgcn_readlane(nk[c], i);
        if (cb >= v) a += min(kb, (cb - v) / 4 + 1);
      }
    }
    cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(v <= p.max_qb && a > k));
    // A is non-increasing in v, so the works with A(v) > k are 1 .. cnt;
    // A(cnt + 1) is this lane's value where v == cnt + 1.
    const uint64_t m = __builtin_amdgcn_ballot_w64(v == cnt + 1);
    if (m) a_next = __builtin_amdgcn_readlane(a, __builtin_ctzll(m));
  }
  if (cnt == 0) return false;  // k >= A(1), the number of items
  const int vs = cnt;
  int r = k - (vs < p.max_qb ? a_next : 0);
#pragma unroll
  for (int c = 0; c < kKMapChunks; ++c) {
    const int d = cq[c] - vs;
    const bool has = 64 * c + lane < p.n_seqs && d >= 0 && (d & 3) == 0 && (d >> 2) < nk[c];
    const uint64_t m = __builtin_amdgcn_ballot_w64(has);
    const int n = __builtin_popcountll(m);
    if (r < n) {
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      const uint64_t sel = __builtin_amdgcn_ballot_w64(has && below == r);
      const int src = __builtin_ctzll(sel);
      b = 64 * c + src;
      kt = __builtin_amdgcn_readlane(d, src) >> 2;
      return true;
    }
    r -= n;
  }
  return false;
}

template <int D, bool STORE_DS, bool ROPE = false>
__global__ __launch_bounds__(kBwdThreads, 1) void dkdv_kernel(BwdParams p) {
  constexpr int NT = D / 16;
  constexpr int ND = D / 32;
  constexpr int CH = D / 8;
  constexpr int RPI = 64 / CH;
  constexpr int IPB = 32 * CH / 64;  // copy instructions per 32-row block of one tensor
  // Team 0 issues every copy (team 1 issues none, so its vmcnt counts only
  // its own dS stores and it never waits for them at the ring barrier).
  constexpr int CPW = 2 * IPB / 4;   // copy instructions per team-0 wave per block (Q and dO)
  static_assert(CPW >= 1 && 2 * IPB == 4 * CPW, "block must split over team 0");
  constexpr int BLK = 32 * D;
  // Ring of query blocks: [stage][Q, dO] tiles (chunk swizzle) and, per
  // stage, LSE * log2(e) (32 floats) then D (32 floats) of the block's rows.
  __shared__ __attribute__((aligned(16))) f16 Xs[kKvStages][2][BLK];
  __shared__ __attribute__((aligned(16))) float Ls[kKvStages][64];
  // P hand-off, [block parity][wave pair][two 16-byte groups per lane].
  __shared__ __attribute__((aligned(16))) f16 Px[2][4][2 * 64 * 8];

  // Key tile 0 of every (sequence, KV head) sees the most query rows: first.
  // Ragged batches walk the work-sorted list of non-empty key tiles.
  int kt, g, b;
  if (p.kmapped) {
    g = (int)blockIdx.x % p.h_kv;
    if (!dkdv_item(p, (int)blockIdx.x / p.h_kv, (int)threadIdx.x & 63, b, kt)) return;
    b = __builtin_amdgcn_readfirstlane(b);
    kt = __builtin_amdgcn_readfirstlane(kt);
  } else {
    const int per = p.n_seqs * p.h_kv;
    kt = (int)blockIdx.x / per;
    const int rem = (int)blockIdx.x % per;
    g = rem % p.h_kv;
    b = rem / p.h_kv;
  }
  const int s0 = p.cu[b];
  const int L = p.cu[b + 1] - s0;
  const int k_wg0 = kt * kBK;
  if (k_wg0 >= L) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int grp = lane >> 4;
  const int j16 = lane & 15;
  // Waves w and w + 4 share a SIMD (measured on gfx950): one of each team,
  // so one's matrix work overlaps the other's arithmetic.
  const int team = wave >> 2;  // 0: S, P, dV;  1: dP, dS, dK (one block behind)
  const int w4 = wave & 3;
  const int kw0 = k_wg0 + 32 * w4;  // first key of this wave pair
  const int key = kw0 + l32;

  // Query blocks at or after the key tile, for each head of the group.
  const int qb_begin = k_wg0 / 32;
  const int n_qb = (L + 31) / 32 - qb_begin;
  const int n_it = p.G * n_qb;
  // Block m is query block qb_begin + m % n_qb of head m / n_qb of the group.
  // Blocks are issued and processed in order, so each stream keeps its
  // (head, block) pair as counters instead of dividing by n_qb per block (a
  // runtime division costs some 25 scalar instructions).
  struct BlkPos {
    int h, qb;
  };
  auto advance = [&](BlkPos& ps) {
    if (++ps.qb == n_qb) {
      ps.qb = 0;
      ++ps.h;
    }
  };

  // Copies of block m into stage st: team-0 wave w4 issues CPW of the block's
  // 2 * IPB copy instructions, all of one tensor (Q for w4 < 2, dO after);
  // instruction ii fills rows ii * RPI + lane / CH. The block's first row is
  // a wave-uniform base in SGPRs and each lane adds a 32-bit offset fixed for
  // the loop; on the sequence's last block rows past the end are clamped to
  // its last row (the mask below zeroes their weights). Wave 0 also copies
  // the row terms.
  const int tsel = (w4 * CPW) / IPB;
  // Byte offset of the lane's chunk of copy c in a block, and the same with
  // its row clamped to `last`.
  auto copy_off = [&](int c, int last) {
    const int r = ((w4 * CPW) % IPB + c) * RPI + lane / CH;
    return (uint32_t)(min(r, last) * p.h_q * D + swz<D>(r, (lane % CH) * 8)) * 2u;
  };
  uint32_t coff[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) coff[c] = copy_off(c, 31);
  const uint32_t xs_lds = lds_addr(&Xs[0][0][0]);
  BlkPos ipos{0, 0};  // next block to issue (team 0)
  auto issue_blk = [&](auto ST) {
    constexpr int st = decltype(ST)::value;
    const int head = g * p.G + ipos.h;
    const int q0 = (qb_begin + ipos.qb) * 32;
    advance(ipos);
    const f16* base = (tsel ? p.dout : p.q) + ((size_t)(s0 + q0) * p.h_q + head) * D;
    // One branch per block (not per copy) between the fixed offsets and, on
    // the sequence's last block, the clamped ones.
    auto copies = [&](bool tail) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const int ii = (w4 * CPW) % IPB + c;
        dma16s_at(base, tail ? copy_off(c, L - 1 - q0) : coff[c],
                  xs_lds + (uint32_t)((st * 2 + tsel) * BLK + ii * 512) * 2u);
      }
    };
    if (q0 + 31 >= L) copies(true);  // wave-uniform
    else copies(false);
    if (wave == 0) {
      const float* src = (lane < 32 ? p.lse2 : p.drow) + (size_t)head * p.T + s0 +
                         min(q0 + l32, L - 1);
      dma4(src, &Ls[st][0]);
    }
  };

  // Block 0's copies go out before the ordinary loads below, so the two
  // latencies overlap.
  if (team == 0) issue_blk(std::integral_constant<int, 0>{});

  // K (team 0) or V (team 1) of the pair's keys as the B operand: lane holds
  // row `key` (rows past the end read the last row; never stored), columns
  // 16t + 8hi .. +7.
  f16x8 kvf[NT];
  {
    const f16* src = (team ? p.v : p.k) + ((size_t)(s0 + min(key, L - 1)) * p.h_kv + g) * D + 8 * hi;
#pragma unroll
    for (int t = 0; t < NT; ++t) kvf[t] = *(const f16x8*)(src + 16 * t);
  }

  // Per-lane LDS offsets (halves) within a block, fixed for the loop; the
  // team's tile (X: rows of the first product; Y: transposed operand of the
  // second) is folded in, so that with compile-time ring stages every read
  // below is a per-lane register plus an immediate.
  const int xsel = team * BLK, ysel = (1 - team) * BLK;
  int xoff[NT];  // row l32, columns 16t + 8hi (first GEMM's A operand)
#pragma unroll
  for (int t = 0; t < NT; ++t) xoff[t] = xsel + l32 * D + swz<D>(l32, 16 * t + 8 * hi);
  // Transpose reads of rows 16u + 4hi + j16/4 (and 8 further), columns
  // 32db + 16(grp&1) + 4(j16&3): A slot e of half hi <-> query row
  // 16u + 8(e/4) + 4hi + e%4, the slot order of the P / dS B operand.
  int yoff0[ND], yoff1[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) {
    const int col = 32 * db + 16 * (grp & 1) + 4 * (j16 & 3);
    const int r0 = 4 * hi + (j16 >> 2);
    const int r1 = r0 + 8;
    yoff0[db] = ysel + r0 * D + swz<D>(r0, col);
    yoff1[db] = ysel + r1 * D + swz<D>(r1, col);
  }
  const int loff = 32 * team + 4 * hi;  // row terms: LSE * log2(e) (team 0) or -D (team 1)

  f32x16 acc[ND];  // dV^T (team 0) or dK^T (team 1): rows = head dim, cols = keys
#pragma unroll
  for (int db = 0; db < ND; ++db) acc[db] = zero_f32x16();

  // Team 1's dS block of query block m (32 rows x the pair's 32 keys) to the
  // workspace for the dQ kernel, lane-major: lane l's 16 values (rows
  // 8(i/4) + 4hi + i%4 of key column l % 32) at halves 16 l .. 16 l + 15,
  // with the two 8-value halves swapped for lanes 32..63 (so that the dQ
  // kernel's transpose reads of lanes l and l + 32, 1 KiB apart, fall in
  // different LDS banks). Pairs wholly past the sequence store nothing. The
  // stores count in vmcnt, so the next iteration's copy wait also waits for
  // them.
  auto store_ds = [&](const BlkPos& ps, const f16x8* f) {
    if (kw0 >= L) return;
    const int head = g * p.G + ps.h;
    const int qb = qb_begin + ps.qb;
    f16* dst = p.ds + ((((size_t)b * p.h_q + head) * p.nbmax + qb) * p.nbmax + (kw0 >> 5)) * 1024 +
               lane * 16;
    *(f16x8*)(dst + 8 * hi) = f[0];
    *(f16x8*)(dst + 8 - 8 * hi) = f[1];
  };

  BlkPos cpos{0, 0};  // next block to process
  // Iteration j of team TEAM on the ring stage of its block (a compile-time
  // constant: the loop below is unrolled by the ring depth, and j = J mod 4).
  // Team 0 works on block j, team 1 on block j - 1.
  auto body = [&](int j, auto J, auto TEAM) {
    constexpr int tm = decltype(TEAM)::value;
    // Block j has landed for every wave (block j + 1 may still be in
    // flight), every wave is done with its block of the previous iteration,
    // and team 0's P of block j - 1 is in LDS.
    if constexpr (tm == 1) {
      lds_barrier();  // no copies of its own; its dS stores stay in flight
    } else {
      if (j + 1 < n_it) {
        if (wave == 0) wait_vm_barrier<CPW + 1>();
        else wait_vm_barrier<CPW>();
      } else {
        wait_vm_barrier<0>();
      }
      // Stage (j + 2) % 4 last held block j - 2, which team 1 finished in
      // the previous iteration.
      if (j + 2 < n_it) issue_blk(std::integral_constant<int, (decltype(J)::value + 2) % kKvStages>{});
    }
    const int m = j - tm;
    if (m < 0 || m >= n_it) return;  // uniform over the wave
    constexpr int st = (decltype(J)::value - tm + kKvStages) % kKvStages;
    constexpr int par = (decltype(J)::value - tm + kKvStages) & 1;  // m & 1
    const BlkPos mpos = cpos;  // block m
    advance(cpos);
    const int q0 = (qb_begin + mpos.qb) * 32;
    const f16* Xb = &Xs[st][0][0];

    // Operand reads are issued in blocks ahead of their uses (scheduling
    // fences keep the compiler from sinking them): the row fragments of the
    // first product (and team 1's row terms, its accumulator's start), then,
    // behind its matrix work, the transposed fragments of the second, team
    // 0's row terms and the P hand-off.
    f16x8 xfr[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) xfr[t] = *(const f16x8*)(Xb + xoff[t]);
    const float* lrow = &Ls[st][loff];
    f32x4 l4[4];
    if constexpr (tm == 1) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) l4[jj] = *(const f32x4*)(lrow + 8 * jj);
    }
    __builtin_amdgcn_sched_barrier(0);
    // S = Q K^T (team 0) or dP - D = dO V^T - D (team 1, started from -D);
    // accumulator element i: query row q0 + 8(i/4) + 4hi + i%4, key `key`.
    // One chain over the k-steps, or two interleaved over even / odd ones
    // (kDkdvChains).
    f32x16 sa, sb = zero_f32x16();
    if constexpr (tm == 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sa[i] = l4[i >> 2][i & 3];
    } else {
      sa = zero_f32x16();
    }
    if constexpr (kDkdvChains == 2) {
#pragma unroll
      for (int t = 0; t < NT; t += 2) {
        sa = mfma32x32x16(xfr[t], kvf[t], sa);
        sb = mfma32x32x16(xfr[t + 1], kvf[t + 1], sb);
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) sa = mfma32x32x16(xfr[t], kvf[t], sa);
    }
    __builtin_amdgcn_sched_barrier(0);
    f16x8 yfr[ND][2];
#pragma unroll
    for (int db = 0; db < ND; ++db) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
        yfr[db][u] = cat4(lds_read_tr(Xb + yoff0[db] + 16 * u * D),
                          lds_read_tr(Xb + yoff1[db] + 16 * u * D));
    }
    f16* px = &Px[par][w4][lane * 8];
    f16x8 p0, p1;
    if constexpr (tm == 0) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) l4[jj] = *(const f32x4*)(lrow + 8 * jj);
    } else {
      p0 = *(const f16x8*)px;
      p1 = *(const f16x8*)(px + 512);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kDkdvChains == 2) sa += sb;
    f16x8 f[2];
    if constexpr (tm == 0) {
      // Causal mask on diagonal blocks, row mask on the sequence's last
      // block; every other block takes the unmasked copy of the loop (two
      // copies, so the compiler does not evaluate the mask everywhere).
      if (kw0 + 31 > q0 || q0 + 31 >= L) {
        // Keep P where key <= row < L, i.e. 0 <= row - key < L - key. Keys
        // past the sequence (lim <= 0) keep nothing, so their dS is zero.
        const int lim = max(L - key, 0);
        const int rel = q0 + 4 * hi - key;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = fast_exp2(fmaf(sa[i], p.scale_log2, -l4[i >> 2][i & 3]));
          const bool keep = (unsigned)(rel + 8 * (i >> 2) + (i & 3)) < (unsigned)lim;
          f[i >> 3][i & 7] = (f16)(keep ? pv : 0.f);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          f[i >> 3][i & 7] = (f16)fast_exp2(fmaf(sa[i], p.scale_log2, -l4[i >> 2][i & 3]));
      }
      *(f16x8*)px = f[0];
      *(f16x8*)(px + 512) = f[1];
    } else {
      // dS = P * (dP - D), one rounding to fp16 per element (the product of
      // an fp16 and an fp32 value, rounded once: v_fma_mix).
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const f16x8 pp = u ? p1 : p0;
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f16x2 r = {(f16)__builtin_fmaf((float)pp[2 * e], sa[8 * u + 2 * e], 0.f),
                           (f16)__builtin_fmaf((float)pp[2 * e + 1], sa[8 * u + 2 * e + 1], 0.f)};
          w[e] = __builtin_bit_cast(uint32_t, r);
        }
        f[u] = __builtin_bit_cast(f16x8, w);
      }
      if constexpr (STORE_DS) store_ds(mpos, f);
    }
    __builtin_amdgcn_sched_barrier(0);

    // dV^T += dO^T P (team 0) or dK^T += Q^T dS (team 1).
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int db = 0; db < ND; ++db) acc[db] = mfma32x32x16(yfr[db][u], f[u], acc[db]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): see dq_kernel
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  static_assert(kKvStages == 4, "the loop is unrolled by the ring depth");
  if (team == 0) {
    if (n_it > 1) issue_blk(I1{});
    for (int j = 0; j <= n_it; j += 4) {
      body(j, I0{}, I0{});
      if (j + 1 <= n_it) body(j + 1, I1{}, I0{});
      if (j + 2 <= n_it) body(j + 2, I2{}, I0{});
      if (j + 3 <= n_it) body(j + 3, I3{}, I0{});
    }
  } else {
    for (int j = 0; j <= n_it; j += 4) {
      body(j, I0{}, I1{});
      if (j + 1 <= n_it) body(j + 1, I1{}, I1{});
      if (j + 2 <= n_it) body(j + 2, I2{}, I1{});
      if (j + 3 <= n_it) body(j + 3, I3{}, I1{});
    }
  }

  if (key >= L) return;
  f16* dst = (team ? p.dk : p.dv) + ((size_t)(s0 + key) * p.h_kv + g) * D;
  if (ROPE && team)
    store_acc_row<D, ROPE>(dst, acc, p.scale, hi, p, key);  // dK, rotated back
  else
    store_acc_row<D, false>(dst, acc, team ? p.scale : 1.f, hi, p, key);
}


// Row terms of the backward for every (token, query head) row: -D =
// -rowsum(dO * O) and LSE * log2(e), stored [h_q, T]. A work-group takes
// tiles of 16 tokens x 16 heads: it reads their O and dO rows in memory
// order (a group of D/8 lanes per row, every row of the tile in flight at
// once; rows past the batch read its last row and are not stored), sums each
// row with v_dot2 products and DPP lane moves, gathers D in LDS, and then
// reads the LSE and writes the two terms token-contiguously for each head.
constexpr int kRowsTB = 16, kRowsHC = 16;  // tokens and heads per tile
template <int D>
__global__ __launch_bounds__(256) void bwd_rows_kernel(BwdParams p) {
  constexpr int LPR = D / 8;             // lanes per row
  constexpr int RPP = 256 / LPR;         // rows per pass
  constexpr int PASSES = kRowsTB * kRowsHC / RPP;
  static_assert(kRowsTB * kRowsHC == 256 && PASSES * RPP == 256, "tile must split over the passes");
  __shared__ float dsh[kRowsHC][kRowsTB + 1];
  const int tid = threadIdx.x;
  const int gl = tid % LPR;
  const int rg = tid / LPR;
  const int nhc = (p.h_q + kRowsHC - 1) / kRowsHC;
  const int n_tiles = (p.T + kRowsTB - 1) / kRowsTB * nhc;
  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int t0 = tile / nhc * kRowsTB;
    const int h0 = tile % nhc * kRowsHC;
    f16x8 ov[PASSES], gv[PASSES];
#pragma unroll
    for (int u = 0; u < PASSES; ++u) {
      const int r = u * RPP + rg;  // (token, head) of the tile, heads fastest
      const int t = min(t0 + r / kRowsHC, p.T - 1), h = min(h0 + r % kRowsHC, p.h_q - 1);
      const size_t row = (size_t)t * p.h_q + h;
      ov[u] = *(const f16x8*)(p.o + row * D + 8 * gl);
      gv[u] = *(const f16x8*)(p.dout + row * D + 8 * gl);
    }
#pragma unroll
    for (int u = 0; u < PASSES; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        acc = __builtin_amdgcn_fdot2(f16x2{gv[u][e], gv[u][e + 1]}, f16x2{ov[u][e], ov[u][e + 1]},
                                     acc, false);
      acc = group_sum<LPR>(acc);
      const int r = u * RPP + rg;
      if (gl == 0) dsh[r % kRowsHC][r / kRowsHC] = acc;
    }
    __syncthreads();
    {
      const int hl = tid / kRowsTB, tl = tid % kRowsTB;
      const int h = h0 + hl, t = t0 + tl;
      if (h < p.h_q && t < p.T) {
        const size_t i = (size_t)h * p.T + t;
        p.drow[i] = -dsh[hl][tl];
        p.lse2[i] = p.lse[i] * kLog2e;
      }
    }
    __syncthreads();
  }
}

// dQ from the dS blocks the dK/dV kernel stored: dQ^T += K^T dS^T over the
// 32-key blocks at or before each query block. Work items, persistent
// XCD-aware work-groups and the three-stage ring are those of dq_kernel; a
// ring stage holds the K tile (chunk swizzle) and each wave's own dS block
// (2 KiB, copied as stored). Operands come from LDS transpose reads in
// natural key order: k-step u, half hi, slot s <-> key 16u + 8hi + s, both
// for K^T (rows of the K tile) and for dS^T (the stored block's lanes
// 32 hi' + key hold rows 8c + 4hi' + 0..3 in their 8-byte chunk c).
template <int D, bool ROPE = false>
__global__ __launch_bounds__(kBwdThreads, 1) void dq_ds_kernel(BwdParams p) {
  constexpr int ND = D / 32;
  constexpr int CH = D / 8;
  constexpr int RPI = 64 / CH;
  constexpr int NI = kDqBC * CH / 64;  // K copy instructions per tile (8 or 4)
  static_assert(NI >= 1 && 8 % NI == 0, "K tile must split over the waves");
  constexpr int CPW = 3;               // copies per wave and tile: one K, two dS
  constexpr int TILE = kDqBC * D;
  constexpr int STAGE = TILE + 8 * 1024;
  __shared__ __attribute__((aligned(16))) f16 smem[kDqStages * STAGE];
  static_assert(kDqStages == 3, "the ring below has three stages");

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int grp = lane >> 4;
  const int j16 = lane & 15;

  constexpr int kXcds = 8;
  const int BR = 32 * p.nqb;
  const int per = p.n_seqs * p.h_kv * p.n_chunks;
  const int hcq = p.h_kv * p.n_chunks;
  // Ragged batches: item i is entry i / hcq of the list of non-empty query
  // tiles, KV head and head chunk from i % hcq.
  const int n_items = p.qmapped ? p.q_items * hcq : p.n_qtiles * per;
  int ntq[kKMapChunks];
  if (p.qmapped) dq_counts(p, (int)threadIdx.x & 63, 32 * p.nqb, ntq);
  const int NW = (int)gridDim.x;
  const int w = (int)blockIdx.x;
  const int xcd = w % kXcds;
  const int wx = w / kXcds;
  const int nwx = (NW - xcd + kXcds - 1) / kXcds;
  auto item_of = [&](int r) {
    const int j = r * nwx + ((r & 1) ? nwx - 1 - wx : wx);
    return xcd + kXcds * j;
  };
  struct Item {
    int b, g, chunk, s0, L, q_wg0, n_kt;
  };
  auto decode = [&](int i) {
    Item it;
    int qt;
    if (p.qmapped) {
      const int rem = i % hcq;
      it.chunk = rem % p.n_chunks;
      it.g = rem / p.n_chunks;
      int qq = 0, bb = 0;
      if (!dq_item(p, ntq, i / hcq, (int)threadIdx.x & 63, qq, bb)) {  // past the list's end
        it.b = 0;
        it.s0 = it.L = it.q_wg0 = it.n_kt = 0;
        return it;
      }
      qt = __builtin_amdgcn_readfirstlane(qq);
      it.b = __builtin_amdgcn_readfirstlane(bb);
    } else {
      qt = p.n_qtiles - 1 - i / per;
      int rem = i % per;
      it.chunk = rem % p.n_chunks;
      rem /= p.n_chunks;
      it.g = rem % p.h_kv;
      it.b = rem / p.h_kv;
    }
    it.s0 = load_uniform(p.cu, it.b);
    it.L = load_uniform(p.cu, it.b + 1) - it.s0;
    it.q_wg0 = qt * BR;
    it.n_kt = it.q_wg0 < it.L ? (min(it.L, it.q_wg0 + BR) + kDqBC - 1) / kDqBC : 0;
    return it;
  };
  auto next_item = [&](int& r) {
    for (;; ++r) {
      const int i = item_of(r);
      if (i >= n_items) return n_items;
      if (decode(i).n_kt > 0) return i;
    }
  };
  struct Rows {
    int head, q0, qpos, qrow;
    bool has_rows, valid;
    const f16* dsb;  // this wave's dS blocks: query block row of the workspace
    int qbc;         // its query block, clamped into the sequence
  };
  auto rows_of = [&](const Item& it) {
    Rows rw;
    const int hig = it.chunk * p.hpw + wave / p.nqb;
    rw.head = it.g * p.G + min(hig, p.G - 1);
    rw.q0 = it.q_wg0 + (wave % p.nqb) * 32;
    rw.qpos = rw.q0 + l32;
    rw.has_rows = rw.q0 < it.L && hig < p.G;
    rw.valid = rw.qpos < it.L && hig < p.G;
    rw.qrow = it.s0 + min(rw.qpos, it.L - 1);
    rw.qbc = min(rw.q0 >> 5, (it.L - 1) >> 5);
    rw.dsb = p.ds + (((size_t)it.b * p.h_q + rw.head) * p.nbmax + rw.qbc) * p.nbmax * 1024;
    return rw;
  };
  // Copies of tile kt into stage st: one K instruction per wave (rows of
  // instruction wave % NI; with NI < 8 two waves write the same rows with the
  // same data) and this wave's dS block for key block kt, clamped to a block
  // that exists so every wave issues the same number of copies.
  auto issue_tile = [&](const Item& it, const Rows& rw, int kt, int st) {
    f16* stage = smem + st * STAGE;
    const int ii = wave % NI;
    const int r = ii * RPI + lane / CH;
    const int sl = (lane % CH) * 8;
    const size_t row = ((size_t)(it.s0 + min(kt * kDqBC + r, it.L - 1)) * p.h_kv + it.g) * D;
    dma16(p.k + row + swz<D>(r, sl), stage + ii * 512);
    const f16* src = rw.dsb + (size_t)min(kt, rw.qbc) * 1024 + lane * 8;
    dma16(src, stage + TILE + wave * 1024);
    dma16(src + 512, stage + TILE + wave * 1024 + 512);
  };

  // Per-lane LDS offsets (halves). K^T: rows 8hi + 4r + j16/4 (+ 16u),
  // columns 32db + 16(grp&1) + 4(j16&3). dS^T: lane 4e + jj of group grp
  // reads the chunk of stored lane 32 (jj&1) + 16u + 8(grp>>1) + 4r + e,
  // chunk 2(grp&1) + jj/2, which for stored lanes 32..63 sits at chunk
  // position c ^ 2 (the dK/dV kernel swaps their halves).
  int kto[2][ND];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int row = 8 * hi + 4 * r + (j16 >> 2);
      kto[r][db] = row * D + swz<D>(row, 32 * db + 16 * (grp & 1) + 4 * (j16 & 3));
    }
  }
  int dso[2][2];
  {
    const int e = j16 >> 2, jj = j16 & 3;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
        dso[u][r] = (32 * (jj & 1) + 16 * u + 8 * (grp >> 1) + 4 * r + e) * 16 +
                    4 * ((2 * (grp & 1) + (jj >> 1)) ^ (2 * (jj & 1)));
    }
  }

  int round = 0;
  int cur = next_item(round);
  if (cur >= n_items) return;
  Item it = decode(cur);
  Rows rw = rows_of(it);
  issue_tile(it, rw, 0, 0);

  for (;;) {
    f32x16 acc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) acc[db] = zero_f32x16();
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    const int n_kt = it.n_kt;
    if (n_kt > 1) issue_tile(it, rw, 1, 1);
    auto step = [&](int kt, auto S) __attribute__((always_inline)) {
      constexpr int st = decltype(S)::value;
      if (kt + 1 < n_kt) wait_vm_barrier<CPW>();
      else wait_vm_barrier<0>();
      if (kt + 2 < n_kt) issue_tile(it, rw, kt + 2, (st + 2) % kDqStages);
      if (!rw.has_rows || kt * kDqBC > rw.q0 + 31) return;  // no keys of this tile are seen
      const f16* Kb = smem + st * STAGE;
      const f16* Db = Kb + TILE + wave * 1024;
      f16x8 dsf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) dsf[u] = cat4(lds_read_tr(Db + dso[u][0]), lds_read_tr(Db + dso[u][1]));
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const f16x8 kt8 = cat4(lds_read_tr(Kb + kto[0][db] + 16 * u * D),
                                 lds_read_tr(Kb + kto[1][db] + 16 * u * D));
          acc[db] = mfma32x32x16(kt8, dsf[u], acc[db]);
        }
      }
    };
    for (int kt = 0; kt < n_kt; kt += kDqStages) {
      step(kt, std::integral_constant<int, 0>{});
      if (kt + 1 < n_kt) step(kt + 1, std::integral_constant<int, 1>{});
      if (kt + 2 < n_kt) step(kt + 2, std::integral_constant<int, 2>{});
    }
    if (rw.valid) {
      f16* dqrow = p.dq + ((size_t)rw.qrow * p.h_q + rw.head) * D;
      store_acc_row<D, ROPE>(dqrow, acc, p.scale, hi, p, rw.qpos);
    }
    lds_barrier();
    ++round;
    const int nxt = next_item(round);
    if (nxt >= n_items) break;
    it = decode(nxt);
    rw = rows_of(it);
    issue_tile(it, rw, 0, 0);
  }
}

}  // namespace

namespace {

// Recompute path (ds = false): dq (which also forms the row terms) then
// dK/dV. dS path: row terms, then dK/dV (which also stores dS), then dQ from
// dS. ROPE: dq and dk are rotated back at their stores.
template <int D, bool ROPE>
void launch_bwd_kernels(const BwdParams& p, bool ds, dim3 gq, dim3 gk, dim3 gr,
                        hipStream_t stream) {
  if (!ds) {
    hipLaunchKernelGGL((dq_kernel<D, ROPE>), gq, dim3(kBwdThreads), 0, stream, p);
    hipLaunchKernelGGL((dkdv_kernel<D, false, ROPE>), gk, dim3(kBwdThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(bwd_rows_kernel<D>, gr, dim3(256), 0, stream, p);
    hipLaunchKernelGGL((dkdv_kernel<D, true, ROPE>), gk, dim3(kBwdThreads), 0, stream, p);
    hipLaunchKernelGGL((dq_ds_kernel<D, ROPE>), gq, dim3(kBwdThreads), 0, stream, p);
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
  p.lse2 = a.lse2;
  p.ds = (f16*)a.ds;
  p.nbmax = (a.max_seqlen + 31) / 32;
  p.dq = (f16*)a.dq;
  p.dk = (f16*)a.dk;
  p.dv = (f16*)a.dv;
  p.n_seqs = a.n_seqs;
  p.T = a.total_tokens;
  p.h_q = a.h_q;
  p.h_kv = a.h_kv;
  p.G = a.h_q / a.h_kv;
  // dq work items: eight (head, 32-row block) slots, one per wave; hpw heads
  // of the group times 8 / hpw query blocks.
  const QTileLayout lay = qtile_layout(p.G);
  p.hpw = lay.hpw;
  p.nqb = lay.nqb;
  p.n_chunks = lay.n_chunks;
  p.n_qtiles = (a.max_seqlen + 32 * p.nqb - 1) / (32 * p.nqb);
  p.n_ktiles = (a.max_seqlen + kBK - 1) / kBK;
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  // Ragged batches: the list of non-empty query tiles has at most
  // floor(T / BR) + n_seqs entries, against n_qtiles * n_seqs slots.
  const int BRq = 32 * p.nqb;
  const long long qslots = (long long)p.n_qtiles * a.n_seqs;
  const long long qitems = std::min<long long>(qslots, (long long)a.total_tokens / BRq + a.n_seqs);
  // (only the dq-from-dS kernel of the ragged path walks the list)
  p.qmapped = a.ds != nullptr && qitems < qslots && a.n_seqs <= 64 * kKMapChunks &&
              (long long)a.n_seqs * ((p.n_qtiles + 63) / 64) <= 512;
  p.q_items = (int)qitems;
  const int n_items = (int)((p.qmapped ? qitems : qslots) * a.h_kv * p.n_chunks);
  // Persistent dq grids; items are dealt by their residue mod 8, so the grid
  // is the item count or at least 8.
  const int resident = a.num_cus > 8 ? a.num_cus : 8;
  const dim3 gq(n_items < resident ? n_items : resident);
  // Ragged batches: the list of non-empty key tiles has at most
  // floor(T / 128) + n_seqs entries (each sequence adds at most one partial
  // tile), against n_ktiles * n_seqs slots.
  const long long kslots = (long long)p.n_ktiles * a.n_seqs;
  const long long kitems = std::min<long long>(kslots, (long long)a.total_tokens / kBK + a.n_seqs);
  p.max_qb = (a.max_seqlen + 31) / 32;
  p.kmapped = kitems < kslots && a.n_seqs <= 64 * kKMapChunks &&
              (long long)a.n_seqs * ((p.max_qb + 63) / 64) <= 512;
  const dim3 gk((unsigned)((p.kmapped ? kitems : kslots) * a.h_kv));
  const long long wgs = (long long)((a.total_tokens + kRowsTB - 1) / kRowsTB) *
                        ((a.h_q + kRowsHC - 1) / kRowsHC);  // row-term tiles
  const dim3 gr((unsigned)(wgs < 4 * a.num_cus ? wgs : 4 * a.num_cus));
  const bool ds = a.ds != nullptr;
  if (a.rope_cos != nullptr) {
    p.cos_t = a.rope_cos;
    p.sin_t = a.rope_sin;
    p.max_pos = a.rope_max_pos;
    if (a.head_dim == 128)
      launch_bwd_kernels<128, true>(p, ds, gq, gk, gr, stream);
    else
      launch_bwd_kernels<64, true>(p, ds, gq, gk, gr, stream);
  } else {
    p.cos_t = p.sin_t = nullptr;
    p.max_pos = 0;
    if (a.head_dim == 128)
      launch_bwd_kernels<128, false>(p, ds, gq, gk, gr, stream);
    else
      launch_bwd_kernels<64, false>(p, ds, gq, gk, gr, stream);
  }
  return hipGetLastError();
}

}  // namespace cgqa
