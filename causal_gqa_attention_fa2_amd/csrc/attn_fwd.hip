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
// Work decomposition. An item is one (sequence, query tile, KV head, head
// chunk): hpw heads of the KV head's group times 32 * W / hpw query
// positions, one wave per (head, 32 positions), on a work-group of W waves.
// For the usual group sizes (1, 2, 4, 8) there is one chunk, so every K/V
// tile is read from HBM once per item and shared by its G heads through LDS
// (grouped-query sharing). Work-groups are persistent: as many as stay
// resident, each walking its share of the items heaviest first.
//
// Two shapes, chosen from the batch's dims (launch_fwd_impl):
//   W = 8 (long sequences): eight waves, two per SIMD, share each K/V tile;
//     a three-stage LDS ring (96 KB at d = 128) whose copies of tile t+2 are
//     issued right after the barrier that opens tile t, so they have the
//     compute of tiles t and t+1 to arrive. One work-group per CU.
//   W = 4 (sequences up to 4096): four waves and a two-stage ring (64 KB),
//     copies of tile t+1 issued at tile t, so two independent work-groups
//     share each CU: one's item start, end and barrier waits overlap the
//     other's tiles, and the two waves of a SIMD are not tied to one barrier.
// Either way one barrier per tile. K is stored with the
// row-read chunk swizzle and V with the transpose-read swizzle (cdna4.h), so
// both operand loads are free of bank conflicts.
//
// Per wave and tile, everything else stays in registers:
//   S^T = K Q^T      32x32x16 MFMA; K from LDS (rows = keys), Q^T from
//                    registers. In the accumulator layout lane l owns query
//                    column l % 32, so a row's max and sum are an in-lane
//                    reduction plus one permlane32 exchange.
//   P^T = exp2(S^T * scale * log2(e) - m)        (fp32, then fp16)
//   O^T += V^T P^T   32x32x16 MFMA; P^T feeds the B operand straight from
//                    the S^T accumulators; V^T is read from the row-major V
//                    tile with ds_read_b64_tr_b16.
// The softmax reference point m moves only when some row's maximum passes it
// by more than 2^8 in weight, so O is rescaled in few tiles (with random data
// almost only the first), not whenever any of the wave's 32 row maxima grows.
#include "cdna4.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>


namespace cgqa {
namespace {

constexpr int kBC = 64;                // keys per tile
constexpr float kLazy = 8.f;           // headroom (log2 units) of the softmax reference
constexpr int kStages = 3;             // LDS ring depth with eight waves (two with four)

struct FwdParams {
  const f16* __restrict__ q;
  const f16* __restrict__ k;  // packed keys, or the paged key pool
  const f16* __restrict__ v;  // packed values, or the paged value pool
  const int32_t* __restrict__ cu;
  f16* __restrict__ o;
  float* __restrict__ lse;    // may be null for the paged prefill
  // Paged prefill only: block table [n_seqs, max_blocks], context lengths
  // (new tokens included) and the pool size.
  const int32_t* __restrict__ bt;
  const int32_t* __restrict__ ctx;
  int max_blocks, num_blocks, max_ctx;
  // Paged prefill with RoPE only: cos / sin tables [max_pos, D / 2].
  const float* __restrict__ cos_t;
  const float* __restrict__ sin_t;
  int max_pos;
  int n_seqs, T, h_q, h_kv, G, hpw, nqb, n_chunks, n_qtiles;
  // Ragged batches: 1 when work-groups walk the list of non-empty query tiles
  // (varlen_item) instead of every (query tile, sequence) slot.
  int mapped;
  int n_items;       // items: slots (or list entries) times h_kv * n_chunks
  // List keys base_b + map_s * qt in 0 .. map_keys - 1, with base_b the
  // cached context in units of map_unit = min(BR, 64) keys.
  int map_unit, map_s, map_keys;
  float scale_log2;  // scale * log2(e)
};

// Largest batch the query-tile list handles: n_seqs <= kMapSeqs, and the
// host also bounds n_seqs * ceil(map_keys / 64) (the cost of the list).
constexpr int kMapChunks = 4;
constexpr int kMapSeqs = 64 * kMapChunks;

// The list of a ragged batch's query tiles, heaviest first: the pairs
// (sequence b, query tile qt) with qt * BR < L_b, ordered by the number of
// keys they read, then by b. In units of u = min(BR, 64) keys that is
// base_b + s qt + s (s = BR / u >= 1; base_b = ceil(off_b / u), the cached
// context in the paged prefill, 0 for packed sequences), up to one less on
// a sequence's partial last tile, so the list is sorted by
// key_b(qt) = base_b + s qt.
// Every wave of the work-group computes the same answer from cu_seqlens
// (and the context lengths); lane l handles the sequences l + 64c.
//   nt_b = ceil(L_b / BR) (at most n_qtiles) and
//   A(t) = sum_b #{qt < nt_b : base_b + s qt >= t}
//        = sum_b clamp(nt_b - ceil(max(t - base_b, 0) / s), 0, nt_b)
//   counts the items with key >= t, so item k has the largest key t with
//   A(t) > k, and is the (k - A(t + 1))-th sequence, by b, whose tiles
//   include one with that key: t - base_b >= 0, divisible by s, and
//   (t - base_b) / s < nt_b.
// nt_b and base_b of the sequences lane + 64c (zero past the batch), loaded
// once per work-group.
template <bool PAGED>
__device__ __forceinline__ void varlen_counts(const FwdParams& p, int lane, int BR,
                                              int (&nt)[kMapChunks], int (&base)[kMapChunks]) {
#pragma unroll
  for (int c = 0; c < kMapChunks; ++c) {
    const int bb = lane + 64 * c;
    nt[c] = 0;
    base[c] = 0;
    if (bb < p.n_seqs) {
      const int len = p.cu[bb + 1] - p.cu[bb];
      nt[c] = min((len + BR - 1) / BR, p.n_qtiles);
      if constexpr (PAGED) {
        const int off = max(min(p.ctx[bb], p.max_ctx) - len, 0);
        base[c] = (off + p.map_unit - 1) / p.map_unit;
      }
    }
  }
}

__device__ __forceinline__ bool varlen_item(const FwdParams& p, const int (&nt)[kMapChunks],
                                            const int (&base)[kMapChunks], int k, int lane,
                                            int& qt, int& b) {
  const int s = max(p.map_s, 1);  // BR / map_unit, at least 1
  // A(t) for t = lane + 64 j, by broadcasting each sequence's counts.
  int cnt = 0;       // keys t with A(t) > k
  int a_next = 0;    // A(cnt), found below
  const int nj = (p.map_keys + 63) >> 6;
  for (int j = 0; j < nj; ++j) {
    const int t = lane + 64 * j;
    int a = 0;
#pragma unroll
    for (int c = 0; c < kMapChunks; ++c) {
      if (64 * c >= p.n_seqs) break;  // uniform
      const int nb = min(p.n_seqs - 64 * c, 64);
      for (int i = 0; i < nb; ++i) {
        const int n = __builtin_amdgcn_readlane(nt[c], i);
        const int d = max(t - __builtin_amdgcn_readlane(base[c], i), 0);
        a += max(n - (d + s - 1) / s, 0);
      }
    }
    cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(t < p.map_keys && a > k));
    // A is non-increasing in t, so the keys with A(t) > k are 0 .. cnt - 1;
    // A(cnt) is this lane's value where t == cnt.
    const uint64_t m = __builtin_amdgcn_ballot_w64(t == cnt);
    if (m) a_next = __builtin_amdgcn_readlane(a, __builtin_ctzll(m));
  }
  if (cnt == 0) return false;  // k >= A(0), the number of items
  const int key = cnt - 1;
  int r = k - (cnt < p.map_keys ? a_next : 0);
#pragma unroll
  for (int c = 0; c < kMapChunks; ++c) {
    const int d = key - base[c];
    const bool has = 64 * c + lane < p.n_seqs && d >= 0 && d % s == 0 && d / s < nt[c];
    const uint64_t m = __builtin_amdgcn_ballot_w64(has);
    const int n = __builtin_popcountll(m);
    if (r < n) {
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      const uint64_t sel = __builtin_amdgcn_ballot_w64(has && below == r);
      const int src = __builtin_ctzll(sel);
      b = 64 * c + src;
      qt = __builtin_amdgcn_readlane(d, src) / s;
      return true;
    }
    r -= n;
  }
  return false;
}

// PAGED = false: the packed varlen forward (keys and values of sequence b
// are rows cu[b] .. cu[b+1]-1 of k and v; query i sits at position i).
// PAGED = true: the chunked prefill over a paged cache. The queries of
// sequence b (rows cu[b] .. cu[b+1]-1 of q) are the last L_b of its ctx[b]
// context positions, so query i sits at position ctx[b] - L_b + i; the keys
// and values of position t are slot t % 16 of pool block bt[b][t / 16].
// ROPE (paged only): the queries are rotated by their context positions as
// they are loaded (the keys were rotated when they were appended).
template <int D, bool PAGED, bool ROPE, int W>
__global__ __launch_bounds__(64 * W, W == 4 ? 2 : 1) void fwd_kernel(FwdParams p) {
  static_assert(W == 8 || W == 4, "eight or four waves");
  constexpr int NS = W == 8 ? kStages : 2;  // ring stages
  static_assert(PAGED || !ROPE, "query rotation is a prefill option");
  constexpr int NT = D / 16;   // MFMA k-steps over the head dimension
  constexpr int ND = D / 32;   // 32-wide output blocks over the head dimension
  constexpr int CH = D / 8;    // 16-byte chunks per row
  constexpr int RPI = 64 / CH; // tile rows per copy instruction
  constexpr int IPW = kBC * CH / 64 / W;  // copy instructions per wave per tensor
  static_assert(IPW >= 1 && kBC * CH == 64 * W * IPW, "tile must split over the waves");
  // K (row reads, chunk swizzle) and V (transpose reads, transpose swizzle)
  // tiles, unpadded so that the direct copies fill them in lane order.
  __shared__ __attribute__((aligned(16))) f16 Ks[NS][kBC * D];
  __shared__ __attribute__((aligned(16))) f16 Vs[NS][kBC * D];

  const int BR = 32 * p.nqb;
  // Work-group and lane ids come straight from the hardware registers: this
  // file is built without IEEE mode, so device-library helpers (compiled
  // with it) are not inlined here and none may be called.
  const int hc = p.h_kv * p.n_chunks;
  const int tid = (int)__builtin_amdgcn_workitem_id_x();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int grp = lane >> 4;
  const int j16 = lane & 15;

  // Persistent work-groups walk the items: item i is the (query tile,
  // sequence) slot i / hc (or entry i / hc of the list of non-empty query
  // tiles of a ragged batch), KV head and head chunk from i % hc; slots and
  // list run heaviest first. As in the dq kernel, work-group w on XCD
  // x = w % 8 takes only items x + 8j (the query tiles of one (sequence, KV
  // head) then share one L2), in snake order over that XCD's work-groups.
  // Staying resident, a work-group starts its next item while the stores of
  // the last one drain, and the ragged list's tile counts load once.
  constexpr int kXcds = 8;
  const int NW = (int)__builtin_amdgcn_readfirstlane((int)gridDim.x);
  const int wgi = (int)__builtin_amdgcn_workgroup_id_x();
  const int xcd = wgi % kXcds;
  const int wx = wgi / kXcds;
  const int nwx = (NW - xcd + kXcds - 1) / kXcds;  // groups on this XCD
  int nt[kMapChunks], nbase[kMapChunks];
  if (p.mapped) varlen_counts<PAGED>(p, lane, BR, nt, nbase);

  // Copy offsets (fixed per lane for every item) and LDS bases.
  auto copy_off = [&](int i, int last, bool tr) {
    const int r = (wave * IPW + i) * RPI + lane / CH;
    const int col = tr ? swz_tr<D>(r, (lane % CH) * 8) : swz<D>(r, (lane % CH) * 8);
    const int rr = PAGED ? lane / CH : r;
    return (uint32_t)(min(rr, last) * p.h_kv * D + col) * 2u;
  };
  uint32_t koffc[IPW], voffc[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    koffc[i] = copy_off(i, PAGED ? RPI - 1 : kBC - 1, false);
    voffc[i] = copy_off(i, PAGED ? RPI - 1 : kBC - 1, true);
  }
  const uint32_t ks_lds = lds_addr(&Ks[0][0]), vs_lds = lds_addr(&Vs[0][0]);
  // Per-lane LDS offsets (halves) of the operand reads, fixed for the whole
  // kernel: the chunk swizzles depend on the row only through row % 16 (K)
  // and row % 4 (V), so the other rows of a lane's reads sit at constant
  // distances and every read below is base + per-lane offset + immediate.
  int koff[NT];  // K row l32, columns 16t + 8hi (row 32 + l32: + 32 D)
#pragma unroll
  for (int t = 0; t < NT; ++t) koff[t] = l32 * D + swz<D>(l32, 16 * t + 8 * hi);
  int voff[ND];  // V rows 4hi + j16/4 (+ 16u, + 8), columns 32db + 16(grp&1) + 4(j16&3)
#pragma unroll
  for (int db = 0; db < ND; ++db) {
    const int r = 4 * hi + (j16 >> 2);
    voff[db] = r * D + swz_tr<D>(r, 32 * db + 16 * (grp & 1) + 4 * (j16 & 3));
  }

  for (int round = 0;; ++round) {
    const int item = xcd + kXcds * (round * nwx + ((round & 1) ? nwx - 1 - wx : wx));
    if (item >= p.n_items) break;  // uniform; later rounds only go further
    const int chunk = (item % hc) % p.n_chunks;
    const int g = (item % hc) / p.n_chunks;
    int qt, b;
    if (p.mapped) {
      if (!varlen_item(p, nt, nbase, item / hc, lane, qt, b)) continue;  // past the list's end
      qt = __builtin_amdgcn_readfirstlane(qt);
      b = __builtin_amdgcn_readfirstlane(b);
    } else {
      // Every (query tile, sequence) slot, tile index descending.
      qt = p.n_qtiles - 1 - item / (p.n_seqs * hc);
      b = (item % (p.n_seqs * hc)) / hc;
    }
    const int s0 = load_uniform(p.cu, b);
    const int L = load_uniform(p.cu, b + 1) - s0;  // queries of the sequence
    const int q_wg0 = qt * BR;
    if (q_wg0 >= L) continue;  // uniform over the work-group
    // off: position of the sequence's first query; Lk: its number of keys.
    int off = 0, Lk = L;
    if constexpr (PAGED) {
      Lk = min(load_uniform(p.ctx, b), p.max_ctx);  // a context past the table is clamped
      if (Lk < L) continue;  // invalid batch (a chunk longer than its context)
      off = Lk - L;
    }
    const int n_kt = (off + min(L, q_wg0 + BR) + kBC - 1) / kBC;

    const int hig = chunk * p.hpw + wave / p.nqb;  // head within the group
    const int head = g * p.G + min(hig, p.G - 1);
    const int q0 = q_wg0 + (wave % p.nqb) * 32;  // first query row of the wave
    const int qpos = q0 + l32;                    // this lane's query row
    const int q0a = off + q0;                     // their context positions
    const int qposa = off + qpos;
    const bool wave_has_rows = q0 < L && hig < p.G;
    const bool qvalid = qpos < L && hig < p.G;

    // Copy of K/V tile kt into ring stage `stage`: instruction i of this wave
    // fills rows (wave * IPW + i) * RPI + lane / CH; lane l lands in chunk
    // slot l % CH of its row and fetches the global chunk that the swizzle
    // maps there. Keys past the sequence fetch its last row: their scores
    // are masked and their weights are zero. In the paged case the RPI rows
    // of one instruction lie in one 16-token block (RPI divides 16), so its
    // physical block is one wave-uniform scalar load; out-of-range table
    // entries are clamped into the pool, so no access leaves it.
    // Packed keys and values: the tile's first row is a wave-uniform base in
    // SGPRs and each lane adds a 32-bit byte offset fixed for the kernel
    // (recomputed with the clamp only on the sequence's last tile).
    // Paged keys and values: the RPI rows of one copy instruction lie in one
    // 16-token block, so the base is that instruction's first row and the
    // lane's row is lane / CH rows further (clamped like the row itself).
    auto issue_tile = [&](int kt, int stage) {
      // One branch per tile (not per copy) between the fixed offsets and, on
      // the sequence's last tile, the clamped ones.
      if constexpr (PAGED) {
        auto copies = [&](bool tail) __attribute__((always_inline)) {
#pragma unroll
          for (int i = 0; i < IPW; ++i) {
            const int t0 = min(kt * kBC + (wave * IPW + i) * RPI, Lk - 1);  // wave-uniform
            const int lb = min(t0 >> 4, p.max_blocks - 1);
            const int phys = min(max(load_uniform(p.bt, b * p.max_blocks + lb), 0), p.num_blocks - 1);
            const size_t base = ((size_t)(phys * 16 + (t0 - (lb << 4))) * p.h_kv + g) * D;
            const uint32_t dst = (uint32_t)(stage * kBC * D + (wave * IPW + i) * 64 * 8) * 2u;
            dma16s_at(p.k + base, tail ? copy_off(i, Lk - 1 - t0, false) : koffc[i], ks_lds + dst);
            dma16s_at(p.v + base, tail ? copy_off(i, Lk - 1 - t0, true) : voffc[i], vs_lds + dst);
          }
        };
        if (kt * kBC + kBC > Lk) copies(true);  // wave-uniform
        else copies(false);
      } else {
        const int k0 = kt * kBC;
        const size_t base = ((size_t)(s0 + k0) * p.h_kv + g) * D;
        auto copies = [&](bool tail) __attribute__((always_inline)) {
#pragma unroll
          for (int i = 0; i < IPW; ++i) {
            const uint32_t dst = (uint32_t)(stage * kBC * D + (wave * IPW + i) * 64 * 8) * 2u;
            dma16s_at(p.k + base, tail ? copy_off(i, L - 1 - k0, false) : koffc[i], ks_lds + dst);
            dma16s_at(p.v + base, tail ? copy_off(i, L - 1 - k0, true) : voffc[i], vs_lds + dst);
          }
        };
        if (k0 + kBC > L) copies(true);  // wave-uniform
        else copies(false);
      }
    };

    // The first tile's copies go out before the Q loads below, so the two
    // latencies overlap instead of adding up.
    issue_tile(0, 0);

    // Q^T as the B operand: lane holds Q[qpos][16t + 8hi .. +7]. Rows past
    // the sequence read its last row (loads stay unconditional) and are never
    // stored.
    f16x8 qf[NT];
    {
      const f16* qrow = p.q + ((size_t)(s0 + min(qpos, L - 1)) * p.h_q + head) * D + 8 * hi;
#pragma unroll
      for (int t = 0; t < NT; ++t) qf[t] = *(const f16x8*)(qrow + 16 * t);
    }
    if constexpr (ROPE) {
      // Dimension 16t + 8hi + e (t < NT/2) pairs with the one D/2 further,
      // which is element e of fragment t + NT/2 of the same lane.
      const int pos = min(off + min(qpos, L - 1), p.max_pos - 1);
      const float* ct = p.cos_t + (size_t)pos * (D / 2) + 8 * hi;
      const float* st = p.sin_t + (size_t)pos * (D / 2) + 8 * hi;
#pragma unroll
      for (int t = 0; t < NT / 2; ++t) rope_rotate8(qf[t], qf[t + NT / 2], ct + 16 * t, st + 16 * t, 1.f);
    }

    f32x16 oacc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[db] = zero_f32x16();
    float m_run = kMaxInit;  // reference maximum of the scaled scores (log2 units)
    float l_run = 0.f;       // this half-wave's share of the row sum
    // One tile step on ring stage S = kt % NS (a compile-time constant).
    // Three stages: the copies of tile kt + 2 go to stage (S + 2) % 3, which
    // held tile kt - 1. Two stages: those of tile kt + 1 go to stage
    // (S + 1) % 2, which held tile kt - 1.
    auto step = [&](int kt, auto S) {
      constexpr int stage = decltype(S)::value;
      // Tile kt has landed (this wave's copies; with three stages tile
      // kt + 1's may still fly), then every wave's copies have, and every wave
      // is done with tile kt - 1.
      if constexpr (NS == 3) {
        if (kt + 1 < n_kt) wait_vm_barrier<2 * IPW>();
        else wait_vm_barrier<0>();
        if (kt + 2 < n_kt) issue_tile(kt + 2, (stage + 2) % NS);
      } else {
        wait_vm_barrier<0>();
        if (kt + 1 < n_kt) issue_tile(kt + 1, (stage + 1) % NS);
      }

      if (!wave_has_rows || kt * kBC > q0a + 31) return;  // fully masked for this wave
      const f16* Kb = Ks[stage];
      const f16* Vb = Vs[stage];
      // S^T for the two 32-key halves of the tile, as two interleaved chains.
      // Every K fragment of the tile is read in one batch before the products
      // (scheduling fences keep the compiler from pairing each read with its
      // use, which left the matrix core waiting on LDS latency), and the V^T
      // fragments go out right behind them, so they land during the softmax.
      f32x16 s[2] = {zero_f32x16(), zero_f32x16()};
      {
        f16x8 kf[2][NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          kf[0][t] = *(const f16x8*)(Kb + koff[t]);
          kf[1][t] = *(const f16x8*)(Kb + 32 * D + koff[t]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          s[0] = mfma32x32x16(kf[0][t], qf[t], s[0]);
          s[1] = mfma32x32x16(kf[1][t], qf[t], s[1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      f16x8 vf[4][ND];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int db = 0; db < ND; ++db)
          vf[u][db] = cat4(lds_read_tr(Vb + voff[db] + 16 * u * D),
                           lds_read_tr(Vb + voff[db] + (16 * u + 8) * D));
      }
      __builtin_amdgcn_sched_barrier(0);
      // Causal mask (diagonal tiles only) and the tile maximum of raw scores.
      if (kt * kBC + kBC - 1 > q0a) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kt * kBC + kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
            if (key > qposa) s[kb][i] = -INFINITY;
          }
        }
      }
      // Two independent three-input max chains (v_max3_f32) over the 32 scores.
      float mx0 = fmaxf(s[0][0], s[1][0]), mx1 = fmaxf(s[0][1], s[1][1]);
#pragma unroll
      for (int i = 2; i < 16; i += 2) {
        mx0 = __builtin_fmaxf(__builtin_fmaxf(mx0, s[0][i]), s[1][i]);
        mx1 = __builtin_fmaxf(__builtin_fmaxf(mx1, s[0][i + 1]), s[1][i + 1]);
      }
      float mx = fmaxf(mx0, mx1);
      mx = half_swap_max(mx) * p.scale_log2;
      // m_run is a reference point, not always the exact running maximum: it
      // moves (and O and l are rescaled) only when a row's maximum passes it by
      // more than kLazy, so the weights below stay <= 2^kLazy and the wave
      // skips the rescale in almost every tile after the first. The result is
      // the same softmax up to rounding, whatever the reference.
      const bool grow = mx > m_run + kLazy;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? mx : m_run;
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db) {
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        }
        m_run = m_new;
      }
      const float m_new = m_run;

      // P^T = exp2(S^T * scale * log2(e) - m), as B operands: k-step u covers
      // tile keys 16u..16u+15; slot e of half hi holds key 16u + 8(e/4) +
      // 4hi + e%4.
      f16x8 pf[4];
      float rs = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = fast_exp2(fmaf(s[u >> 1][8 * (u & 1) + e], p.scale_log2, -m_new));
          rs += x;
          pf[u][e] = (f16)x;
        }
      }
      l_run += rs;

      // O^T += V^T P^T. A-operand slot e of half hi must hold V[key(e)][d]
      // for the same keys: transpose reads (above) of rows 16u + 4hi + j16/4
      // and 8 rows further. The k-step loop is outermost, so consecutive
      // products go to different accumulators (four independent chains).
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int db = 0; db < ND; ++db) oacc[db] = mfma32x32x16(vf[u][db], pf[u], oacc[db]);
      }
    };

    // Q^T was loaded with ordinary loads: wait for them here with the builtin
    // (whose effect the compiler tracks), so it places no wait of its own inside
    // the loop, where such a wait would also stall on the copies in flight.
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0); tile 0 included
    if (NS == 3 && n_kt > 1) issue_tile(1, 1);
    for (int kt = 0; kt < n_kt; kt += NS) {
      step(kt, std::integral_constant<int, 0>{});
      if (kt + 1 < n_kt) step(kt + 1, std::integral_constant<int, 1>{});
      if constexpr (NS == 3) {
        if (kt + 2 < n_kt) step(kt + 2, std::integral_constant<int, 2>{});
      }
    }

    const float l_tot = half_swap_sum(l_run);  // all lanes take part in the exchange
    if (qvalid) {
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
      if (hi == 0 && (!PAGED || p.lse != nullptr))
        p.lse[(size_t)head * p.T + s0 + qpos] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    // Every wave is done with the ring before the next item's copies land in
    // it (an LDS-only barrier: the stores above stay in flight).
    lds_barrier();
  }
}

}  // namespace

namespace {

template <bool PAGED, int W>
void launch_fwd_shape(const FwdParams& p, const FwdArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(64 * W);
  if (PAGED && a.rope_cos != nullptr) {
    if (a.head_dim == 128)
      hipLaunchKernelGGL((fwd_kernel<128, true, true, W>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_kernel<64, true, true, W>), grid, block, 0, stream, p);
  } else if (a.head_dim == 128) {
    hipLaunchKernelGGL((fwd_kernel<128, PAGED, false, W>), grid, block, 0, stream, p);
  } else {
    hipLaunchKernelGGL((fwd_kernel<64, PAGED, false, W>), grid, block, 0, stream, p);
  }
}

template <bool PAGED>
hipError_t launch_fwd_impl(const FwdArgs& a, hipStream_t stream) {
  FwdParams p;
  p.q = (const f16*)a.q;
  p.k = (const f16*)a.k;
  p.v = (const f16*)a.v;
  p.cu = a.cu_seqlens;
  p.o = (f16*)a.o;
  p.lse = a.lse;
  p.bt = a.block_table;
  p.ctx = a.ctx_lens;
  p.max_blocks = a.max_blocks_per_seq;
  p.num_blocks = a.num_blocks;
  p.max_ctx = a.max_ctx_len;
  p.cos_t = a.rope_cos;
  p.sin_t = a.rope_sin;
  p.max_pos = a.rope_max_pos;
  p.n_seqs = a.n_seqs;
  p.T = a.total_tokens;
  p.h_q = a.h_q;
  p.h_kv = a.h_kv;
  p.G = a.h_q / a.h_kv;
  // Sequences (or contexts) up to 4096 keys take four-wave work-groups, two
  // per CU; longer ones eight-wave work-groups, one per CU (same-run timing:
  // the four-wave shape is 2-8% faster up to 4096 keys and 1-3% slower at
  // 8192).
  const int max_keys = PAGED ? a.max_ctx_len : a.max_seqlen;
  const int W = max_keys <= 4096 ? 4 : 8;
  const QTileLayout lay = qtile_layout(p.G, W);
  p.hpw = lay.hpw;
  p.nqb = lay.nqb;
  p.n_chunks = lay.n_chunks;
  const int BR = 32 * p.nqb;
  p.n_qtiles = (a.max_seqlen + BR - 1) / BR;
  p.scale_log2 = a.scale * kLog2e;
  // Ragged batches walk the list of non-empty query tiles: at most
  // floor(T / BR) + n_seqs of them (each sequence adds at most one partial
  // tile), against n_qtiles * n_seqs slots.
  const long long slots = (long long)p.n_qtiles * a.n_seqs;
  const long long items = std::min<long long>(slots, (long long)a.total_tokens / BR + a.n_seqs);
  p.map_unit = std::min(BR, kBC);
  p.map_s = BR / p.map_unit;
  p.map_keys = (PAGED ? (a.max_ctx_len + p.map_unit - 1) / p.map_unit : 0) +
               p.map_s * (p.n_qtiles - 1) + 1;
  p.mapped = items < slots && a.n_seqs <= kMapSeqs &&
             (long long)a.n_seqs * ((p.map_keys + 63) / 64) <= 512;
  // Persistent grid: at most one work-group per CU (eight waves) or two
  // (four waves), each walking its share of the items. Items are dealt by
  // their residue mod 8, so the grid is the item count or at least 8.
  p.n_items = (int)((p.mapped ? items : slots) * a.h_kv * p.n_chunks);
  const int resident = std::max((W == 4 ? 2 : 1) * a.num_cus, 8);
  const dim3 grid((unsigned)std::max(1, std::min(p.n_items, resident)));
  if (W == 4)
    launch_fwd_shape<PAGED, 4>(p, a, grid, stream);
  else
    launch_fwd_shape<PAGED, 8>(p, a, grid, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  return launch_fwd_impl<false>(a, stream);
}

hipError_t launch_prefill(const FwdArgs& a, hipStream_t stream) {
  return launch_fwd_impl<true>(a, stream);
}

}  // namespace cgqa
