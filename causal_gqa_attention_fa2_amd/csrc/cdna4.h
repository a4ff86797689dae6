// cdna4.h -- small device helpers for gfx950 (CDNA4): fp16 MFMA, LDS transpose
// reads and half-wave exchanges. Lane layouts below were checked on the
// hardware with an in-bounds probe.
//
// v_mfma_f32_32x32x16_f16 (one wave, 64 lanes; l32 = lane % 32, hi = lane / 32):
//   A operand (8 halves): A[row = l32][k = 8*hi + s], s = 0..7
//   B operand (8 halves): B[k = 8*hi + s][col = l32]
//   C/D (16 floats):      C[row = 8*(i/4) + 4*hi + (i%4)][col = l32], i = 0..15
// ds_read_b64_tr_b16: inside each group of 16 lanes, lane j returns element e
//   (e = 0..3) of the 4-element chunk addressed by lane 4*e + j/4, taken at
//   position j%4. If lane j of a group addresses row (r0 + j/4), column
//   (c0 + 4*(j%4)) of a row-major fp16 tile, lane j receives column c0 + j of
//   rows r0..r0+3 -- a 4x16 transpose straight out of LDS.
// v_permlane32_swap(x, x) returns {x[lane], x[lane ^ 32]} in some order, so
//   max/sum of the two halves of a wave takes one exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cgqa {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x4_raw __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running maxima start at this finite value (not -inf) so that a row whose
// scores are all masked never computes (-inf) - (-inf).
constexpr float kMaxInit = -1.0e30f;

__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16 on an LDS address.
__device__ __forceinline__ f16x4 lds_read_tr(const f16* p) {
  fp16x4_raw r = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (__attribute__((address_space(3))) fp16x4_raw*)(p));
  return __builtin_bit_cast(f16x4, r);
}

__device__ __forceinline__ f16x8 cat4(f16x4 a, f16x4 b) {
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ float half_swap_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float half_swap_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane move by a DPP control (the source lane's value; 0 where the pattern
// has none).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over each aligned group of N lanes (N = 8 or 16) with DPP moves; every
// lane of the group ends with the total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "groups of 8 or 16 lanes");
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]: partner lane ^ 1
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]: partner lane ^ 2
  x += dpp_mov<0x141>(x);  // row_half_mirror: the other quad of the 8-lane half
  if constexpr (N == 16) x += dpp_mov<0x140>(x);  // row_mirror: other half of the row
  return x;
}

// Lane index (0..63) recomputed where it is used (two VALU instructions that
// the compiler can neither hoist nor keep live), for per-lane constants that
// are cheaper to rebuild than to hold in registers through a loop.
__device__ __forceinline__ int lane_id_fresh() {
  int r;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
  return r;
}

__device__ __forceinline__ f16x8 zero_f16x8() { return f16x8{0, 0, 0, 0, 0, 0, 0, 0}; }

// Column (in halves) of element (row, col) in an LDS tile of D-half rows with
// no padding whose 16-byte chunks are XOR-swizzled per row, for tiles read
// both ways by the MFMA operand loads. With D = 128 on the 64-bank LDS,
// 16-byte row reads of 16 consecutive rows hit 16 distinct chunk slots, and
// ds_read_b64_tr_b16 over 4 consecutive rows (row % 4 == 0) by two 16-lane
// groups 32 bytes apart hits 8 distinct 32-byte slots (measured on gfx950:
// row reads at the conflict-free rate, transpose reads at ~80% of the rate of
// a 160-half padded tile). `col` may be any multiple of 4.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  const int f = D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((row >> 1) & 7);
  return (((col >> 3) ^ f) << 3) | (col & 7);
}

// Column of element (row, col) in an unpadded D-half LDS tile read only by
// ds_read_b64_tr_b16 (4 consecutive rows, row % 4 == 0, two 16-lane groups
// 32 bytes apart): the 16-byte chunks of row r are XOR-ed with 4 * (r % 4),
// which keeps every 32-byte pair in order and spreads the 8 pairs of a pass
// over all 64 banks (measured on gfx950 at the rate of a 160-half padded
// tile).
template <int D>
__device__ __forceinline__ int swz_tr(int row, int col) {
  const int f = D == 128 ? ((row & 3) << 2) : (((row & 3) << 1) & 7);
  return (((col >> 3) ^ f) << 3) | (col & 7);
}

// Asynchronous 16-byte-per-lane copy from global memory straight into LDS
// (global_load_lds_dwordx4): lane l's 16 bytes land at lds_wave_base + 16 l,
// so one wave fills 1 KB of LDS in lane order; lds_wave_base must be the same
// for every lane of the wave. Completion is tracked by vmcnt, like an
// ordinary load. The copy is issued from inline assembly so the compiler's
// wait insertion does not see it: otherwise it cannot tell the ring stage
// being read from the stages still being filled and waits for every copy in
// flight before each LDS read. The caller therefore owns the waits
// (wait_vm_barrier) and must not issue other vector-memory loads whose
// completion the compiler would track while copies are in flight. M0 holds
// the LDS address; nothing else in these kernels uses M0.
__device__ __forceinline__ void dma16(const void* gptr, f16* lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(gptr)
               : "memory", "m0");
}

// Same copy with a wave-uniform 64-bit base (kept in SGPRs) and a 32-bit
// per-lane byte offset: one VGPR per lane instead of a 64-bit address.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, f16* lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff),
               "s"(sbase)
               : "memory", "m0");
}

// dma16s with the LDS destination given as a wave-uniform byte address in
// the LDS aperture (lds_addr(...) of a __shared__ object plus an offset), so
// no generic pointer is formed.
__device__ __forceinline__ void dma16s_at(const void* sbase, uint32_t voff, uint32_t lds_byte) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff),
               "s"(sbase)
               : "memory", "m0");
}

// Byte address of a __shared__ object in the LDS aperture.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 4-byte-per-lane variant (global_load_lds_dword): lane l's dword lands at
// lds_wave_base + 4 l. Same rules as dma16.
__device__ __forceinline__ void dma4(const void* gptr, void* lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(gptr)
               : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight
// and all its LDS operations are done, then barrier. No memory fence is
// emitted (a fence would also wait for the copies still meant to be in
// flight); the asm memory clobber keeps the compiler from moving memory
// accesses across the barrier.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wave-uniform read of a read-only int32 array through the constant address
// space, so it becomes a scalar load (waited for with lgkmcnt). A vector load
// of the same word would be waited for with vmcnt, which also waits for every
// copy and store of the wave still in flight.
__device__ __forceinline__ int32_t load_uniform(const int32_t* a, int i) {
  return ((const __attribute__((address_space(4))) int32_t*)a)[i];
}

// Work-group barrier that orders LDS accesses only: this wave's LDS
// operations complete, then s_barrier. Unlike __syncthreads() it emits no
// vmcnt(0) wait, so global loads, stores and copies still in flight stay in
// flight across it (their consumers wait for them where they are used).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ f32x16 zero_f32x16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// fp64 -> fp16 with a single correct rounding (to nearest even). The value
// is first rounded to fp32; fp16 midpoints are fp32 numbers, so that step
// never moves it across one, and fp32 -> fp16 then rounds correctly unless
// it landed exactly on a midpoint it was not on before (the tie would be
// broken to even instead of by the discarded part). Only then (and in the
// fp16 subnormal range, where the test below does not apply) is the fp32
// value redone with round-to-odd (truncate, set the last bit if anything
// was dropped), after which the fp32 -> fp16 rounding equals a direct one.
__device__ __forceinline__ f16 f64_to_f16_rn(double y) {
  float t = (float)y;
  const uint32_t u = __builtin_bit_cast(uint32_t, t) & 0x7fffffffu;
  if ((u & 0x1fffu) == 0x1000u || u < 0x38800000u) {  // midpoint, or |t| < 2^-14
    if ((double)t != y) {
      uint32_t b = __builtin_bit_cast(uint32_t, t);
      if (__builtin_fabs((double)t) > __builtin_fabs(y)) b -= 1u;  // toward zero
      t = __builtin_bit_cast(float, b | 1u);
    }
  }
  return (f16)t;
}

// Rotary position embedding of one dimension pair (a = dimension j, b =
// dimension j + d/2) by the angle whose cosine and sine are c and s (fp32
// table values; pass -s for the inverse rotation):
//   a' = a c - b s,   b' = b c + a s.
// Products of an fp16 and an fp32 value are exact in fp64 and each fma rounds
// once, so a' and b' are the fp64 values of the formula, rounded once more to
// fp16 by f64_to_f16_rn.
__device__ __forceinline__ void rope_pair(f16& a, f16& b, float c, float s) {
  const double x1 = (double)a, x2 = (double)b, cd = (double)c, sd = (double)s;
  const double y1 = __builtin_fma(x1, cd, -(x2 * sd));
  const double y2 = __builtin_fma(x2, cd, x1 * sd);
  a = f64_to_f16_rn(y1);
  b = f64_to_f16_rn(y2);
}

// The rotation of rope_pair for fp32 inputs (the backward's dq and dk
// accumulators, rotated back with -s), in fp32: each output is one fma over
// one rounded product, then rounded to fp16, so it is within one fp16 unit
// of the correctly rounded value and almost always equal to it. Gradients
// need no bit-exact rotation, and the fp64 form of rope_pair cost the
// backward's epilogues as much as a separate inverse pass.
__device__ __forceinline__ void rope_pair_f32(float x1, float x2, float c, float s, f16& a,
                                              f16& b) {
  a = (f16)__builtin_fmaf(x1, c, -(x2 * s));
  b = (f16)__builtin_fmaf(x2, c, x1 * s);
}

// rope_pair on the 8 pairs (lo[e], hi[e]), e = 0..7, with cosines c0, c1 and
// sines s0, s1 (elements 0-3 and 4-7); sgn = -1 turns the other way (the
// inverse rotation).
__device__ __forceinline__ void rope_rotate8(f16x8& lo, f16x8& hi, f32x4 c0, f32x4 c1, f32x4 s0,
                                             f32x4 s1, float sgn) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    f16 a = lo[e], b = hi[e];
    rope_pair(a, b, e < 4 ? c0[e & 3] : c1[e & 3], sgn * (e < 4 ? s0[e & 3] : s1[e & 3]));
    lo[e] = a;
    hi[e] = b;
  }
}

// The same with the 8 table entries c[e], s[e] read from memory (8
// consecutive fp32 values each, 16-byte aligned).
__device__ __forceinline__ void rope_rotate8(f16x8& lo, f16x8& hi, const float* c,
                                             const float* s, float sgn) {
  rope_rotate8(lo, hi, ((const f32x4*)c)[0], ((const f32x4*)c)[1], ((const f32x4*)s)[0],
               ((const f32x4*)s)[1], sgn);
}

}  // namespace cgqa
