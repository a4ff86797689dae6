// probe_peaks.hip -- measurement kernels for the second roofline denominator
// (measured peaks next to the published ones). Built into libattn_probe.so,
// which only the benchmark loads; the attention library does not contain or
// call them.
//
//   probe_mfma_f16    independent chains of v_mfma_f32_32x32x16_f16 from
//                     register operands: the dense fp16 MFMA rate this chip
//                     sustains, and the shader clock during that load
//                     (s_memtime against the constant 100 MHz s_memrealtime).
//   probe_stream_read 16-byte non-temporal loads over a large buffer: the HBM
//                     streaming-read rate.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;
constexpr int kMfmaThreads = 256;
constexpr int kReadThreads = 256;

__global__ __launch_bounds__(kMfmaThreads) void mfma_kernel(int iters, float* out,
                                                            unsigned long long* clocks) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (f16)(0.001f * (lane + e));
    b[e] = (f16)(0.002f * (lane - e));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  }
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  unsigned long long t0 = 0, r0 = 0;
  if (timer) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  }
  out[blockIdx.x * kMfmaThreads + threadIdx.x] = s;
  if (timer) {
    clocks[0] = __builtin_amdgcn_s_memtime() - t0;
    clocks[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

// Each wave reads 64 kU consecutive 16-byte pieces per step (lane l, piece
// u at 64 u + l of the wave's span), waves striding over the buffer.
__global__ __launch_bounds__(kReadThreads) void read_kernel(const u32x4* __restrict__ buf,
                                                            size_t n16, uint32_t* out) {
  constexpr int kU = 8;  // loads in flight per thread
  const int lane = threadIdx.x & 63;
  const size_t n_waves = (size_t)gridDim.x * (kReadThreads / 64);
  size_t w = (size_t)blockIdx.x * (kReadThreads / 64) + (threadIdx.x >> 6);
  uint32_t x = 0;
  for (; (w + 1) * 64 * kU <= n16; w += n_waves) {
    const u32x4* p = buf + w * 64 * kU + lane;
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = __builtin_nontemporal_load(p + 64 * u);
#pragma unroll
    for (int u = 0; u < kU; ++u) x ^= v[u].x ^ v[u].w;
  }
  // The tail (fewer than 64 kU pieces) is read piece by piece by wave 0.
  if (blockIdx.x == 0 && threadIdx.x < 64) {
    for (size_t i = (n16 / (64 * kU)) * 64 * kU + lane; i < n16; i += 64)
      x ^= __builtin_nontemporal_load(buf + i).x;
  }
  out[blockIdx.x * kReadThreads + threadIdx.x] = x;
}

}  // namespace

extern "C" {

// FLOPs of one probe_mfma_f16 launch.
double probe_mfma_flops(int n_wg, int iters) {
  return (double)n_wg * (kMfmaThreads / 64) * iters * kChains * 32.0 * 32.0 * 16.0 * 2.0;
}

// n_wg work-groups of 4 waves, each wave kChains chains of `iters` MFMAs.
// out: float [n_wg * 256] (device); clocks: uint64 [2] (device): shader
// clock ticks and 100 MHz ticks of work-group 0. Returns 0 or a HIP error.
int probe_mfma_f16(int n_wg, int iters, float* out, unsigned long long* clocks, void* stream) {
  if (n_wg <= 0 || iters <= 0 || !out || !clocks) return -1;
  hipLaunchKernelGGL(mfma_kernel, dim3(n_wg), dim3(kMfmaThreads), 0, (hipStream_t)stream, iters,
                     out, clocks);
  return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 16) of `buf` once; out: uint32 [n_wg * 256].
int probe_stream_read(const void* buf, size_t bytes, int n_wg, uint32_t* out, void* stream) {
  if (!buf || bytes < 16 || (bytes & 15) || n_wg <= 0 || !out) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(n_wg), dim3(kReadThreads), 0, (hipStream_t)stream,
                     (const u32x4*)buf, bytes / 16, out);
  return (int)hipGetLastError();
}

}  // extern "C"
