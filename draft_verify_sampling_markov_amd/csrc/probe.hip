// Peak probes for the measurement, not part of the method: a streaming read
// and a matrix-core loop, so that the bench can report the bandwidth and the
// bf16 matrix rate this GPU actually reaches beside the published peaks
// (8 TB/s HBM, 2.5 PFLOP/s dense bf16) that the rooflines are priced against.
//
//   read: a grid-stride sweep of 16-byte nontemporal loads over a buffer,
//         four loads in flight per lane, folded into one word that is stored
//         only if it equals a constant the sweep never produces (the loads
//         cannot be dropped);
//   mfma: each wave runs `iters` rounds of eight independent
//         v_mfma_f32_16x16x32_bf16 (16 x 16 x 32, 16384 FLOP each), the
//         accumulators folded and stored the same way.
#include "dspark_device.hpp"
#include "dspark_host.hpp"

namespace dspark {
namespace {

constexpr int kProbeReadThreads = 512;
constexpr int kProbeMfmaThreads = 256;
constexpr int kProbeMfmaChains = 8;

__global__ __launch_bounds__(kProbeReadThreads) void probe_read_kernel(
    const u32x4* __restrict__ src, size_t n, unsigned* __restrict__ sink) {
  unsigned acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a[0] ^ b[1] ^ c[2] ^ d[3];
  }
  for (; i < n; i += stride) acc ^= src[i][0];
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ __launch_bounds__(kProbeMfmaThreads) void probe_mfma_kernel(float* __restrict__ sink,
                                                                      int iters) {
  const int lane = threadIdx.x & (kWave - 1);
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1.0f + 0.001f * (float)(lane + e));
    b[e] = (__bf16)(0.5f - 0.001f * (float)(lane ^ e));
  }
  f32x4 acc[kProbeMfmaChains];
#pragma unroll
  for (int j = 0; j < kProbeMfmaChains; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeMfmaChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kProbeMfmaChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (s == 1234.5f) sink[threadIdx.x] = s;
}

}  // namespace
}  // namespace dspark

using namespace dspark;

extern "C" int dspark_probe_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return DSPARK_EINVAL;
  if (bytes < 16 || (bytes % 16) != 0 || (reinterpret_cast<uintptr_t>(src) % 16) != 0)
    return DSPARK_ESIZE;
  const int grid = 4 * device_cu_count();
  hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(kProbeReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), bytes / 16,
                     static_cast<unsigned*>(sink));
  return launch_status();
}

extern "C" int dspark_probe_mfma(void* sink, int grid, int iters, void* stream) {
  if (!sink) return DSPARK_EINVAL;
  if (grid < 1 || grid > (1 << 16) || iters < 1) return DSPARK_ESIZE;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(grid), dim3(kProbeMfmaThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<float*>(sink), iters);
  return launch_status();
}

extern "C" double dspark_probe_mfma_flops(int grid, int iters) {
  return (double)grid * (kProbeMfmaThreads / kWave) * (double)iters * kProbeMfmaChains * 16384.0;
}
