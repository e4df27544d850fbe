// Sequential temperature scaling of the confidence head, fitted on the GPU.
//
// DSpark digest ("DSpark: Confidence-Scheduled Speculative Decoding with
// Semi-Autoregressive Generation", zhao9797.github.io), "Verification
// scheduling (system side)": neural confidences are over-confident while the
// scheduler needs their absolute size, so each position gets a temperature,
// fitted left to right on the running products prod_{i<=k} c_i by a
// one-dimensional grid search that minimises the expected calibration error;
// a positive temperature keeps the ranking.
//
// Per position k three launches:
//   curve   grid (slices of the samples) x (candidates): each workgroup adds
//           its samples' pairs (a_k = a_{k-1} sigmoid(z_k beta_j), label y_k)
//           to the candidate's bins in LDS, then to the candidate's bins in
//           the workspace -- integer counts and fixed-point sums, so the
//           totals do not depend on the order of accumulation;
//   pick    one workgroup: ECE of every candidate from its bins, the first
//           minimiser, the bins cleared for the next position;
//   advance a_k of every sample with the chosen beta.
// a_k is formed exactly as the confidence kernel forms it (float32,
// 1 / (1 + exp(-z beta)) then the running product), so the fitted values
// reproduce on the chain.
#include "dspark_device.hpp"
#include "dspark_host.hpp"

#include <algorithm>

namespace dspark {

constexpr int kStsMaxGrid = 256;
constexpr int kStsMaxBins = 32;
constexpr int kStsThreads = 256;
constexpr int kStsSliceSamples = 4096;  // samples per curve workgroup

__device__ __forceinline__ float sts_sigmoid(float z) { return 1.0f / (1.0f + __expf(-z)); }

__device__ __forceinline__ int sts_bin(float p, int n_bins) {
  const double q = (double)fminf(fmaxf(p, 0.0f), 1.0f) * (double)n_bins;  // exact
  return min((int)floor(q), n_bins - 1);
}

__device__ __forceinline__ unsigned long long sts_fixed(float p) {
  return (unsigned long long)floor((double)fminf(fmaxf(p, 0.0f), 1.0f) * 4294967296.0);
}

__global__ __launch_bounds__(kStsThreads) void sts_init_kernel(float* __restrict__ a_prev, int N,
                                                               unsigned long long* __restrict__ bins,
                                                               int n_words) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N) a_prev[i] = 1.0f;
  if (i < n_words) bins[i] = 0ull;
}

// bins layout: [n_grid][n_bins][3] = (count, sum of a * 2^32, sum of y * 2^32)
__global__ __launch_bounds__(kStsThreads) void sts_curve_kernel(
    const float* __restrict__ z, const float* __restrict__ y, const unsigned char* __restrict__ mask,
    const float* __restrict__ a_prev, const float* __restrict__ betas, int N, int gamma, int k,
    int n_bins, unsigned long long* __restrict__ bins) {
  __shared__ unsigned long long lb[kStsMaxBins * 3];
  const int j = blockIdx.y, tid = threadIdx.x;
  for (int i = tid; i < n_bins * 3; i += kStsThreads) lb[i] = 0ull;
  __syncthreads();
  const float beta = betas[j];
  const int n0 = blockIdx.x * kStsSliceSamples;
  const int n1 = min(N, n0 + kStsSliceSamples);
  for (int n = n0 + tid; n < n1; n += kStsThreads) {
    const size_t e = (size_t)n * gamma + k;
    if (mask != nullptr && mask[e] == 0) continue;
    const float a = a_prev[n] * sts_sigmoid(z[e] * beta);
    const int b = sts_bin(a, n_bins);
    atomicAdd(&lb[b * 3], 1ull);
    atomicAdd(&lb[b * 3 + 1], sts_fixed(a));
    atomicAdd(&lb[b * 3 + 2], sts_fixed(y[e]));
  }
  __syncthreads();
  for (int i = tid; i < n_bins * 3; i += kStsThreads)
    if (lb[i] != 0ull) atomicAdd(&bins[(size_t)j * n_bins * 3 + i], lb[i]);
}

__global__ __launch_bounds__(kStsThreads) void sts_pick_kernel(
    const float* __restrict__ betas, int n_grid, int n_bins, int k,
    unsigned long long* __restrict__ bins, float* __restrict__ inv_temp,
    float* __restrict__ ece_out) {
  __shared__ double ece_s[kStsMaxGrid];
  const int tid = threadIdx.x;
  for (int j = tid; j < n_grid; j += kStsThreads) {
    const unsigned long long* bj = bins + (size_t)j * n_bins * 3;
    unsigned long long cnt = 0ull;
    double err = 0.0;
    for (int b = 0; b < n_bins; ++b) {
      cnt += bj[b * 3];
      const double d = (double)(long long)(bj[b * 3 + 1] - bj[b * 3 + 2]);  // two's complement
      err += fabs(d);
    }
    const double e = cnt ? err / 4294967296.0 / (double)cnt : (double)__builtin_nan("");
    ece_s[j] = e;
    ece_out[(size_t)k * n_grid + j] = (float)e;
  }
  __syncthreads();
  if (tid == 0) {
    int best = 0;
    for (int j = 1; j < n_grid; ++j)
      if (ece_s[j] < ece_s[best]) best = j;  // first minimiser (NaN never wins)
    inv_temp[k] = betas[best];
  }
  __syncthreads();
  for (int i = tid; i < n_grid * n_bins * 3; i += kStsThreads) bins[i] = 0ull;
}

__global__ __launch_bounds__(kStsThreads) void sts_advance_kernel(
    const float* __restrict__ z, float* __restrict__ a_prev, const float* __restrict__ inv_temp,
    int N, int gamma, int k) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n < N) a_prev[n] = a_prev[n] * sts_sigmoid(z[(size_t)n * gamma + k] * inv_temp[k]);
}

size_t sts_ws_bytes(int N, int n_grid, int n_bins) {
  return align_up((size_t)N * 4, 256) + (size_t)n_grid * n_bins * 3 * 8;
}

}  // namespace dspark

using namespace dspark;

extern "C" size_t dspark_sts_workspace_bytes(int N, int gamma, int n_grid, int n_bins) {
  if (N < 1 || gamma < 1 || gamma > kMaxGamma || n_grid < 1 || n_grid > kStsMaxGrid ||
      n_bins < 1 || n_bins > kStsMaxBins)
    return 0;
  if ((long long)N * gamma > (1ll << 31)) return 0;
  return sts_ws_bytes(N, n_grid, n_bins);
}

extern "C" int dspark_sts_fit(const float* z, const float* y, const uint8_t* mask, int N,
                              int gamma, const float* betas, int n_grid, int n_bins,
                              float* inv_temp, float* ece, void* ws, size_t ws_bytes,
                              void* stream) {
  const size_t need = dspark_sts_workspace_bytes(N, gamma, n_grid, n_bins);
  if (need == 0) return DSPARK_ESIZE;
  if (!z || !y || !betas || !inv_temp || !ece) return DSPARK_EINVAL;
  if (!ws || ws_bytes < need) return DSPARK_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* a_prev = static_cast<float*>(ws);
  unsigned long long* bins = reinterpret_cast<unsigned long long*>(
      static_cast<char*>(ws) + align_up((size_t)N * 4, 256));
  const int n_words = n_grid * n_bins * 3;
  hipLaunchKernelGGL(sts_init_kernel, dim3(ceil_div(std::max(N, n_words), kStsThreads)),
                     dim3(kStsThreads), 0, s, a_prev, N, bins, n_words);
  int st = launch_status();
  if (st) return st;
  const dim3 curve_grid(ceil_div(N, kStsSliceSamples), n_grid);
  for (int k = 0; k < gamma; ++k) {
    hipLaunchKernelGGL(sts_curve_kernel, curve_grid, dim3(kStsThreads), 0, s, z, y, mask, a_prev,
                       betas, N, gamma, k, n_bins, bins);
    if ((st = launch_status())) return st;
    hipLaunchKernelGGL(sts_pick_kernel, dim3(1), dim3(kStsThreads), 0, s, betas, n_grid, n_bins, k,
                       bins, inv_temp, ece);
    if ((st = launch_status())) return st;
    hipLaunchKernelGGL(sts_advance_kernel, dim3(ceil_div(N, kStsThreads)), dim3(kStsThreads), 0, s,
                       z, a_prev, inv_temp, N, gamma, k);
    if ((st = launch_status())) return st;
  }
  return DSPARK_OK;
}
