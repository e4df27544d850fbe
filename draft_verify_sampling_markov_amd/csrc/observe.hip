// Observability accumulator: per-step acceptance, ceiling, window and
// calibration counts summed into a device block, so that a decode loop (or a
// captured graph of it) can keep its metrics without reading anything back
// per step.
//
// SGLang DSpark blog, "Observability": a cap-accept run commits what compact
// commits while exposing the ceiling a full-block verification would reach,
// and the engine reports per-request confidence and calibration (ECE); its
// "Per-request differentiation on mixed traffic" reports windows and the
// utilisation against the ceiling. DSpark digest, "Verification scheduling
// (system side)": the confidence c_k is the probability that slot k passes
// given an accepted prefix, and temperature scaling calibrates the running
// products per position.
//
// Every quantity is an integer (probabilities enter as floor(p * 2^32)), so
// the totals are exact and do not depend on the order of accumulation. One
// workgroup: per-request rows are updated by their own thread, the shared
// counts are gathered in LDS and added to the block once.
#include "dspark_device.hpp"
#include "dspark_host.hpp"

namespace dspark {

constexpr int kObsThreads = 1024;
constexpr int kObsMaxBins = 32;
constexpr int kObsHeader = 8;
constexpr int kObsMaxCells = 2 * kMaxGamma * kObsMaxBins * 3;

struct ObsLayout {
  int hist, req, bins, words;
};

__host__ __device__ inline ObsLayout obs_layout(int R, int gamma, int n_bins) {
  ObsLayout L;
  L.hist = kObsHeader;
  L.req = L.hist + 3 * (gamma + 1);
  L.bins = L.req + 3 * R;
  L.words = L.bins + 2 * gamma * n_bins * 3;
  return L;
}

__device__ __forceinline__ int obs_bin(float p, int n_bins) {
  if (!(p == p)) return 0;  // NaN
  const double q = (double)fminf(fmaxf(p, 0.0f), 1.0f) * (double)n_bins;  // exact
  return min((int)floor(q), n_bins - 1);
}

__device__ __forceinline__ unsigned long long obs_scaled(float p) {
  if (!(p == p)) return 0ull;
  const double q = (double)fminf(fmaxf(p, 0.0f), 1.0f) * 4294967296.0;  // exact
  return (unsigned long long)floor(q);
}

__device__ __forceinline__ void lds_add(unsigned long long* a, unsigned long long v) {
  atomicAdd(a, v);
}

__global__ __launch_bounds__(kObsThreads) void observe_kernel(
    const float* __restrict__ conf, const float* __restrict__ surv,
    const int* __restrict__ win_len, const int* __restrict__ accept_len,
    const int* __restrict__ ceiling_len, const int* __restrict__ cu_seqlens, int R, int gamma,
    int n_bins, unsigned long long* __restrict__ stats) {
  __shared__ unsigned long long head[kObsHeader];
  __shared__ unsigned long long hist[3 * (kMaxGamma + 1)];
  __shared__ unsigned long long cells[kObsMaxCells];
  const ObsLayout L = obs_layout(R, gamma, n_bins);
  const int tid = threadIdx.x;
  const int n_hist = 3 * (gamma + 1), n_cells = 2 * gamma * n_bins * 3;
  for (int i = tid; i < kObsHeader; i += kObsThreads) head[i] = 0ull;
  for (int i = tid; i < n_hist; i += kObsThreads) hist[i] = 0ull;
  for (int i = tid; i < n_cells; i += kObsThreads) cells[i] = 0ull;
  __syncthreads();
  for (int r = tid; r < R; r += kObsThreads) {
    const int A = min(max(accept_len[r], 0), gamma);
    const int C = min(max(ceiling_len[r], 0), gamma);
    const int Lw = min(max(win_len[r], 0), gamma);
    const int Lv = min(max(cu_seqlens[r + 1] - cu_seqlens[r] - 1, 0), gamma);
    lds_add(&head[2], (unsigned long long)(A + 1));
    lds_add(&head[3], (unsigned long long)A);
    lds_add(&head[4], (unsigned long long)C);
    lds_add(&head[5], (unsigned long long)Lw);
    lds_add(&head[6], (unsigned long long)Lv);
    lds_add(&hist[Lw], 1ull);
    lds_add(&hist[(gamma + 1) + A], 1ull);
    lds_add(&hist[2 * (gamma + 1) + C], 1ull);
    stats[L.req + r] += (unsigned long long)A;
    stats[L.req + R + r] += (unsigned long long)C;
    stats[L.req + 2 * R + r] += (unsigned long long)Lw;
    for (int k = 1; k <= gamma; ++k) {
      if (k <= min(C + 1, Lv)) {  // conditional: c_k against slot k accepted
        const float p = conf[(size_t)r * gamma + k - 1];
        unsigned long long* cell = &cells[((0 * gamma + (k - 1)) * n_bins + obs_bin(p, n_bins)) * 3];
        lds_add(cell, 1ull);
        lds_add(cell + 1, obs_scaled(p));
        lds_add(cell + 2, k <= C ? 1ull : 0ull);
      }
      if (k <= Lv) {  // prefix: a_k against the whole prefix accepted
        const float p = surv[(size_t)r * gamma + k - 1];
        unsigned long long* cell = &cells[((1 * gamma + (k - 1)) * n_bins + obs_bin(p, n_bins)) * 3];
        lds_add(cell, 1ull);
        lds_add(cell + 1, obs_scaled(p));
        lds_add(cell + 2, C >= k ? 1ull : 0ull);
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    stats[0] += 1ull;
    stats[1] += (unsigned long long)R;
  }
  for (int i = tid; i < 5; i += kObsThreads) stats[2 + i] += head[2 + i];
  for (int i = tid; i < n_hist; i += kObsThreads) stats[L.hist + i] += hist[i];
  for (int i = tid; i < n_cells; i += kObsThreads) stats[L.bins + i] += cells[i];
}

}  // namespace dspark

using namespace dspark;

extern "C" size_t dspark_observe_words(int R, int gamma, int n_bins) {
  if (R < 1 || gamma < 1 || gamma > kMaxGamma || n_bins < 1 || n_bins > kObsMaxBins) return 0;
  if ((long long)R * (gamma + 1) > kMaxRows) return 0;
  return (size_t)obs_layout(R, gamma, n_bins).words;
}

extern "C" int dspark_observe(const float* conf, const float* surv, const int32_t* win_len,
                              const int32_t* accept_len, const int32_t* ceiling_len,
                              const int32_t* cu_seqlens, int R, int gamma, int n_bins,
                              uint64_t* stats, size_t stats_words, void* stream) {
  const size_t need = dspark_observe_words(R, gamma, n_bins);
  if (need == 0) return DSPARK_ESIZE;
  if (!conf || !surv || !win_len || !accept_len || !ceiling_len || !cu_seqlens || !stats)
    return DSPARK_EINVAL;
  if (stats_words < need) return DSPARK_EWORKSPACE;
  hipLaunchKernelGGL(observe_kernel, dim3(1), dim3(kObsThreads), 0, static_cast<hipStream_t>(stream),
                     conf, surv, win_len, accept_len, ceiling_len, cu_seqlens, R, gamma, n_bins,
                     reinterpret_cast<unsigned long long*>(stats));
  return launch_status();
}
