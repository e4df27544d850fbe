// Decode-loop advance: the per-step state update that lets a sequence of chain
// steps run back to back on the device, with no host read-back between them.
//
// After a step's verify, the next step's anchor x_0 is the last token that
// step committed (the correction or bonus token at out_tokens[r, A_r]); the
// Philox step counter moves on by one; and the survivals join a short history
// so that a later step can size its verify budget from confidences one or two
// steps old (DSpark digest, "Infra": the budget comes from confidences two
// steps back, a causal barrier, while candidates are still ranked by the latest
// ones; vLLM adaptive verification with DSpark, "Execution pipeline": the
// budget comes from the previous step's double-buffered confidences).
#include "dspark_device.hpp"
#include "dspark_host.hpp"

#include <algorithm>

namespace dspark {

constexpr int kMaxHist = 8;

// One thread per (request, slot) element of the survival history, and per
// request for the anchor. Thread 0 also advances the step counter. Every
// history element is shifted by one thread, oldest level first, so the copy
// never reads a level it has already overwritten.
__global__ __launch_bounds__(256) void advance_kernel(
    int* __restrict__ anchor, const int* __restrict__ accept_len,
    const int* __restrict__ out_tokens, int R, int gamma, uint64_t* __restrict__ step_dev,
    float* __restrict__ hist, const float* __restrict__ surv, int n_hist) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < R) {
    const int A = min(max(accept_len[i], 0), gamma);
    anchor[i] = out_tokens[(size_t)i * (gamma + 1) + A];
  }
  if (i == 0 && step_dev != nullptr) step_dev[0] = step_dev[0] + 1ull;
  const int n = R * gamma;
  if (n_hist > 0 && i < n) {
    for (int h = n_hist - 1; h > 0; --h) hist[(size_t)h * n + i] = hist[(size_t)(h - 1) * n + i];
    hist[i] = surv[i];
  }
}

}  // namespace dspark

using namespace dspark;

extern "C" int dspark_advance(int32_t* anchor, const int32_t* accept_len,
                              const int32_t* out_tokens, int R, int gamma, uint64_t* step_dev,
                              float* surv_hist, const float* surv, int n_hist, void* stream) {
  if (R < 1 || gamma < 1 || gamma > kMaxGamma || (long long)R * (gamma + 1) > kMaxRows)
    return DSPARK_ESIZE;
  if (n_hist < 0 || n_hist > kMaxHist) return DSPARK_ESIZE;
  if (!anchor || !accept_len || !out_tokens) return DSPARK_EINVAL;
  if (n_hist > 0 && (!surv_hist || !surv)) return DSPARK_EINVAL;
  const int n = std::max(R, n_hist > 0 ? R * gamma : 0);
  hipLaunchKernelGGL(advance_kernel, dim3(ceil_div(n, 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), anchor, accept_len, out_tokens, R, gamma,
                     step_dev, surv_hist, surv, n_hist);
  return launch_status();
}
