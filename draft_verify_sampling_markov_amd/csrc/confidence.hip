// Confidence head and prefix survival on gfx950.
//
// DSpark digest ("DSpark: Confidence-Scheduled Speculative Decoding with
// Semi-Autoregressive Generation", zhao9797.github.io), section "Verification
// scheduling (system side)": c_k is a sigmoid of a linear projection of
// [h_k ; W1[x_{k-1}]] and estimates the chance that draft k passes given an
// accepted prefix; the prefix survival is the running product
// a_{r,j} = prod_{i <= j} c_{r,i}, so it never grows with j. An optional
// per-position inverse temperature scales the logit (the digest's sequential
// temperature scaling calibrates per position; the pages give no formula).
//
// One workgroup per request, one wave per slot: two coalesced dot products
// (the hidden state, then the gathered W1 row), a fixed-order wave sum, and a
// float32 running product over the slots in order.
#include "dspark_device.hpp"
#include "dspark_host.hpp"

namespace dspark {

template <bool BF16>
__global__ __launch_bounds__(256) void confidence_kernel(
    const typename Elem<BF16>::T* __restrict__ h, const typename Elem<BF16>::T* __restrict__ W1,
    const int* __restrict__ anchor, const int* __restrict__ tokens, const float* __restrict__ w,
    float b, const float* __restrict__ inv_temp, int gamma, int d, int V, int r,
    float* __restrict__ conf, float* __restrict__ surv) {
  typedef typename Elem<BF16>::T T;
  __shared__ float cs[kMaxGamma];
  const int req = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  for (int k = 1 + wave; k <= gamma; k += nwaves) {
    const int prev = clamp_token(k == 1 ? anchor[req] : tokens[(size_t)req * gamma + k - 2], V);
    const T* hk = h + ((size_t)req * gamma + (k - 1)) * d;
    const T* e = W1 + (size_t)prev * r;
    float acc = 0.0f;
    for (int i = lane; i < d; i += kWave) acc += to_f32(hk[i]) * w[i];
    for (int i = lane; i < r; i += kWave) acc += to_f32(e[i]) * w[d + i];
    acc = wave_sum(acc);
    float z = acc + b;
    if (inv_temp) z *= inv_temp[k - 1];
    if (lane == 0) cs[k - 1] = 1.0f / (1.0f + __expf(-z));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = 1.0f;
    for (int k = 0; k < gamma; ++k) {
      a *= cs[k];
      conf[(size_t)req * gamma + k] = cs[k];
      surv[(size_t)req * gamma + k] = a;
    }
  }
}

}  // namespace dspark

using namespace dspark;

extern "C" int dspark_confidence(const void* h, const void* W1, const int32_t* anchor,
                                 const int32_t* tokens, const float* w, float b,
                                 const float* inv_temp, int R, int gamma, int d, int V, int r,
                                 int dtype, float* conf, float* surv, void* stream) {
  int st = check_sizes(R, gamma, V, r, dtype);
  if (st) return st;
  if (d < 1) return DSPARK_ESIZE;
  if (!h || !W1 || !anchor || !tokens || !w || !conf || !surv) return DSPARK_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == DSPARK_BF16)
    hipLaunchKernelGGL(confidence_kernel<true>, dim3(R), dim3(256), 0, s,
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(W1), anchor,
                       tokens, w, b, inv_temp, gamma, d, V, r, conf, surv);
  else
    hipLaunchKernelGGL(confidence_kernel<false>, dim3(R), dim3(256), 0, s,
                       static_cast<const float*>(h), static_cast<const float*>(W1), anchor, tokens,
                       w, b, inv_temp, gamma, d, V, r, conf, surv);
  return launch_status();
}
