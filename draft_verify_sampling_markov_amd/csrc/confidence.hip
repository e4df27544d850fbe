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
// One workgroup per request, one wave per slot: two dot products with 16-byte
// loads (the hidden state, then the gathered W1 row), a fixed-order wave sum,
// and a float32 running product over the slots in order. The draft's GEMM
// pass can score its slot with the same wave code (conf_logit), which gives the
// same values.
#include "dspark_device.hpp"
#include "dspark_host.hpp"

namespace dspark {

template <bool BF16>
__global__ __launch_bounds__(1024) void confidence_kernel(
    const typename Elem<BF16>::T* __restrict__ h, const typename Elem<BF16>::T* __restrict__ W1,
    const int* __restrict__ anchor, const int* __restrict__ tokens, const float* __restrict__ w,
    float b, const float* __restrict__ inv_temp, int gamma, int d, int V, int r, bool vec_h,
    bool vec_w1, float* __restrict__ conf, float* __restrict__ surv, float* __restrict__ logit) {
  typedef typename Elem<BF16>::T T;
  __shared__ float cs[kMaxGamma];
  const int req = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1), k = 1 + threadIdx.x / kWave;  // one wave per slot
  if (k <= gamma) {
    const int prev = clamp_token(k == 1 ? anchor[req] : tokens[(size_t)req * gamma + k - 2], V);
    float z = conf_logit<BF16>(h + ((size_t)req * gamma + (k - 1)) * d, W1 + (size_t)prev * r, w,
                               b, d, r, vec_h, vec_w1, lane);
    if (logit != nullptr && lane == 0) logit[(size_t)req * gamma + k - 1] = z;
    if (inv_temp) z *= inv_temp[k - 1];
    if (lane == 0) cs[k - 1] = 1.0f / (1.0f + __expf(-z));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = 1.0f;
    for (int kk = 0; kk < gamma; ++kk) {
      a *= cs[kk];
      conf[(size_t)req * gamma + kk] = cs[kk];
      surv[(size_t)req * gamma + kk] = a;
    }
  }
}

}  // namespace dspark

using namespace dspark;

void dspark::confidence_vec_flags(const void* h, const void* W1, const float* w, int d, int r,
                                  int dtype, bool& vec_h, bool& vec_w1) {
  const int vec = dtype == DSPARK_BF16 ? 8 : 4;
  const bool al_h = (reinterpret_cast<uintptr_t>(h) % 16) == 0;
  const bool al_w1 = (reinterpret_cast<uintptr_t>(W1) % 16) == 0;
  const bool al_w = (reinterpret_cast<uintptr_t>(w) % 16) == 0;
  // the weight is read in vector-width groups starting at 0 and at d
  vec_h = al_h && al_w && d % vec == 0;
  vec_w1 = al_w1 && al_w && r % vec == 0 && (d * 4) % 16 == 0;
}

extern "C" int dspark_confidence(const void* h, const void* W1, const int32_t* anchor,
                                 const int32_t* tokens, const float* w, float b,
                                 const float* inv_temp, int R, int gamma, int d, int V, int r,
                                 int dtype, float* conf, float* surv, float* logit,
                                 void* stream) {
  int st = check_sizes(R, gamma, V, r, dtype);
  if (st) return st;
  if (d < 1) return DSPARK_ESIZE;
  if (!h || !W1 || !anchor || !tokens || !w || !conf || !surv) return DSPARK_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool vec_h, vec_w1;
  confidence_vec_flags(h, W1, w, d, r, dtype, vec_h, vec_w1);
  const dim3 block(gamma * kWave);
  if (dtype == DSPARK_BF16)
    hipLaunchKernelGGL(confidence_kernel<true>, dim3(R), block, 0, s,
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(W1), anchor,
                       tokens, w, b, inv_temp, gamma, d, V, r, vec_h, vec_w1, conf, surv, logit);
  else
    hipLaunchKernelGGL(confidence_kernel<false>, dim3(R), block, 0, s,
                       static_cast<const float*>(h), static_cast<const float*>(W1), anchor, tokens,
                       w, b, inv_temp, gamma, d, V, r, vec_h, vec_w1, conf, surv, logit);
  return launch_status();
}
