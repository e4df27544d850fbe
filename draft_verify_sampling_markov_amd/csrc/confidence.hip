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
// and a float32 running product over the slots in order.
#include "dspark_device.hpp"
#include "dspark_host.hpp"

namespace dspark {

// Dot product of `len` stored elements with float weights, by one wave: 16-byte
// loads when `vec` (len a multiple of the vector width, rows aligned), all of a
// lane's loads issued before the sums.
template <bool BF16>
__device__ __forceinline__ float wave_dot(const typename Elem<BF16>::T* __restrict__ x,
                                          const float* __restrict__ w, int len, bool vec, int lane) {
  constexpr int VEC = Elem<BF16>::kVec;
  float acc = 0.0f;
  if (vec) {
    const int nv = len / VEC;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    constexpr int U = 4;
    for (int base = 0; base < nv; base += U * kWave) {
      u32x4 q[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int c = base + i * kWave + lane;
        q[i] = c < nv ? xv[c] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int c = base + i * kWave + lane;
        if (c < nv) {
          const float* wc = w + c * VEC;
          if constexpr (BF16) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc += __uint_as_float(q[i][e] << 16) * wc[2 * e];
              acc += __uint_as_float(q[i][e] & 0xFFFF0000u) * wc[2 * e + 1];
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc += __uint_as_float(q[i][e]) * wc[e];
          }
        }
      }
    }
  } else {
    for (int i = lane; i < len; i += kWave) acc += to_f32(x[i]) * w[i];
  }
  return wave_sum(acc);
}

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
    const float zh = wave_dot<BF16>(h + ((size_t)req * gamma + (k - 1)) * d, w, d, vec_h, lane);
    const float ze = wave_dot<BF16>(W1 + (size_t)prev * r, w + d, r, vec_w1, lane);
    float z = zh + ze + b;
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
  const int vec = dtype == DSPARK_BF16 ? 8 : 4;
  const bool al_h = (reinterpret_cast<uintptr_t>(h) % 16) == 0;
  const bool al_w1 = (reinterpret_cast<uintptr_t>(W1) % 16) == 0;
  const bool al_w = (reinterpret_cast<uintptr_t>(w) % 16) == 0;
  // the weight is read in vector-width groups starting at 0 and at d
  const bool vec_h = al_h && al_w && d % vec == 0;
  const bool vec_w1 = al_w1 && al_w && r % vec == 0 && (d * 4) % 16 == 0;
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
