// Global top-B prefix scheduler and ragged pack on gfx950, plus the host
// cost-table preparation.
//
// Scheduler -- DSpark digest ("DSpark: Confidence-Scheduled Speculative
// Decoding with Semi-Autoregressive Generation", zhao9797.github.io):
// "Verification scheduling (system side)" maximises Theta = tau * SPS over
// global, survival-ordered admission with an O(1) table read and an early
// stop; "Infra (online production @ DeepSeek-V4)" drops the early stop when the
// budget comes from older confidences, while the current slots are still ranked
// by the newest survivals. vLLM adaptive verification page ("DSpark
// confidence-scheduling mechanism"): global top-B across requests, each
// request keeping a contiguous prefix; slot assignment stays on the GPU so the
// host never reads back. SGLang DSpark blog ("Cost-table profiling"): the cost
// is read at M = bs + K verify tokens.
//
// Everything is integer fixed point (survival quantised to 2^-20, Theta as a
// uint64 product), so the result does not depend on the order in which the
// workgroup's threads combine it. One workgroup: quantise, sort the R*gamma
// keys in LDS (rank counting up to one key per thread, a bitonic network
// beyond), integer prefix sums, Theta per K, reduction, window counts.
//
// Pack -- SGLang DSpark blog ("Ragged verify under full CUDA graphs"): windows
// packed front to back into a cu_seqlens buffer, total rounded up to the
// nearest captured tier. One workgroup: exclusive scan of (1 + L_r), then one
// thread per packed row (binary search of its request).
#include "dspark_device.hpp"
#include "dspark_host.hpp"

#include <cmath>

namespace dspark {

constexpr int kSchedThreads = 1024;
constexpr int kSchedMaxKeys = 4096;
constexpr uint32_t kQOne = 1u << 20;

__device__ __forceinline__ uint32_t quantize_survival(float a) {
  if (!(a == a)) return 0u;
  a = fminf(fmaxf(a, 0.0f), 1.0f);
  return (uint32_t)(a * 1048576.0f);  // exact scaling; truncation = floor for a >= 0
}

// keys[i] = ((2^20 - a_q) << 32) | i for i = r*gamma + j, padded to P with ~0.
__device__ void build_keys(const float* __restrict__ a, int R, int gamma, int P,
                           unsigned long long* keys) {
  const int N = R * gamma;
  for (int req = threadIdx.x; req < R; req += blockDim.x) {
    uint32_t run = kQOne;
    for (int j = 0; j < gamma; ++j) {
      const int i = req * gamma + j;
      run = min(run, quantize_survival(a[i]));
      keys[i] = ((unsigned long long)(kQOne - run) << 32) | (unsigned long long)i;
    }
  }
  for (int i = N + threadIdx.x; i < P; i += blockDim.x) keys[i] = ~0ull;
  __syncthreads();
}

__device__ void bitonic_sort(unsigned long long* keys, int P) {
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long x = keys[i], y = keys[ixj];
          const bool up = (i & k) == 0;
          if ((x > y) == up) {
            keys[i] = y;
            keys[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Sort the first N keys ascending. Keys are distinct (they carry their index).
// Up to one key per thread: a key's position is the number of smaller keys,
// counted in one pass over the array (LDS broadcast reads, eight in flight),
// then a scatter through `scratch`. More keys: a bitonic network over the P
// keys (padded with ~0).
__device__ void sort_keys(unsigned long long* keys, unsigned long long* scratch, int N, int P) {
  if (N <= (int)blockDim.x) {
    const int i = threadIdx.x;
    if (i < N) {
      const unsigned long long mine = keys[i];
      int rank = 0;
      const int N8 = N & ~7;
      for (int j = 0; j < N8; j += 8) {
        unsigned long long kj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kj[u] = keys[j + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) rank += kj[u] < mine;
      }
      for (int j = N8; j < N; ++j) rank += keys[j] < mine;
      scratch[rank] = mine;
    }
    __syncthreads();
    if (i < N) keys[i] = scratch[i];
    __syncthreads();
  } else {
    bitonic_sort(keys, P);
  }
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(
    const float* __restrict__ surv, const float* __restrict__ surv_budget,
    const uint32_t* __restrict__ sps, int M_max, int R, int gamma, int B_cap, int mode, int K_fixed,
    int* __restrict__ win_len, int* __restrict__ K_out) {
  __shared__ unsigned long long keys[kSchedMaxKeys];
  __shared__ unsigned long long sort_scratch[kSchedMaxKeys];
  // inclusive prefix of the sorted a_q, then window counts: reuses the sort
  // scratch, which is dead once the sorted keys are back in `keys`
  uint32_t* pre = reinterpret_cast<uint32_t*>(sort_scratch);
  __shared__ uint32_t wtot[kSchedThreads / kWave];
  __shared__ unsigned long long red_theta[kSchedThreads / kWave];
  __shared__ int red_k[kSchedThreads / kWave];
  __shared__ int K_sh;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int nw = blockDim.x / kWave;
  const int N = R * gamma;
  int P = 1;
  while (P < N) P <<= 1;
  const int K_cap = max(0, min(min(B_cap, N), M_max - R));

  int K = 0;
  if (mode == DSPARK_SCHED_FIXED) {
    K = min(max(K_fixed, 0), K_cap);
  } else {
    // this thread's cost-table entries, fetched before the sort so the load
    // overlaps it: sps[R + Kc] and sps[R + Kc + 1] for Kc = tid + i * threads
    constexpr int kMaxPer = kSchedMaxKeys / kSchedThreads + 1;
    uint32_t sp0[kMaxPer], sp1[kMaxPer];
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int Kc = tid + i * (int)blockDim.x;
      sp0[i] = Kc <= K_cap ? sps[R + Kc] : 0u;
      sp1[i] = Kc < K_cap ? sps[R + Kc + 1] : 0u;
    }
    build_keys(surv_budget ? surv_budget : surv, R, gamma, P, keys);
    sort_keys(keys, sort_scratch, N, P);
    // inclusive prefix sums of the sorted a_q (each thread: 4 consecutive keys)
    const int per = (P + blockDim.x - 1) / blockDim.x;
    const int b0 = tid * per;
    uint32_t local = 0;
    for (int i = b0; i < min(b0 + per, N); ++i) local += kQOne - (uint32_t)(keys[i] >> 32);
    uint32_t incl = local;
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t t = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) wtot[wave] = incl;
    __syncthreads();
    uint32_t woff = 0;
    for (int w = 0; w < wave; ++w) woff += wtot[w];
    uint32_t run = woff + incl - local;
    for (int i = b0; i < min(b0 + per, N); ++i) {
      run += kQOne - (uint32_t)(keys[i] >> 32);
      pre[i] = run;
    }
    __syncthreads();
    const unsigned long long base = (unsigned long long)R * kQOne;
    // Theta_K = tau_K * sps[R + K], tau_K = R*2^20 + pre[K-1]
    unsigned long long best_t = 0;
    int best_k = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int Kc = tid + i * (int)blockDim.x;
      if (Kc > K_cap) continue;
      const unsigned long long tau = base + (Kc ? pre[Kc - 1] : 0u);
      const unsigned long long th = tau * (unsigned long long)sp0[i];
      if (mode == DSPARK_SCHED_ARGMAX) {
        if (best_k == 0x7fffffff || th > best_t) {
          best_t = th;
          best_k = Kc;
        }
      } else if (Kc < K_cap) {  // GREEDY: first K with Theta_{K+1} <= Theta_K
        const unsigned long long tau1 = base + pre[Kc];
        const unsigned long long th1 = tau1 * (unsigned long long)sp1[i];
        if (th1 <= th && Kc < best_k) best_k = Kc;
      }
    }
    // reduce: ARGMAX -> (largest Theta, then smallest K); GREEDY -> smallest K
    for (int o = kWave / 2; o >= 1; o >>= 1) {
      const unsigned long long ot = __shfl_xor(best_t, o, kWave);
      const int ok = __shfl_xor(best_k, o, kWave);
      if (mode == DSPARK_SCHED_ARGMAX) {
        if (ok != 0x7fffffff && (best_k == 0x7fffffff || ot > best_t || (ot == best_t && ok < best_k))) {
          best_t = ot;
          best_k = ok;
        }
      } else if (ok < best_k) {
        best_k = ok;
      }
    }
    if (lane == 0) {
      red_theta[wave] = best_t;
      red_k[wave] = best_k;
    }
    __syncthreads();
    if (tid == 0) {
      unsigned long long bt = red_theta[0];
      int bk = red_k[0];
      for (int w = 1; w < nw; ++w) {
        if (mode == DSPARK_SCHED_ARGMAX) {
          if (red_k[w] != 0x7fffffff &&
              (bk == 0x7fffffff || red_theta[w] > bt || (red_theta[w] == bt && red_k[w] < bk))) {
            bt = red_theta[w];
            bk = red_k[w];
          }
        } else if (red_k[w] < bk) {
          bk = red_k[w];
        }
      }
      if (mode == DSPARK_SCHED_GREEDY && bk == 0x7fffffff) bk = K_cap;
      if (bk == 0x7fffffff) bk = 0;
      K_sh = bk;
    }
    __syncthreads();
    K = K_sh;
  }

  // selection: the K best keys of the current survivals
  if (mode == DSPARK_SCHED_FIXED || surv_budget != nullptr) {
    build_keys(surv, R, gamma, P, keys);
    sort_keys(keys, sort_scratch, N, P);
  }
  for (int i = tid; i < R; i += blockDim.x) pre[i] = 0u;
  __syncthreads();
  for (int i = tid; i < K; i += blockDim.x) {
    const int idx = (int)(keys[i] & 0xffffffffull);
    atomicAdd(&pre[idx / gamma], 1u);
  }
  __syncthreads();
  for (int i = tid; i < R; i += blockDim.x) win_len[i] = (int)pre[i];
  if (tid == 0) K_out[0] = K;
}

struct TierList {
  int n;
  int v[kMaxTiers];
};

__global__ __launch_bounds__(1024) void pack_kernel(
    const int* __restrict__ anchor, const int* __restrict__ tokens, const int* __restrict__ win_len,
    int R, int gamma, TierList tiers, int M_cap, int* __restrict__ cu_seqlens,
    int* __restrict__ ptok, int* __restrict__ preq, int* __restrict__ pslot,
    int* __restrict__ totals) {
  __shared__ int cu[kMaxRows / 2 + 1];
  __shared__ int wtot[1024 / kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  // requests 2*tid, 2*tid + 1 (R <= 2048)
  int len[2] = {0, 0};
  for (int e = 0; e < 2; ++e) {
    const int req = 2 * tid + e;
    if (req < R) {
      int L = win_len ? win_len[req] : gamma;
      L = min(max(L, 0), gamma);
      len[e] = 1 + L;
    }
  }
  const int local = len[0] + len[1];
  int incl = local;
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) wtot[wave] = incl;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wave; ++w) off += wtot[w];
  const int excl = off + incl - local;
  if (2 * tid < R) cu[2 * tid] = excl;
  if (2 * tid + 1 < R) cu[2 * tid + 1] = excl + len[0];
  if (tid == 0) {
    int tot = 0;
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w) tot += wtot[w];
    cu[R] = tot;
  }
  __syncthreads();
  const int M = cu[R];
  for (int i = tid; i <= R; i += blockDim.x) cu_seqlens[i] = cu[i];
  for (int i = tid; i < M_cap; i += blockDim.x) {
    if (i < M) {
      int lo = 0, hi = R - 1;  // last request with cu[req] <= i
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= i) lo = mid; else hi = mid - 1;
      }
      const int j = i - cu[lo];
      ptok[i] = j == 0 ? anchor[lo] : tokens[(size_t)lo * gamma + j - 1];
      preq[i] = lo;
      pslot[i] = j;
    } else {
      ptok[i] = 0;
      preq[i] = -1;
      pslot[i] = -1;
    }
  }
  if (tid == 0) {
    int pad = -1;
    for (int t = 0; t < tiers.n; ++t)
      if (tiers.v[t] >= M) {
        pad = tiers.v[t];
        break;
      }
    totals[0] = M;
    totals[1] = pad;
  }
}

}  // namespace dspark

using namespace dspark;

extern "C" int dspark_schedule_topb(const float* surv, const float* surv_budget,
                                    const uint32_t* sps_milli, int M_max, int R, int gamma,
                                    int B_cap, int mode, int K_fixed, int32_t* win_len,
                                    int32_t* K_out, void* stream) {
  if (!surv || !sps_milli || !win_len || !K_out) return DSPARK_EINVAL;
  if (mode < DSPARK_SCHED_ARGMAX || mode > DSPARK_SCHED_FIXED) return DSPARK_EINVAL;
  if (R < 1 || gamma < 1 || gamma > kMaxGamma) return DSPARK_ESIZE;
  if ((long long)R * (gamma + 1) > kMaxRows) return DSPARK_ESIZE;
  if (M_max < R || M_max > kMaxRows) return DSPARK_ESIZE;
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0,
                     static_cast<hipStream_t>(stream), surv, surv_budget, sps_milli, M_max, R,
                     gamma, B_cap, mode, K_fixed, win_len, K_out);
  return launch_status();
}

static int check_tiers(const int32_t* tiers, int n_tiers) {
  if (!tiers || n_tiers < 1 || n_tiers > kMaxTiers) return DSPARK_ETIER;
  for (int i = 0; i < n_tiers; ++i) {
    if (tiers[i] <= 0) return DSPARK_ETIER;
    if (i && tiers[i] <= tiers[i - 1]) return DSPARK_ETIER;
  }
  return DSPARK_OK;
}

extern "C" int dspark_pack_ragged(const int32_t* anchor, const int32_t* tokens,
                                  const int32_t* win_len, int R, int gamma, const int32_t* tiers,
                                  int n_tiers, int M_cap, int32_t* cu_seqlens,
                                  int32_t* packed_tokens, int32_t* packed_req,
                                  int32_t* packed_slot, int32_t* totals, void* stream) {
  if (!anchor || !tokens || !cu_seqlens || !packed_tokens || !packed_req || !packed_slot || !totals)
    return DSPARK_EINVAL;
  if (R < 1 || gamma < 1 || gamma > kMaxGamma) return DSPARK_ESIZE;
  if ((long long)R * (gamma + 1) > kMaxRows) return DSPARK_ESIZE;
  if (M_cap < R * (gamma + 1)) return DSPARK_ESIZE;
  int st = check_tiers(tiers, n_tiers);
  if (st) return st;
  TierList tl;
  tl.n = n_tiers;
  for (int i = 0; i < kMaxTiers; ++i) tl.v[i] = i < n_tiers ? tiers[i] : 0;
  hipLaunchKernelGGL(pack_kernel, dim3(1), dim3(1024), 0, static_cast<hipStream_t>(stream), anchor,
                     tokens, win_len, R, gamma, tl, M_cap, cu_seqlens, packed_tokens, packed_req,
                     packed_slot, totals);
  return launch_status();
}

extern "C" int dspark_cost_table_prepare(const double* raw_step_time_s, int M_max,
                                         const int32_t* tiers, int n_tiers, int staircase,
                                         uint32_t* sps_milli) {
  if (!raw_step_time_s || !sps_milli) return DSPARK_EINVAL;
  if (M_max < 0) return DSPARK_ESIZE;
  int st = check_tiers(tiers, n_tiers);
  if (st) return st;
  // running maximum: a profiled curve is forced monotone in M
  double* mono = new double[(size_t)M_max + 1];
  double run = -INFINITY;
  for (int m = 0; m <= M_max; ++m) {
    const double t = raw_step_time_s[m];
    if (t > run) run = t;
    mono[m] = run;
  }
  for (int m = 0; m <= M_max; ++m) {
    double T;
    if (staircase) {
      int tier = -1;
      for (int i = 0; i < n_tiers; ++i)
        if (tiers[i] >= m) {
          tier = tiers[i];
          break;
        }
      if (tier < 0) {
        sps_milli[m] = 0;
        continue;
      }
      T = mono[tier < M_max ? tier : M_max];
    } else {
      T = mono[m];
    }
    if (!(T > 0.0) || std::isinf(T)) {
      sps_milli[m] = 0;
      continue;
    }
    double v = std::floor(1000.0 / T + 0.5);
    if (v < 0.0) v = 0.0;
    if (v > 4294967295.0) v = 4294967295.0;
    sps_milli[m] = (uint32_t)v;
  }
  delete[] mono;
  return DSPARK_OK;
}
