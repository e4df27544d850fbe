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
// keys in LDS (a stable LSD radix sort over the 21-bit code 2^20 - a_q, three
// passes of 7 bits: ties keep index order, which is the key order), integer
// prefix sums, Theta per K, an argmax, and the window counts, read off the
// K-th smallest key as a threshold.
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
constexpr int kSchedWaves = kSchedThreads / kWave;
constexpr int kSchedMaxKeys = 4096;
constexpr int kSchedMaxRows = kSchedMaxKeys / kWave;  // rows of 64 keys
constexpr int kRadixBits = 7;
constexpr int kRadixBuckets = 1 << kRadixBits;
constexpr int kRadixPasses = 3;                        // 21-bit codes
constexpr uint32_t kQOne = 1u << 20;
constexpr unsigned long long kPadCode = (1ull << (kRadixBits * kRadixPasses)) - 1;  // above any code

__device__ __forceinline__ uint32_t quantize_survival(float a) {
  if (!(a == a)) return 0u;
  a = fminf(fmaxf(a, 0.0f), 1.0f);
  return (uint32_t)(a * 1048576.0f);  // exact scaling; truncation = floor for a >= 0
}

struct SchedShared {
  unsigned long long orig[kSchedMaxKeys];  // keys in index order
  unsigned long long a[kSchedMaxKeys];     // radix ping-pong buffers; result in a
  unsigned long long b[kSchedMaxKeys];
  // radix passes: per (row, digit) counts, row-major, then their prefix down
  // each digit's column; the scan of the sorted values afterwards
  uint32_t hist[kRadixBuckets * kSchedMaxRows];
  uint32_t dbase[kRadixBuckets];  // keys of smaller digits
  uint32_t wsum[kSchedWaves];
  unsigned long long th[kSchedWaves];
  int k[kSchedWaves];
};

// orig[i] = ((2^20 - a_q) << 32) | i for i = r*gamma + j (a_q the prefix-min
// quantised survival of request r), padded to NP keys that sort last.
__device__ __forceinline__ void build_keys(const float* __restrict__ a, int R, int gamma, int NP,
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
  for (int i = N + threadIdx.x; i < NP; i += blockDim.x)
    keys[i] = (kPadCode << 32) | (unsigned long long)i;
  __syncthreads();
}

// In-place exclusive prefix sum of x[0..n) over the workgroup (n <= 8192).
__device__ __forceinline__ void block_exclusive_scan(uint32_t* x, int n, uint32_t* wsum) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  constexpr int kE = kRadixBuckets * kSchedMaxRows / kSchedThreads;  // 8
  const int e0 = tid * kE;
  uint32_t v[kE];
  uint32_t local = 0;
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    v[e] = e0 + e < n ? x[e0 + e] : 0u;
    local += v[e];
  }
  const uint32_t incl = wave_inclusive_scan_u32(local);
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  uint32_t run = incl - local;
#pragma unroll
  for (int w = 0; w < kSchedWaves; ++w) run += w < wave ? wsum[w] : 0u;
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    if (e0 + e < n) x[e0 + e] = run;
    run += v[e];
  }
  __syncthreads();
}

// One stable counting pass on digit (code >> shift) & 127 of NR rows of 64
// keys: a key's place = keys of smaller digits + keys of its digit in earlier
// rows + earlier keys of its digit in its row. The last is a ballot match; the
// last key of each digit in a row writes the row's count of that digit (the
// wave that owns the row clears the row's counts first). Wave 0 then runs the
// prefix down each digit's column (lane l: digits 2l, 2l+1) and the digit
// bases, with no workgroup-wide scan.
__device__ __forceinline__ void radix_pass(const unsigned long long* src, unsigned long long* dst, int NR,
                           int shift, SchedShared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  constexpr int kRowsPerWave = kSchedMaxRows / kSchedWaves;  // 4
  unsigned long long kk[kRowsPerWave];
  int dig[kRowsPerWave], rk[kRowsPerWave];
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int u = 0; u < kRowsPerWave; ++u) {
    const int row = wave + kSchedWaves * u;
    kk[u] = 0ull;
    dig[u] = 0;
    rk[u] = 0;
    if (row < NR) {  // wave-uniform
      const unsigned long long key = src[row * kWave + lane];
      const int d = (int)((key >> (32 + shift)) & (kRadixBuckets - 1));
      unsigned long long m = ~0ull;
#pragma unroll
      for (int bt = 0; bt < kRadixBits; ++bt) {
        const unsigned long long B = __ballot((d >> bt) & 1);
        m &= ((d >> bt) & 1) ? B : ~B;
      }
      rk[u] = __popcll(m & below);
      uint32_t* h = sh.hist + row * kRadixBuckets;
      h[lane] = 0u;
      h[lane + kWave] = 0u;
      if ((m >> lane) == 1ull) h[d] = (uint32_t)rk[u] + 1u;  // no later key of this digit
      kk[u] = key;
      dig[u] = d;
    }
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t run0 = 0u, run1 = 0u;
    uint2* col = reinterpret_cast<uint2*>(sh.hist) + lane;  // digits 2 lane, 2 lane + 1
    constexpr int kBatch = 8;  // rows read before their prefixes are written
    for (int r0 = 0; r0 < NR; r0 += kBatch) {  // uniform
      uint2 c[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) c[i] = r0 + i < NR ? col[(r0 + i) * (kRadixBuckets / 2)] : make_uint2(0u, 0u);
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (r0 + i < NR) col[(r0 + i) * (kRadixBuckets / 2)] = make_uint2(run0, run1);
        run0 += c[i].x;
        run1 += c[i].y;
      }
    }
    const uint32_t pair = run0 + run1;
    const uint32_t ex = wave_inclusive_scan_u32(pair) - pair;
    sh.dbase[2 * lane] = ex;
    sh.dbase[2 * lane + 1] = ex + run0;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kRowsPerWave; ++u) {
    const int row = wave + kSchedWaves * u;
    if (row < NR)
      dst[sh.dbase[dig[u]] + sh.hist[row * kRadixBuckets + dig[u]] + rk[u]] = kk[u];
  }
  __syncthreads();
}

// Sort orig[0 .. 64 NR) ascending into sh.a (orig is kept).
__device__ __forceinline__ void radix_sort(int NR, SchedShared& sh) {
  radix_pass(sh.orig, sh.a, NR, 0, sh);
  radix_pass(sh.a, sh.b, NR, kRadixBits, sh);
  radix_pass(sh.b, sh.a, NR, 2 * kRadixBits, sh);
}

// The scheduler's work for one workgroup of kSchedThreads threads. win_s
// (nullable, shared memory): also receives the windows, for a pack that
// follows in the same launch.
__device__ __forceinline__ void schedule_body(
    const float* __restrict__ surv, const float* __restrict__ surv_budget,
    const uint32_t* __restrict__ sps, int M_max, int R, int gamma, int B_cap, int mode, int K_fixed,
    int* __restrict__ win_len, int* __restrict__ K_out, SchedShared& sh, int* win_s) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int N = R * gamma;
  const int NR = (N + kWave - 1) / kWave;
  const int NP = NR * kWave;
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
      const int Kc = tid + i * kSchedThreads;
      sp0[i] = sps[R + min(Kc, K_cap)];
      sp1[i] = sps[R + min(Kc + 1, K_cap)];
    }
    build_keys(surv_budget ? surv_budget : surv, R, gamma, NP, sh.orig);
    radix_sort(NR, sh);
    // ex[K] = sum of the K largest a_q (exclusive prefix over the sorted keys)
    for (int i = tid; i <= N; i += kSchedThreads)
      sh.hist[i] = i < N ? kQOne - (uint32_t)(sh.a[i] >> 32) : 0u;
    __syncthreads();
    block_exclusive_scan(sh.hist, N + 1, sh.wsum);
    const unsigned long long base = (unsigned long long)R * kQOne;
    // Theta_K = tau_K * sps[R + K], tau_K = R*2^20 + ex[K]
    unsigned long long best_t = 0;
    int best_k = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int Kc = tid + i * kSchedThreads;
      if (Kc > K_cap) continue;
      const unsigned long long th = (base + sh.hist[Kc]) * (unsigned long long)sp0[i];
      if (mode == DSPARK_SCHED_ARGMAX) {
        if (best_k == 0x7fffffff || th > best_t) {
          best_t = th;
          best_k = Kc;
        }
      } else if (Kc < K_cap) {  // GREEDY: first K with Theta_{K+1} <= Theta_K
        const unsigned long long th1 = (base + sh.hist[Kc + 1]) * (unsigned long long)sp1[i];
        if (th1 <= th && Kc < best_k) best_k = Kc;
      }
    }
    // ARGMAX: largest Theta, then smallest K; GREEDY: smallest K
    if (mode == DSPARK_SCHED_ARGMAX) {
      wave_argmax_u64(best_t, best_k);
    } else {
      best_k = wave_min_int(best_k);
    }
    if (lane == 0) {
      sh.th[wave] = best_t;
      sh.k[wave] = best_k;
    }
    __syncthreads();
    // every wave reduces the waves' results itself (lanes 0..15). A wave
    // without a candidate holds (0, INT_MAX), which no candidate loses to.
    unsigned long long bt = lane < kSchedWaves ? sh.th[lane] : 0ull;
    int bk = lane < kSchedWaves ? sh.k[lane] : 0x7fffffff;
    if (mode == DSPARK_SCHED_ARGMAX) {
      wave_argmax_u64(bt, bk);
    } else {
      bk = wave_min_int(bk);
    }
    if (mode == DSPARK_SCHED_GREEDY && bk == 0x7fffffff) bk = K_cap;
    if (bk == 0x7fffffff) bk = 0;
    K = bk;
  }

  // selection: the K best keys of the current survivals; within a request
  // they form a prefix, so its window is the count of its keys below the
  // K-th smallest key
  if (mode == DSPARK_SCHED_FIXED || surv_budget != nullptr) {
    build_keys(surv, R, gamma, NP, sh.orig);
    radix_sort(NR, sh);
  }
  const unsigned long long thr = K < N ? sh.a[K] : ~0ull;
  for (int r = tid; r < R; r += kSchedThreads) {
    int cnt = 0;
    for (int j = 0; j < gamma; ++j) cnt += sh.orig[r * gamma + j] < thr;
    win_len[r] = cnt;
    if (win_s != nullptr) win_s[r] = cnt;
  }
  if (tid == 0) K_out[0] = K;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(
    const float* __restrict__ surv, const float* __restrict__ surv_budget,
    const uint32_t* __restrict__ sps, int M_max, int R, int gamma, int B_cap, int mode, int K_fixed,
    int* __restrict__ win_len, int* __restrict__ K_out) {
  __shared__ SchedShared sh;
  schedule_body(surv, surv_budget, sps, M_max, R, gamma, B_cap, mode, K_fixed, win_len, K_out, sh,
                nullptr);
}

struct TierList {
  int n;
  int v[kMaxTiers];
};

struct PackShared {
  int cu[kMaxRows / 2 + 1];
  int wtot[1024 / kWave];
};

// The pack's work for one workgroup of 1024 threads. win_len (nullable: every
// window is gamma) may point to global or shared memory.
__device__ __forceinline__ void pack_body(
    const int* __restrict__ anchor, const int* __restrict__ tokens, const int* win_len,
    int R, int gamma, const TierList& tiers, int M_cap, int* __restrict__ cu_seqlens,
    int* __restrict__ ptok, int* __restrict__ preq, int* __restrict__ pslot,
    int* __restrict__ totals, PackShared& ps) {
  int* cu = ps.cu;
  int* wtot = ps.wtot;
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

// The pack of full blocks (every window gamma): row i of request i / (gamma
// + 1) at slot i mod (gamma + 1), so no scan and no search and no barrier;
// the same outputs as pack_body with win_len == nullptr.
__device__ __forceinline__ void pack_full_body(
    const int* __restrict__ anchor, const int* __restrict__ tokens, int R, int gamma,
    const TierList& tiers, int M_cap, int* __restrict__ cu_seqlens, int* __restrict__ ptok,
    int* __restrict__ preq, int* __restrict__ pslot, int* __restrict__ totals) {
  const int tid = threadIdx.x, G = gamma + 1, M = R * G;
  for (int i = tid; i <= R; i += blockDim.x) cu_seqlens[i] = i * G;
  for (int i = tid; i < M_cap; i += blockDim.x) {
    if (i < M) {
      const int req = i / G, j = i - req * G;
      ptok[i] = j == 0 ? anchor[req] : tokens[(size_t)req * gamma + j - 1];
      preq[i] = req;
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

__global__ __launch_bounds__(1024) void pack_kernel(
    const int* __restrict__ anchor, const int* __restrict__ tokens, const int* __restrict__ win_len,
    int R, int gamma, TierList tiers, int M_cap, int* __restrict__ cu_seqlens,
    int* __restrict__ ptok, int* __restrict__ preq, int* __restrict__ pslot,
    int* __restrict__ totals) {
  __shared__ PackShared ps;
  if (win_len == nullptr) {  // uniform
    pack_full_body(anchor, tokens, R, gamma, tiers, M_cap, cu_seqlens, ptok, preq, pslot, totals);
    return;
  }
  pack_body(anchor, tokens, win_len, R, gamma, tiers, M_cap, cu_seqlens, ptok, preq, pslot, totals,
            ps);
}

// Schedule, then pack, in one workgroup: the windows pass through shared
// memory. pack_windows == 0: the pack keeps every window at gamma (the static
// and cap-accept blocks), as a pack call with win_len NULL; it does not depend
// on the schedule then, so it goes first and its stores drain while the
// scheduler sorts.
__global__ __launch_bounds__(kSchedThreads) void schedule_pack_kernel(
    const float* __restrict__ surv, const float* __restrict__ surv_budget,
    const uint32_t* __restrict__ sps, int M_max, int R, int gamma, int B_cap, int mode, int K_fixed,
    int* __restrict__ win_len, int* __restrict__ K_out, const int* __restrict__ anchor,
    const int* __restrict__ tokens, int pack_windows, TierList tiers, int M_cap,
    int* __restrict__ cu_seqlens, int* __restrict__ ptok, int* __restrict__ preq,
    int* __restrict__ pslot, int* __restrict__ totals) {
  __shared__ SchedShared sh;
  __shared__ PackShared ps;
  __shared__ int win_s[kMaxRows / 2];
  if (!pack_windows)  // uniform
    pack_full_body(anchor, tokens, R, gamma, tiers, M_cap, cu_seqlens, ptok, preq, pslot, totals);
  schedule_body(surv, surv_budget, sps, M_max, R, gamma, B_cap, mode, K_fixed, win_len, K_out, sh,
                win_s);
  if (!pack_windows) return;
  __syncthreads();
  pack_body(anchor, tokens, win_s, R, gamma, tiers, M_cap, cu_seqlens, ptok, preq, pslot, totals,
            ps);
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

extern "C" int dspark_schedule_pack(const float* surv, const float* surv_budget,
                                    const uint32_t* sps_milli, int M_max, int R, int gamma,
                                    int B_cap, int mode, int K_fixed, int32_t* win_len,
                                    int32_t* K_out, const int32_t* anchor, const int32_t* tokens,
                                    int pack_windows, const int32_t* tiers, int n_tiers, int M_cap,
                                    int32_t* cu_seqlens, int32_t* packed_tokens,
                                    int32_t* packed_req, int32_t* packed_slot, int32_t* totals,
                                    void* stream) {
  if (!surv || !sps_milli || !win_len || !K_out) return DSPARK_EINVAL;
  if (!anchor || !tokens || !cu_seqlens || !packed_tokens || !packed_req || !packed_slot || !totals)
    return DSPARK_EINVAL;
  if (mode < DSPARK_SCHED_ARGMAX || mode > DSPARK_SCHED_FIXED) return DSPARK_EINVAL;
  if (R < 1 || gamma < 1 || gamma > kMaxGamma) return DSPARK_ESIZE;
  if ((long long)R * (gamma + 1) > kMaxRows) return DSPARK_ESIZE;
  if (M_max < R || M_max > kMaxRows) return DSPARK_ESIZE;
  if (M_cap < R * (gamma + 1)) return DSPARK_ESIZE;
  int st = check_tiers(tiers, n_tiers);
  if (st) return st;
  TierList tl;
  tl.n = n_tiers;
  for (int i = 0; i < kMaxTiers; ++i) tl.v[i] = i < n_tiers ? tiers[i] : 0;
  hipLaunchKernelGGL(schedule_pack_kernel, dim3(1), dim3(kSchedThreads), 0,
                     static_cast<hipStream_t>(stream), surv, surv_budget, sps_milli, M_max, R,
                     gamma, B_cap, mode, K_fixed, win_len, K_out, anchor, tokens,
                     pack_windows ? 1 : 0, tl, M_cap, cu_seqlens, packed_tokens, packed_req,
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
  // running maximum: a profiled curve is forced monotone in M. The staircase
  // reads it at the tiers only, so those values are taken in one pass first
  // (no buffer: nothing here allocates, so the call cannot throw)
  double at_tier[kMaxTiers];
  if (staircase) {
    double run = -INFINITY;
    int i = 0;
    for (int m = 0; m <= M_max && i < n_tiers; ++m) {
      const double t = raw_step_time_s[m];
      if (t > run) run = t;
      while (i < n_tiers && (tiers[i] < M_max ? tiers[i] : M_max) == m) at_tier[i++] = run;
    }
  }
  double run = -INFINITY;
  for (int m = 0; m <= M_max; ++m) {
    double T;
    if (staircase) {
      int tier = -1;
      for (int i = 0; i < n_tiers; ++i)
        if (tiers[i] >= m) {
          tier = i;
          break;
        }
      if (tier < 0) {
        sps_milli[m] = 0;
        continue;
      }
      T = at_tier[tier];
    } else {
      const double t = raw_step_time_s[m];
      if (t > run) run = t;
      T = run;
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
  return DSPARK_OK;
}
