// Resident-W2 Markov draft on gfx950: the whole gamma-slot block in one
// launch, with the projection factor W2 held on chip for all the slots.
//
// DSpark digest ("DSpark: Confidence-Scheduled Speculative Decoding with
// Semi-Autoregressive Generation", zhao9797.github.io), "Architecture
// (drafter)": the block is sampled left to right from
// softmax(U_k + W1[x_{k-1}] W2), k = 1..gamma, with the same W2 at every
// slot. Launched once per slot, a draft re-reads all of W2 (r x V, 77.8 MB
// at the Qwen3 shape) for every slot. Here W2 is read from memory once per
// call and kept on chip, so a slot streams only U_k.
//
// One workgroup of eight waves (two per SIMD) per compute unit, all resident
// at once. Compute unit c owns the 64-entry vocabulary tiles
// [c n_t / G, (c+1) n_t / G) (at most 8 + LT of them): wave w keeps tile
// lo + w of the pre-packed W2 in registers (128 registers, read by the matrix
// cores in place), and LT = 2 more tiles (lo + 8, lo + 9) sit in LDS, of
// which wave w computes the 16 columns of sub-tile w % 4 of tile
// lo + 8 + w / 4. Per slot k:
//
//   gemm    the gathered W1 rows of up to 128 requests are staged in LDS per
//           phase; every 16-request block meets every resident tile on the
//           matrix cores, U_k is added, and each (request, tile) forms its
//           softmax partial (max, sum of exp), kept in LDS until the phase
//           ends and then written out at once;
//   hand-off each compute unit marks its partials ready (a per-unit word);
//   select  request n on workgroup n mod G: merge the request's partials,
//           draw u S with the slot's Philox uniform, find the crossing tile,
//           recompute it (its W2 tile staged through LDS) with the same
//           matrix-core order, finish the inverse-CDF search;
//   hand-off the token goes out with the slot's tag in one word, which the
//           next slot's staging waits on before it gathers W1[x_k].
//
// After the last slot, each workgroup scores its own requests with the
// confidence head (slot k needs only x_{k-1}, which it drew itself).
//
// The U_k loads run two block-steps ahead of the products and continue
// across phases and slots. Data that one compute unit writes and another
// reads within the launch (partials, ready words, tagged tokens) goes through
// agent-scope accesses, which reach the point of coherence across the XCDs'
// L2 caches without a whole-cache write-back. Instead of grid-wide barriers,
// each reader polls just the words it needs: select thread p waits for unit
// p's ready word and then reads unit p's partials; staging thread n waits for
// request n's tagged token. Tags are epoch * 32 + slot, with a per-call
// epoch the last workgroup advances, so a word left by an earlier slot or
// call never satisfies a wait and nothing needs clearing between calls. No
// buffer is rewritten while a reader may still need it: a unit rewrites
// request n's partials only after it has seen request n's next token, which
// its select writes after reading them. Every wait is bounded; a wait that
// runs out sets an error word in the workspace and lets the launch finish.
#include "dspark_device.hpp"
#include "dspark_host.hpp"

#include <algorithm>

namespace dspark {

namespace {

typedef Elem<true>::Frag Frag;  // 8 bfloat16 values: one matrix-core operand
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kResThreads = 512;             // eight waves, two per SIMD
constexpr int kResWaves = kResThreads / kWave;
constexpr int kResKC = 8;                    // 32-rank chunks: rank up to 256
constexpr int kResTileFrags = kResKC * 4 * kWave;  // 2048 fragments = 32 KB per tile
constexpr int kResRegTilesCU = kResWaves;    // one W2 tile per wave in registers
constexpr int kResLdsTiles = 2;              // W2 tiles in LDS (when a unit needs more than 8)
constexpr int kResPhaseReq = 128;            // requests whose W1 rows one phase stages
constexpr int kResLdw = kResKC * kChunkK + kLdsPad;  // staged row stride (elements)
constexpr int kResCMax = 10;                 // tiles per unit, and per select thread
constexpr int kSpinLimit = 1 << 17;          // polls before a wait gives up

constexpr size_t kResTileBytes = (size_t)kResTileFrags * sizeof(Frag);
constexpr size_t kResStageBytes = (size_t)kResPhaseReq * kResLdw * sizeof(uint16_t);

constexpr int kResMaxTilesCU = kResRegTilesCU + kResLdsTiles;
static_assert(kResMaxTilesCU == kResCMax, "a unit's tiles fill one select thread");
// LDS: LT W2 tiles, the staged W1 rows, the LDS tiles' per-wave sub-tile
// partials, and the phase's (request, tile) partials before they go out
size_t res_lds_bytes(int LT) {
  return LT * kResTileBytes + kResStageBytes + (size_t)LT * 4 * kResPhaseReq * sizeof(float2) +
         (size_t)kResMaxTilesCU * kResPhaseReq * sizeof(float2);
}

// agent-scope (cross-XCD coherent) accesses of words other compute units read
__device__ __forceinline__ void st_coh(float2* p, float2 v) {
  const unsigned long long bits =
      ((unsigned long long)__float_as_uint(v.y) << 32) | __float_as_uint(v.x);
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), bits, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_coh(const float2* p) {
  const unsigned long long bits = __hip_atomic_load(
      reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((unsigned)bits), __uint_as_float((unsigned)(bits >> 32)));
}
__device__ __forceinline__ void st_coh(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_coh(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_coh(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// Hand-off words in the draft workspace (byte offsets in its resident block):
// the call epoch, the exit counter and the error word on lines of their own,
// then one ready word per unit (up to 256) and one tagged token word per
// request (up to 256: token in the low half, tag in the high half).
constexpr int kHoEpoch = 0, kHoDone = 64, kHoErr = 128;   // words
constexpr int kHoReady = 192;                              // words, 256 of them
constexpr size_t kHoTokByte = 2048;                        // 8-byte words, 256 of them
static_assert(kHoTokByte + 256 * 8 == kResidentBarBytes, "hand-off block size");
static_assert(kHoErr * 4 == kResidentErrByte, "error word offset");

namespace {

// The bounded wait: poll *p (agent scope) until it is at least `want`.
__device__ __forceinline__ unsigned wait_at_least(const unsigned* p, unsigned want, unsigned* err) {
  unsigned v = ld_coh(p);
  int spins = 0;
  while (v < want) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > kSpinLimit) {
      __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    v = ld_coh(p);
  }
  return v;
}
__device__ __forceinline__ unsigned long long wait_tag(const unsigned long long* p, unsigned want,
                                                       unsigned* err) {
  unsigned long long v =
      __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int spins = 0;
  while ((unsigned)(v >> 32) < want) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > kSpinLimit) {
      __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return v;
}

}  // namespace

// The select's workgroup reductions and inverse-CDF tile search
// (dspark_device.hpp's block_max / block_tile_search) for a workgroup of NW
// waves; threads that own no tiles take part with cnt = 0.
template <int NW>
struct ResSearchShared {
  float red[NW];
  float wsum[NW];
  int wlast[NW];
  int wfirst[NW];
  int tstar;
  float pb;
};

template <int NW>
__device__ __forceinline__ float res_block_max(float v, ResSearchShared<NW>& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  v = wave_max(v);
  if (lane == 0) sh.red[wave] = v;
  __syncthreads();
  float m = sh.red[0];
#pragma unroll
  for (int q = 1; q < NW; ++q) m = fmaxf(m, sh.red[q]);
  return m;
}

template <int CMAX, int NW, typename WFn>
__device__ __forceinline__ WaveSearch res_tile_search(WFn w, int t0, int cnt, float u,
                                                      ResSearchShared<NW>& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  float ls = 0.0f;
#pragma unroll
  for (int i = 0; i < CMAX; ++i)
    if (i < cnt) ls += w(i);
  float incl = wave_inclusive_scan(ls, lane);
  if (lane == kWave - 1) sh.wsum[wave] = incl;
  __syncthreads();
  float off = 0.0f, S = 0.0f;
#pragma unroll
  for (int q = 0; q < NW; ++q) {
    if (q < wave) off += sh.wsum[q];
    S += sh.wsum[q];
  }
  WaveSearch r;
  r.S = S;
  r.T = u * S;
  const float prev = wave_shift_up1(incl) + off;
  incl += off;
  const unsigned long long pm = __ballot(incl > r.T);
  if (lane == 0) sh.wfirst[wave] = pm ? wave * kWave + __ffsll((long long)pm) - 1 : 0x7fffffff;
  __syncthreads();
  int pstar = 0x7fffffff;
#pragma unroll
  for (int q = 0; q < NW; ++q) pstar = min(pstar, sh.wfirst[q]);
  int tstar = -1;
  r.pb = -INFINITY;
  if (pstar != 0x7fffffff) {  // uniform over the workgroup
    if (tid == pstar) {
      float cum = prev, pbv = -INFINITY;
      int found = -1, last = -1;
#pragma unroll
      for (int i = 0; i < CMAX; ++i)
        if (i < cnt) {
          const float wi = w(i);
          const float cn = cum + wi;
          if (found < 0 && cn > r.T) {
            found = t0 + i;
            pbv = cum;
          }
          if (wi > 0.0f) last = t0 + i;
          cum = cn;
        }
      sh.tstar = found >= 0 ? found : last;
      sh.pb = found >= 0 ? pbv : -INFINITY;
    }
    __syncthreads();
    tstar = sh.tstar;
    r.pb = sh.pb;
  }
  if (tstar < 0) {  // no crossing (rounding): the last tile with positive weight
    int last = -1;
#pragma unroll
    for (int i = 0; i < CMAX; ++i)
      if (i < cnt && w(i) > 0.0f) last = t0 + i;
    const int wl = wave_max_int(last);
    if (lane == 0) sh.wlast[wave] = wl;
    __syncthreads();
    int glast = -1;
#pragma unroll
    for (int q = 0; q < NW; ++q) glast = max(glast, sh.wlast[q]);
    tstar = glast;
    r.pb = -INFINITY;
  }
  r.tstar = tstar;
  return r;
}

struct ResArgs {
  const uint16_t* U;       // [R, gamma, V] base logits (row stride ldU = gamma V)
  long long ldU;
  const uint16_t* W1;      // [V, r]
  const uint16_t* W2p;     // pre-packed W2
  const int* anchor;       // [R] x_0
  uint64_t seed;
  StepArg step;
  const uint32_t* req_ids;
  int R, gamma, V, r, n_t;
  int* tokens;             // [R, gamma]
  float* p_draft;          // [R, gamma]
  float* lse_draft;        // [R, gamma]
  float2* part;            // [R, ldn] tile partials (part_pos order)
  int ldn, c;
  unsigned* bar;
  ConfArgs ca;             // ca.h == nullptr: no confidence head
};

// U of one block-step, prefetched: 16 entries of the register tile and 4 of
// the wave's LDS sub-tile.
struct ResPre {
  Raw16<true> full;
  u32x2 quart;
};

template <int LT>
__global__ __launch_bounds__(kResThreads) void resident_draft_kernel(ResArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ ResSearchShared<kResWaves> sh;
  __shared__ int s_tok[kResPhaseReq];  // the phase's previous tokens, read once per workgroup
  Frag* lds_w2 = reinterpret_cast<Frag*>(smem);
  uint16_t* lds_b = reinterpret_cast<uint16_t*>(smem + LT * kResTileBytes);
  float2* lds_q = reinterpret_cast<float2*>(smem + LT * kResTileBytes + kResStageBytes);
  float2* lds_p = lds_q + LT * 4 * kResPhaseReq;  // [tile i of this unit][request of the phase]

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int g = lane >> 4, nl = lane & 15;
  const int G = gridDim.x, cu = blockIdx.x;
  const int R = a.R, V = a.V, r = a.r, n_t = a.n_t, gamma = a.gamma;
  const int lo = (int)((long long)n_t * cu / G), hi = (int)((long long)n_t * (cu + 1) / G);
  const uint64_t stp = a.step.get();
  const Frag* w2f = reinterpret_cast<const Frag*>(a.W2p);
  unsigned* const ho = a.bar;  // hand-off words
  unsigned* const ready = ho + kHoReady;
  unsigned long long* const tok_tag =
      reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(ho) + kHoTokByte);
  unsigned* const err = ho + kHoErr;
  const unsigned tag0 = ld_coh(ho + kHoEpoch) * 32u;  // slot k's tag: tag0 + k

  // ---- resident W2: tile lo + wave in registers, LT tiles in LDS ----
  const int t_own = lo + wave;
  const bool v_own = t_own < hi;
  const int treg = min(t_own, n_t - 1);
  const int ql = wave & 3;                     // the wave's sub-tile of its LDS tile
  const int t_l = lo + kResRegTilesCU + (wave >> 2);
  const bool v_l = LT > 0 && t_l < hi;
  const int tl = min(t_l, n_t - 1);
  Frag A[kResKC * 4];
#pragma unroll
  for (int f = 0; f < kResKC * 4; ++f) A[f] = w2f[(size_t)treg * kResTileFrags + f * kWave + lane];
#pragma unroll
  for (int j = 0; j < LT; ++j) {
    const int t = min(lo + kResRegTilesCU + j, n_t - 1);
#pragma unroll
    for (int q = 0; q < kResTileFrags / kResThreads; ++q)
      lds_w2[j * kResTileFrags + q * kResThreads + tid] =
          w2f[(size_t)t * kResTileFrags + q * kResThreads + tid];
  }
  const Frag* lds_aq = lds_w2 + (wave >> 2) * kResTileFrags;  // the wave's LDS tile

  // ---- the block-step sequence: step s = (slot s / nbp + 1, block s % nbp) ----
  const int nblk = (R + kTileN - 1) / kTileN;
  const int nbp = nblk + (nblk & 1);  // padded to even (two steps per loop trip)
  const long long last_step = (long long)gamma * nbp - 1;
  auto issue = [&](long long s, ResPre& p) {
    s = s < last_step ? s : last_step;
    const int k = (int)(s / nbp) + 1, nb = (int)(s % nbp);
    const int n = min(nb * kTileN + nl, R - 1);
    const uint16_t* row = a.U + (size_t)n * a.ldU + (size_t)(k - 1) * V;
    const int v0 = treg * kTileV + 16 * g;
    load16_clamped<true, true>(row, v0, min(16, V - v0), V, p.full);
    if constexpr (LT > 0) {
      const int vq = tl * kTileV + 16 * g + 4 * ql;
      const int off = vq + 4 <= V ? vq : 0;
      p.quart = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(row + off));
    }
  };

  // one block-step: the register tile and the wave's LDS sub-tile against the
  // staged W1 rows of block nb (local block nbl), U_k added, softmax partials
  // into LDS
  auto step = [&](int nb, int nbl, const ResPre& p) {
    const uint16_t* brow = lds_b + (nbl * kTileN + nl) * kResLdw + 8 * g;
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 aq = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < kResKC; ++kc) {
      const Frag b = *reinterpret_cast<const Frag*>(brow + kc * kChunkK);
#pragma unroll
      for (int j = 0; j < 4; ++j) mma_step<true>(acc[j], A[kc * 4 + j], b);
      if constexpr (LT > 0) mma_step<true>(aq, lds_aq[(kc * 4 + ql) * kWave + lane], b);
    }
    const int n = nb * kTileN + nl;
    const bool act = n < R;
    {
      const int v0 = treg * kTileV + 16 * g;
      float u16[16], z[16];
      unpack16<true>(p.full, u16);
      tile_logits<true>(acc, u16, min(16, V - v0), act && v_own, z);
      float m, sm;
      softmax16_merge4(z, m, sm);
      // into LDS; the phase's partials go out together after its last step
      // (a write-through store per step would hold up the U loads behind it,
      // memory operations completing in order). The four lane groups hold
      // the same merged value; slots of masked requests are never read.
      lds_p[wave * kResPhaseReq + nbl * kTileN + nl] = make_float2(m, sm);
    }
    if constexpr (LT > 0) {
      // entries v = 64 t + 16 g + 4 ql + i of request n, i < 4
      const int vq = tl * kTileV + 16 * g + 4 * ql;
      const int nv = act && v_l ? max(0, min(4, V - vq)) : 0;
      const float uq[4] = {__uint_as_float(p.quart.x << 16), __uint_as_float(p.quart.x & 0xFFFF0000u),
                           __uint_as_float(p.quart.y << 16), __uint_as_float(p.quart.y & 0xFFFF0000u)};
      float z[4], m = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = i < nv ? aq[i] + uq[i] : -INFINITY;
        m = fmaxf(m, z[i]);
      }
      const float mb = -(m == -INFINITY ? 0.0f : m) * kLog2e;
      float sm = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) sm += __builtin_amdgcn_exp2f(fmaf(z[i], kLog2e, mb));
#pragma unroll
      for (int o = 0; o < 2; ++o) {  // partners l ^ 16, then l ^ 32
        const float m2 = o == 0 ? lane_partner<true>(m) : lane_partner<false>(m);
        const float s2 = o == 0 ? lane_partner<true>(sm) : lane_partner<false>(sm);
        const float mm = fmaxf(m, m2);
        const float mr = mm == -INFINITY ? 0.0f : mm;
        const float sa = m == -INFINITY ? 0.0f : sm * __expf(m - mr);
        const float sb = m2 == -INFINITY ? 0.0f : s2 * __expf(m2 - mr);
        sm = sa + sb;
        m = mm;
      }
      lds_q[wave * kResPhaseReq + nbl * kTileN + nl] = make_float2(m, sm);
    }
  };

  ResPre pa, pb;
  issue(0, pa);
  issue(1, pb);
  long long s_next = 2;  // the step the next issue() fetches
  const int nph = (R + kResPhaseReq - 1) / kResPhaseReq;

  for (int k = 1; k <= gamma; ++k) {
    // ================= gemm =================
    for (int ph = 0; ph < nph; ++ph) {
      const int base = ph * kResPhaseReq;
      const int count = min(kResPhaseReq, R - base);
      // stage the W1 rows of the phase's requests (rows >= count: zero).
      // The tokens of slot k-1 were written by other workgroups: each is read
      // once per workgroup at agent scope (every compute unit reads the same
      // few lines, which bypass the L2) and shared through LDS.
      if (tid < kResPhaseReq) {
        const int n = base + min(tid, count - 1);
        const int x = k == 1 ? a.anchor[n] : (int)(unsigned)wait_tag(tok_tag + n, tag0 + k - 1, err);
        s_tok[tid] = clamp_token(x, V);
      }
      __syncthreads();
      constexpr int kVecRow = kResKC * kChunkK / 8;  // 32 16-byte pieces per row
#pragma unroll
      for (int q = 0; q < kResPhaseReq * kVecRow / kResThreads; ++q) {
        const int idx = q * kResThreads + tid;
        const int nloc = idx / kVecRow, cv = idx % kVecRow;
        const int x = s_tok[nloc];
        const Frag f = *reinterpret_cast<const Frag*>(a.W1 + (size_t)x * r + min(cv * 8, r - 8));
        *reinterpret_cast<Frag*>(lds_b + nloc * kResLdw + cv * 8) = (nloc < count && cv * 8 < r) ? f : Frag{};
      }
      __syncthreads();
      const int nb0 = base / kTileN;
      const int nb1 = min(nbp, nb0 + kResPhaseReq / kTileN);  // nb1 - nb0 is even
      for (int nb = nb0; nb + 2 < nb1; nb += 2) {
        step(nb, nb - nb0, pa);
        issue(s_next++, pa);
        step(nb + 1, nb + 1 - nb0, pb);
        issue(s_next++, pb);
      }
      step(nb1 - 2, nb1 - 2 - nb0, pa);
      step(nb1 - 1, nb1 - 1 - nb0, pb);
      // the slot's last two steps issue their successors only after the
      // grid barrier, whose wait would otherwise include those loads
      if (ph + 1 < nph) {
        issue(s_next++, pa);
        issue(s_next++, pb);
      }
      __syncthreads();
      // the LDS tiles' partials: merge the four waves' sub-tiles in order
      if (LT > 0 && tid < LT * kResPhaseReq) {
        const int j = tid / kResPhaseReq, nloc = tid % kResPhaseReq;
        float m = -INFINITY, sm = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float2 q = lds_q[(j * 4 + w) * kResPhaseReq + nloc];
          softmax_merge(m, sm, q.x, q.y);
        }
        lds_p[(kResRegTilesCU + j) * kResPhaseReq + nloc] = make_float2(m, sm);
      }
      __syncthreads();
      // the phase's partials out: tile lo + i of request n at
      // part[n][i * 256 + cu], so that select thread p reads unit p's tiles
      for (int idx = tid; idx < (hi - lo) * count; idx += kResThreads) {
        const int i = idx / count, nloc = idx - i * count;
        st_coh(a.part + (size_t)(base + nloc) * a.ldn + i * kSelThreads + cu,
               lds_p[i * kResPhaseReq + nloc]);
      }
    }
    // this unit's partials of slot k are out: mark them ready
    __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
    __syncthreads();
    if (tid == 0) __hip_atomic_store(ready + cu, tag0 + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    issue(s_next++, pa);  // the next slot's first steps (clamped after the last slot)
    issue(s_next++, pb);

    // ================= select =================
    for (int n = cu; n < R; n += G) {  // workgroup-uniform
      // thread p < G holds unit p's tiles [lo_p, hi_p); the others none
      const float2* prow = a.part + (size_t)n * a.ldn;
      const int pu = min(tid, G - 1);
      const int t0 = (int)((long long)n_t * pu / G);
      const int cnt = tid < G ? (int)((long long)n_t * (pu + 1) / G) - t0 : 0;
      wait_at_least(ready + pu, tag0 + k, err);  // unit pu's partials of slot k
      float2 pv[kResCMax];
#pragma unroll
      for (int i = 0; i < kResCMax; ++i) pv[i] = ld_coh(prow + min(i, a.c - 1) * kSelThreads + pu);
      const int xp = clamp_token(
          k == 1 ? a.anchor[n]
                 : (int)(unsigned)__hip_atomic_load(tok_tag + n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
          V);
      Frag bsel[kResKC];
      load_b_row<true, kResKC, true>(a.W1 + (size_t)xp * r, r, lane, bsel);
      const float u = slot_uniform(a.seed, stp, a.req_ids[n], k, kPurposeDraft);
      float lm = -INFINITY;
#pragma unroll
      for (int i = 0; i < kResCMax; ++i) lm = fmaxf(lm, i < cnt ? pv[i].x : -INFINITY);
      const float m = res_block_max(lm, sh);
      float w[kResCMax];
#pragma unroll
      for (int i = 0; i < kResCMax; ++i) w[i] = i < cnt ? pv[i].y * __expf(pv[i].x - m) : 0.0f;
      const WaveSearch ws = res_tile_search<kResCMax>([&](int i) { return w[i]; }, t0, cnt, u, sh);
      // the crossing tile's W2 through LDS (the staging area is free here)
      const int t = min(max(ws.tstar, 0), n_t - 1);
      const int v = t * kTileV + lane;
      const bool valid = v < V;
      const float uo = to_f32(a.U[(size_t)n * a.ldU + (size_t)(k - 1) * V + min(v, V - 1)]);
      Frag* lds_t = reinterpret_cast<Frag*>(lds_b);
#pragma unroll
      for (int q = 0; q < kResTileFrags / kResThreads; ++q)
        lds_t[q * kResThreads + tid] = w2f[(size_t)t * kResTileFrags + q * kResThreads + tid];
      __syncthreads();
      if (wave == 0) {
        f32x4 acc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < kResKC; ++kc)
#pragma unroll
          for (int j = 0; j < 4; ++j) mma_step<true>(acc[j], lds_t[(kc * 4 + j) * kWave + lane], bsel[kc]);
        const float zo = own_entry(acc, lane) + uo;  // the same sum the gemm formed
        const float e = valid ? __expf(zo - m) : 0.0f;
        const int sel = tile_pick(e, valid, ws.pb, ws.T, lane);
        const float esel = readlane_f(e, sel);
        if (lane == 0) {
          const size_t o = (size_t)n * gamma + k - 1;
          const int x = t * kTileV + sel;
          __hip_atomic_store(tok_tag + n,
                             ((unsigned long long)(tag0 + k) << 32) | (unsigned)x,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          st_coh(a.tokens + o, x);  // the confidence head reads it back at agent scope
          a.p_draft[o] = esel / ws.S;
          a.lse_draft[o] = m + __logf(ws.S);
        }
      }
      __syncthreads();  // the LDS tile is reused by the next request or slot
    }
  }
  // the last workgroup out advances the call epoch (every workgroup has read
  // it at its start)
  if (tid == 0) {
    const unsigned old =
        __hip_atomic_fetch_add(ho + kHoDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1u == (unsigned)G) {
      __hip_atomic_store(ho + kHoDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(ho + kHoEpoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ================= confidence head =================
  // c_k = sigmoid(z inv_temp_k), z = w . [h_k ; W1[x_{k-1}]] + b, and the
  // survival a_k = a_{k-1} c_k, for every slot of this workgroup's requests:
  // slot k needs only x_{k-1}, which this workgroup drew itself, so no slot
  // waits for it. The confidence kernel's wave code (one wave per slot).
  if (a.ca.h != nullptr) {
    float* s_conf = reinterpret_cast<float*>(lds_b);
    for (int n = cu; n < R; n += G) {  // workgroup-uniform
      for (int k = 1 + wave; k <= gamma; k += kResWaves) {
        const size_t o = (size_t)n * gamma + k - 1;
        const int xp = clamp_token(k == 1 ? a.anchor[n] : ld_coh(a.tokens + o - 1), V);  // drawn here
        float z = conf_logit<true>(static_cast<const uint16_t*>(a.ca.h) + o * a.ca.d,
                                   a.W1 + (size_t)xp * r, a.ca.w, a.ca.b, a.ca.d, r, a.ca.vec_h,
                                   a.ca.vec_w1, lane);
        if (lane == 0) {
          if (a.ca.logit != nullptr) a.ca.logit[o] = z;
          if (a.ca.inv_temp != nullptr) z *= a.ca.inv_temp[k - 1];
          const float cf = 1.0f / (1.0f + __expf(-z));
          a.ca.conf[o] = cf;
          s_conf[k - 1] = cf;
        }
      }
      __syncthreads();
      if (tid == 0) {  // the prefix product, in slot order
        float sv = 1.0f;
        for (int k = 1; k <= gamma; ++k) {
          sv *= s_conf[k - 1];
          a.ca.surv[(size_t)n * gamma + k - 1] = sv;
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

namespace {

int g_draft_path = DSPARK_DRAFT_AUTO;

template <int LT>
bool res_prepare(size_t lds) {
  static bool done[64] = {false};
  static bool ok[64] = {false};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  if (!done[dev]) {
    int max_lds = 0;
    ok[dev] = hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) ==
                  hipSuccess && (size_t)max_lds >= lds &&
              hipFuncSetAttribute(reinterpret_cast<const void*>(&resident_draft_kernel<LT>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess;
    done[dev] = true;
  }
  return ok[dev];
}

}  // namespace

// LDS-resident tiles the shape needs (-1: more than the resident kernel holds)
static int res_lds_tiles(int V, int G) {
  const int per_cu = ceil_div(n_vtiles(V), G);
  if (per_cu > kResMaxTilesCU) return -1;
  return per_cu > kResRegTilesCU ? kResLdsTiles : 0;
}

bool resident_draft_eligible(const void* U, const void* W1, int R, int gamma, int V, int r,
                             int dtype) {
  // AUTO keeps the per-slot launches: on MI355X they are faster at every
  // named shape so far (the resident kernel's two grid-wide hand-offs per
  // slot cost more than the W2 re-read they save)
  if (g_draft_path != DSPARK_DRAFT_RESIDENT) return false;
  if (dtype != DSPARK_BF16 || kc_instance(r) != kResKC || r % 8 != 0) return false;
  if (R > 2 * kResPhaseReq || V % 8 != 0 || gamma < 1) return false;
  if (!rows_vec_ok(U, (long long)gamma * V, V, 8) || !w1_vec_ok(W1, r)) return false;
  if (part_chunk(V) > kResCMax) return false;
  const int G = device_cu_count();
  if (G > kSelThreads) return false;
  const int LT = res_lds_tiles(V, G);
  if (LT < 0) return false;
  // a unit's tiles sit at [i * 256 + unit] of a request's partial row
  if (ceil_div(n_vtiles(V), G) > part_chunk(V)) return false;
  const size_t lds = res_lds_bytes(LT);
  return LT == 0 ? res_prepare<0>(lds) : res_prepare<kResLdsTiles>(lds);
}

int resident_draft_launch(const void* U, const void* W1, const void* W2p, const int32_t* anchor,
                          uint64_t seed, StepArg step, const uint32_t* req_ids, int R, int gamma,
                          int V, int r, int32_t* tokens, float* p_draft, float* lse_draft,
                          void* ws, const ConfArgs& ca, hipStream_t s) {
  float2* part = static_cast<float2*>(ws);
  const int G = device_cu_count();
  const int LT = res_lds_tiles(V, G);
  ResArgs a;
  a.U = static_cast<const uint16_t*>(U);
  a.ldU = (long long)gamma * V;
  a.W1 = static_cast<const uint16_t*>(W1);
  a.W2p = static_cast<const uint16_t*>(W2p);
  a.anchor = anchor;
  a.seed = seed;
  a.step = step;
  a.req_ids = req_ids;
  a.R = R;
  a.gamma = gamma;
  a.V = V;
  a.r = r;
  a.n_t = n_vtiles(V);
  a.tokens = tokens;
  a.p_draft = p_draft;
  a.lse_draft = lse_draft;
  a.part = part;
  a.ldn = part_ld(V);
  a.c = part_chunk(V);
  a.bar = reinterpret_cast<unsigned*>(reinterpret_cast<char*>(part) + resident_bar_offset(R, V));
  a.ca = ca;
  const size_t lds = res_lds_bytes(LT);
  if (LT == 0)
    hipLaunchKernelGGL(resident_draft_kernel<0>, dim3(G), dim3(kResThreads), lds, s, a);
  else
    hipLaunchKernelGGL(resident_draft_kernel<kResLdsTiles>, dim3(G), dim3(kResThreads), lds, s, a);
  return launch_status();
}

}  // namespace dspark

extern "C" int dspark_set_draft_path(int path) {
  if (path != DSPARK_DRAFT_AUTO && path != DSPARK_DRAFT_PER_SLOT && path != DSPARK_DRAFT_RESIDENT)
    return DSPARK_EINVAL;
  const int prev = dspark::g_draft_path;
  dspark::g_draft_path = path;
  return prev;
}
