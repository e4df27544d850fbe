// Markov sequential draft head on gfx950.
//
// DSpark digest ("DSpark: Confidence-Scheduled Speculative Decoding with
// Semi-Autoregressive Generation", zhao9797.github.io), section "Architecture
// (drafter)": the block's base logits U_1..U_gamma come from one parallel
// backbone forward; a Markov head adds the previous-token transition bias
// B = W1 W2 (W1 in R^{V x r} read as a row lookup, W2 in R^{r x V} a
// projection) and the block is sampled left to right from
// softmax(U_k + W1[x_{k-1}] W2). The SGLang DSpark blog ("Performance
// optimisation and zero-overhead scheduling") fuses this sampling path into
// kernels; here it is two launches per slot:
//
//   markov_partials  the [R, r] x [r, V] bias GEMM on the matrix cores
//                    (tile_engine.hpp: W2 tiles staged through LDS, the
//                    gathered W1 rows held in registers); each 64-entry
//                    vocabulary tile adds U_k and emits a softmax partial
//                    (max, sum of exp) per request -- the [R, V] logits never
//                    reach memory;
//   markov_select    one workgroup per request: merge the partials into (m, S),
//                    draw u * S with the slot's Philox uniform, find the tile
//                    where the cumulative mass crosses it, recompute that one
//                    tile with the same matrix-core code (bit-identical
//                    logits) and finish the inverse-CDF search inside it.
#include "dspark_device.hpp"
#include "dspark_host.hpp"
#include "tile_engine.hpp"

#include <algorithm>

namespace dspark {

// ---------------------------------------------------------------------------
// W2 pre-packing (layout documented in dspark_device.hpp)
// ---------------------------------------------------------------------------

template <typename T>
__global__ void prepack_w2_kernel(const T* __restrict__ W2, int r, int V, int KC, int n_t,
                                  T* __restrict__ W2p) {
  const long long groups = (long long)n_t * KC * 4 * kWave;
  for (long long gidx = (long long)blockIdx.x * blockDim.x + threadIdx.x; gidx < groups;
       gidx += (long long)gridDim.x * blockDim.x) {
    const int lane = (int)(gidx % kWave);
    const int j = (int)((gidx / kWave) % 4);
    const int kc = (int)((gidx / (4 * kWave)) % KC);
    const long long t = gidx / ((long long)4 * kWave * KC);
    const int rho = lane & 15;
    const long long v = 64 * t + 16 * (rho >> 2) + 4 * j + (rho & 3);
    const int kb = kc * kChunkK + 8 * (lane >> 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = kb + e;
      W2p[gidx * 8 + e] = (k < r && v < V) ? W2[(size_t)k * V + v] : (T)0;
    }
  }
}

// ---------------------------------------------------------------------------
// pass A: bias GEMM + U add + per-tile softmax partials
// ---------------------------------------------------------------------------

// The slot's Philox draws, taken by the GEMM pass so the select that follows
// only loads them: in workgroup b, lane l of wave 0 draws for request
// 64 b + l, in the prologue once its tile loads are out (the tile queue hands
// these workgroups fewer tiles). u_out == nullptr: the select draws itself.
struct DrawArgs {
  uint64_t seed;
  StepArg step;
  const uint32_t* req_ids;
  int k;
  float* u_out;
};

// Epilogue of the draft pass: z = bias + U_k, then the tile's softmax partial
// (max, sum of exp(z - max)) per request over the four lanes holding its 64
// entries, stored at part[n * ldn + part_pos(t, c)] by the first of them
// (requests past R store nothing).
template <bool BF16, bool VEC>
struct MarkovEpi {
  typedef typename Elem<BF16>::T T;
  typedef Raw16<BF16> Pre;
  struct St {
    const T* row;
    int n;
    bool active;
  };
  const T* U;
  long long ldU;
  int R, V;
  float2* part;
  int ldn, c;
  DrawArgs draw;
  ConfArgs ca;     // ca.h == nullptr: the slot is not scored here
  const T* W1;     // for the head's W1-row dot product
  const int* xprev;
  int xstride, r, gamma;

  __device__ __forceinline__ St prepare(int n) const {
    St s;
    s.n = n;
    s.active = n < R;
    s.row = U + (size_t)min(n, R - 1) * ldU;
    return s;
  }
  // called once per workgroup in the engine's prologue, with the first
  // tiles' loads in flight: the slot's draft uniforms, then (optional) the
  // confidence head for the slot (digest, "Verification scheduling"):
  // c_k = sigmoid(z inv_temp_k), z = w . [h_k ; W1[x_{k-1}]] + b, and the
  // survival a_k = a_{k-1} c_k, a_{k-1} from the previous slot's launch. One
  // wave per request (workgroup b, wave j: requests b + G (j + waves i)), with
  // the wave code of the confidence kernel, so the values are the same.
  __device__ __forceinline__ void side_work() const {
    // wave 0 of every workgroup strides over the requests, so that every
    // request gets its uniform however few workgroups the vocabulary needs
    if (draw.u_out != nullptr && threadIdx.x < kWave) {
      const uint64_t stp = draw.step.get();
      for (int q = (int)blockIdx.x * kWave + (int)threadIdx.x; q < R; q += (int)gridDim.x * kWave)
        draw.u_out[q] = slot_uniform(draw.seed, stp, draw.req_ids[q], draw.k, kPurposeDraft);
    }
    if (ca.h == nullptr) return;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int waves = blockDim.x / kWave, k = draw.k;
    for (int n = blockIdx.x + gridDim.x * wave; n < R; n += gridDim.x * waves) {  // wave-uniform
      const size_t o = (size_t)n * gamma + (k - 1);
      const int x = clamp_token(xprev[(size_t)n * xstride], V);
      float z = conf_logit<BF16>(static_cast<const T*>(ca.h) + o * ca.d, W1 + (size_t)x * r, ca.w,
                                 ca.b, ca.d, r, ca.vec_h, ca.vec_w1, lane);
      if (lane == 0) {
        if (ca.logit != nullptr) ca.logit[o] = z;
        if (ca.inv_temp != nullptr) z *= ca.inv_temp[k - 1];
        const float cf = 1.0f / (1.0f + __expf(-z));
        const float a_prev = k == 1 ? 1.0f : ca.surv[o - 1];
        ca.conf[o] = cf;
        ca.surv[o] = a_prev * cf;
      }
    }
  }
  __device__ __forceinline__ void load(const St& s, int v0, int nvalid, Pre& p) const {
    load16_clamped<BF16, VEC>(s.row, v0, nvalid, V, p);
  }
  __device__ __forceinline__ void finish(const St& s, int v0, int nvalid, const f32x4 acc[4],
                                         const Pre& p, int t, int lane) const {
    float u16[16], z[16];
    unpack16<BF16>(p, u16);
    tile_logits<BF16>(acc, u16, nvalid, s.active, z);
    float m, sm;
    softmax16_merge4(z, m, sm);
    if ((lane >> 4) == 0 && s.active) part[(size_t)s.n * ldn + part_pos(t, c)] = make_float2(m, sm);
  }
};

template <bool BF16, int KC, int NW, int NB, bool VEC>
__global__ __launch_bounds__(NW * 64) void markov_partials_kernel(
    const typename Elem<BF16>::T* __restrict__ U, long long ldU,
    const typename Elem<BF16>::T* __restrict__ W1, const typename Elem<BF16>::T* __restrict__ W2p,
    const int* __restrict__ xprev, int xstride, int R, int V, int r, int n_t, int w1_rows,
    float2* __restrict__ part, int ldn, int c,
    unsigned* __restrict__ queue, DrawArgs draw, ConfArgs ca, int gamma) {
  const MarkovEpi<BF16, VEC> epi{U, ldU, R, V, part, ldn, c, draw, ca, W1, xprev, xstride,
                                 r, gamma};
  run_tile_engine<BF16, KC, NW, NB, VEC>(W1, W2p, [&](int n) { return xprev[(size_t)n * xstride]; },
                                         R, V, r, n_t, epi, queue, w1_rows, (int)gridDim.x,
                                         (int)blockIdx.x);
}

// ---------------------------------------------------------------------------
// pass B: per-request draw
// ---------------------------------------------------------------------------

// One 256-thread workgroup per request. Thread p owns tiles [p c, p c + c) of
// the request's partial row (CMAX >= c: held in registers; CMAX == 0:
// re-read from memory). Wave 0 then recomputes the crossing tile with the W1
// row it loaded at the start and finishes the draw.
template <bool BF16, int KC, int CMAX, bool VW>
__global__ __launch_bounds__(kSelThreads) void markov_select_kernel(
    const typename Elem<BF16>::T* __restrict__ U, long long ldU,
    const typename Elem<BF16>::T* __restrict__ W1, const typename Elem<BF16>::T* __restrict__ W2p,
    const int* __restrict__ xprev, int xstride, int V, int r, int n_t,
    const float2* __restrict__ part, int ldn, int c, uint64_t seed, StepArg step,
    const uint32_t* __restrict__ req_ids, int k, int* __restrict__ tok_out,
    float* __restrict__ p_out, float* __restrict__ lse_out, int ostride,
    unsigned* __restrict__ queue, int n_queue, const float* __restrict__ u_pre) {
  typedef typename Elem<BF16>::Frag Frag;
  __shared__ BlockSearchShared sh;
  const int n = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1);
  // the GEMM pass that wrote these partials has finished: put its tile-queue
  // counters back to zero for the next one
  if (n == 0 && tid < n_queue) queue[tid * kQueueStride] = 0u;
  const float2* prow = part + (size_t)n * ldn;
  const int t0 = tid * c;
  const int cnt = max(0, min(c, n_t - t0));
  float2 pv[CMAX > 0 ? CMAX : 1];
  if constexpr (CMAX > 0) {
#pragma unroll
    for (int i = 0; i < CMAX; ++i) pv[i] = prow[min(i, c - 1) * kSelThreads + tid];
  }
  // B operand (wave 0's): the W1 row of this request's previous token, in
  // every column; every wave loads it, only wave 0 uses it
  const int x = clamp_token(xprev[(size_t)n * xstride], V);
  Frag b[KC];
  load_b_row<BF16, KC, VW>(W1 + (size_t)x * r, r, lane, b);
  // the draw was taken by the GEMM pass, or is taken here (scalar work that
  // overlaps the loads in flight)
  const float u = u_pre != nullptr ? u_pre[n] : slot_uniform(seed, step.get(), req_ids[n], k, kPurposeDraft);
  float m;
  WaveSearch ws;
  if constexpr (CMAX > 0) {
    float lm = -INFINITY;
#pragma unroll
    for (int i = 0; i < CMAX; ++i) lm = fmaxf(lm, i < cnt ? pv[i].x : -INFINITY);
    m = block_max(lm, sh);
    float w[CMAX];
#pragma unroll
    for (int i = 0; i < CMAX; ++i) w[i] = i < cnt ? pv[i].y * __expf(pv[i].x - m) : 0.0f;
    ws = block_tile_search<CMAX>([&](int i) { return w[i]; }, t0, cnt, u, sh);
  } else {
    float lm = -INFINITY;
    for (int i = 0; i < cnt; ++i) lm = fmaxf(lm, prow[i * kSelThreads + tid].x);
    m = block_max(lm, sh);
    ws = block_tile_search<0>([&](int i) {
      const float2 q = prow[i * kSelThreads + tid];
      return q.y * __expf(q.x - m);
    }, t0, cnt, u, sh);
  }
  if (tid >= kWave) return;  // wave 0 finishes; no barrier below

  // recompute the crossing tile; lane l takes entry v = 64 t + l
  const int t = min(max(ws.tstar, 0), n_t - 1);
  ATile<BF16, KC> at;
  load_a_tile<BF16, KC>(W2p, t, lane, at);
  const int v = t * kTileV + lane;
  const bool valid = v < V;
  const float uo = to_f32(U[(size_t)n * ldU + min(v, V - 1)]);
  // every load of the tile in flight before the first product (one memory
  // latency, not one per batch the scheduler would otherwise interleave)
  __builtin_amdgcn_sched_barrier(0);
  f32x4 acc[4];
  tile_mma_regs<BF16, KC>(at, b, acc);
  const float zo = own_entry(acc, lane) + uo;  // the same sum the GEMM pass formed
  const float e = valid ? __expf(zo - m) : 0.0f;
  const int sel = tile_pick(e, valid, ws.pb, ws.T, lane);
  const float esel = readlane_f(e, sel);
  if (lane == 0) {
    tok_out[(size_t)n * ostride] = t * kTileV + sel;
    p_out[(size_t)n * ostride] = esel / ws.S;
    lse_out[(size_t)n * ostride] = m + __logf(ws.S);
  }
}

// ---------------------------------------------------------------------------
// vocabulary-sharded draft: per-rank summary and select
// ---------------------------------------------------------------------------

// SGLang DSpark blog, "Performance optimisation and zero-overhead scheduling":
// the block drafter's matmul is sharded. With tensor parallelism over the
// vocabulary, rank g of G holds columns [v0, v0 + V_g) of W2 and of U_k and
// runs the GEMM pass on them unchanged (dspark_markov_partials). A slot then
// needs one exchange of per-rank softmax summaries (m_g, S_g) per request and
// one of the chosen token; every rank merges the gathered summaries in rank
// order, so all ranks see the same global (m, S), the same threshold u S and
// the same mass P_g before each rank, and exactly one rank (the one with
// P_g <= u S < P_{g+1}, the last rank for anything above) finds the token in
// its own tiles.

// Per request: the rank's (max, sum of exp) over its tile partials.
template <int CMAX>
__global__ __launch_bounds__(kSelThreads) void markov_shard_summary_kernel(
    const float2* __restrict__ part, int ldn, int c, int n_t, float2* __restrict__ summary) {
  __shared__ BlockSearchShared sh;
  const int n = blockIdx.x, tid = threadIdx.x;
  const float2* prow = part + (size_t)n * ldn;
  const int t0 = tid * c;
  const int cnt = max(0, min(c, n_t - t0));
  float2 pv[CMAX > 0 ? CMAX : 1];
  float lm = -INFINITY;
  if constexpr (CMAX > 0) {
#pragma unroll
    for (int i = 0; i < CMAX; ++i) pv[i] = prow[min(i, c - 1) * kSelThreads + tid];
#pragma unroll
    for (int i = 0; i < CMAX; ++i) lm = fmaxf(lm, i < cnt ? pv[i].x : -INFINITY);
  } else {
    for (int i = 0; i < cnt; ++i) lm = fmaxf(lm, prow[i * kSelThreads + tid].x);
  }
  const float m = block_max(lm, sh);
  __syncthreads();  // block_sum below reuses the reduction slots
  float ls = 0.0f;
  if constexpr (CMAX > 0) {
#pragma unroll
    for (int i = 0; i < CMAX; ++i) ls += i < cnt ? pv[i].y * __expf(pv[i].x - m) : 0.0f;
  } else {
    for (int i = 0; i < cnt; ++i) {
      const float2 q = prow[i * kSelThreads + tid];
      ls += q.y * __expf(q.x - m);
    }
  }
  const float S = block_sum(ls, sh);
  if (tid == 0) summary[n] = make_float2(m, S);
}

// Per request: merge the G gathered summaries, decide the owner of u S, and
// on the owning rank search its own tiles (the select's search and one-tile
// recompute, with the global max and an absolute threshold). Writes, at
// n * ostride: the global token id and its probability on the owning rank,
// -1 and 0 elsewhere (ready for MAX / SUM reductions), and the global
// log-sum-exp on every rank.
template <bool BF16, int KC, int CMAX, bool VW>
__global__ __launch_bounds__(kSelThreads) void markov_shard_select_kernel(
    const typename Elem<BF16>::T* __restrict__ U, long long ldU,
    const typename Elem<BF16>::T* __restrict__ W1, const typename Elem<BF16>::T* __restrict__ W2p,
    const int* __restrict__ xprev, int xstride, int Vg, int Vfull, int r, int n_t,
    const float2* __restrict__ part, int ldn, int c, const float2* __restrict__ summaries, int R,
    int G, int g, int v0, uint64_t seed, StepArg step, const uint32_t* __restrict__ req_ids, int k,
    int* __restrict__ tok_out, float* __restrict__ p_out, float* __restrict__ lse_out,
    int ostride, unsigned* __restrict__ queue, int n_queue) {
  typedef typename Elem<BF16>::Frag Frag;
  __shared__ BlockSearchShared sh;
  const int n = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1);
  if (n == 0 && tid < n_queue) queue[tid * kQueueStride] = 0u;
  const float2* prow = part + (size_t)n * ldn;
  const int t0 = tid * c;
  const int cnt = max(0, min(c, n_t - t0));
  float2 pv[CMAX > 0 ? CMAX : 1];
  if constexpr (CMAX > 0) {
#pragma unroll
    for (int i = 0; i < CMAX; ++i) pv[i] = prow[min(i, c - 1) * kSelThreads + tid];
  }
  // the W1 row is gathered with the global token id (W1 is not sharded)
  const int x = clamp_token(xprev[(size_t)n * xstride], Vfull);
  Frag b[KC];
  load_b_row<BF16, KC, VW>(W1 + (size_t)x * r, r, lane, b);
  const float u = slot_uniform(seed, step.get(), req_ids[n], k, kPurposeDraft);
  // global merge in rank order (identical on every rank)
  float m = -INFINITY;
  for (int h = 0; h < G; ++h) m = fmaxf(m, summaries[(size_t)h * R + n].x);
  float S = 0.0f, P = 0.0f, own = 0.0f;
  for (int h = 0; h < G; ++h) {
    const float2 q = summaries[(size_t)h * R + n];
    const float sh_ = q.x == -INFINITY ? 0.0f : q.y * __expf(q.x - m);
    if (h < g) P += sh_;
    if (h == g) own = sh_;
    S += sh_;
  }
  const float T = u * S;
  const bool owner = P <= T && (g == G - 1 || T < P + own);  // workgroup-uniform
  if (!owner) {
    if (tid == 0) {
      tok_out[(size_t)n * ostride] = -1;
      p_out[(size_t)n * ostride] = 0.0f;
      lse_out[(size_t)n * ostride] = m + __logf(S);
    }
    return;
  }
  WaveSearch ws;
  if constexpr (CMAX > 0) {
    float w[CMAX];
#pragma unroll
    for (int i = 0; i < CMAX; ++i) w[i] = i < cnt ? pv[i].y * __expf(pv[i].x - m) : 0.0f;
    ws = block_tile_search<CMAX, true>([&](int i) { return w[i]; }, t0, cnt, T - P, sh);
  } else {
    ws = block_tile_search<0, true>([&](int i) {
      const float2 q = prow[i * kSelThreads + tid];
      return q.y * __expf(q.x - m);
    }, t0, cnt, T - P, sh);
  }
  if (tid >= kWave) return;  // wave 0 finishes; no barrier below
  const int t = min(max(ws.tstar, 0), n_t - 1);
  ATile<BF16, KC> at;
  load_a_tile<BF16, KC>(W2p, t, lane, at);
  const int v = t * kTileV + lane;
  const bool valid = v < Vg;
  const float uo = to_f32(U[(size_t)n * ldU + min(v, Vg - 1)]);
  __builtin_amdgcn_sched_barrier(0);  // all of the tile's loads before the first product
  f32x4 acc[4];
  tile_mma_regs<BF16, KC>(at, b, acc);
  const float zo = own_entry(acc, lane) + uo;
  const float e = valid ? __expf(zo - m) : 0.0f;
  const int sel = tile_pick(e, valid, ws.pb, ws.T, lane);
  const float esel = readlane_f(e, sel);
  if (lane == 0) {
    tok_out[(size_t)n * ostride] = v0 + t * kTileV + sel;
    p_out[(size_t)n * ostride] = esel / S;
    lse_out[(size_t)n * ostride] = m + __logf(S);
  }
}

// ---------------------------------------------------------------------------
// diagnostic: full logits of one slot
// ---------------------------------------------------------------------------

template <bool BF16, int KC>
__global__ __launch_bounds__(256) void markov_logits_kernel(
    const typename Elem<BF16>::T* __restrict__ U, long long ldU, bool vec,
    const typename Elem<BF16>::T* __restrict__ W1, const typename Elem<BF16>::T* __restrict__ W2p,
    const int* __restrict__ xprev, int R, int V, int r, int n_t, float* __restrict__ zout) {
  typedef typename Elem<BF16>::T T;
  constexpr int kpad = KC * kChunkK;
  constexpr int ldw = kpad + kLdsPad;
  __shared__ __align__(16) T w1s[16 * ldw];
  const int nb0 = blockIdx.y * kTileN;
  const int count = min(kTileN, R - nb0);
  stage_rows<BF16>(W1, xprev + nb0, 1, count, 16, r, V, kpad, ldw, w1s);
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int g = lane >> 4, nl = lane & 15;
  const int t = blockIdx.x * (blockDim.x / kWave) + wave;
  if (t >= n_t) return;  // wave-uniform; no barrier follows
  ATile<BF16, KC> at;
  load_a_tile<BF16, KC>(W2p, t, lane, at);
  f32x4 acc[4];
  tile_mma<BF16, KC>(at, w1s, ldw, lane, acc);
  const int n = nb0 + nl;
  const int v0 = t * kTileV + 16 * g;
  const int nvalid = min(16, V - v0);
  if (nl >= count || nvalid <= 0) return;
  float u16[16];
  load16<BF16>(U + (size_t)n * ldU + v0, nvalid, vec, u16);
  float z[16];
  tile_logits<BF16>(acc, u16, nvalid, true, z);
  for (int i = 0; i < nvalid; ++i) zout[(size_t)n * V + v0 + i] = z[i];
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Draft workspace: the request-major tile partials [R, ldn] (float2,
// ldn = 256 c, c = ceil(n_t / 256), tile t of request n at n * ldn +
// part_pos(t, c)), then the bookkeeping tail: the GEMM's tile-queue counters
// (one block of kQueueWordsPerGroup words per group of 128 requests), the
// draft uniforms and the resident kernel's hand-off block.
size_t markov_tail_offset(int R, int V) {
  return align_up((size_t)R * part_ld(V) * sizeof(float2), 256);
}
static size_t markov_queue_offset(int R, int V) { return markov_tail_offset(R, V); }
static size_t markov_u_offset(int R, int V) {
  return markov_queue_offset(R, V) + (size_t)queue_groups(R) * kQueueWordsPerGroup * 4;
}
size_t resident_bar_offset(int R, int V) { return markov_u_offset(R, V) + align_up((size_t)R * 4, 256); }
size_t markov_ws_bytes(int R, int V) { return resident_bar_offset(R, V) + kResidentBarBytes; }
static float* markov_u(float2* part, int R, int V) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(part) + markov_u_offset(R, V));
}
static unsigned* markov_queue(float2* part, int R, int V) {
  return reinterpret_cast<unsigned*>(reinterpret_cast<char*>(part) + markov_queue_offset(R, V));
}

template <bool BF16>
static bool u_vec_ok(const void* U, long long ldU, int V) {
  return rows_vec_ok(U, ldU, V, Elem<BF16>::kVec);
}

// Engine shape of a GEMM launch over Rg requests: waves per workgroup (4 up to
// four 16-request blocks, else 8) and the grid (up to two 4-wave or one
// 8-wave workgroup per CU).
static int partials_waves(int Rg) { return ceil_div(Rg, kTileN) <= 4 ? 4 : 8; }
static int partials_grid(int nw, int V) {
  return engine_grid(n_vtiles(V), device_cu_count() * (nw == 4 ? 2 : 1));
}

template <bool BF16, int KC, int NW, int NB>
static int launch_partials_cfg(const typename Elem<BF16>::T* Uk, long long ldU, bool vec,
                               const typename Elem<BF16>::T* W1, const typename Elem<BF16>::T* W2p,
                               const int32_t* xprev, int xstride, int Rg, int V, int r,
                               int w1_rows, float2* part, unsigned* queue,
                               DrawArgs draw, const ConfArgs& ca, int gamma, hipStream_t s) {
  typedef EngineGeom<BF16, KC, NW> G;
  const int n_t = n_vtiles(V);
  const int grid = partials_grid(NW, V);
  const int ldn = part_ld(V), c = part_chunk(V);
  if (vec)
    hipLaunchKernelGGL((markov_partials_kernel<BF16, KC, NW, NB, true>), dim3(grid), dim3(NW * kWave),
                       G::kLdsBytes, s, Uk, ldU, W1, W2p, xprev, xstride, Rg, V, r, n_t, w1_rows,
                       part, ldn, c, queue, draw, ca, gamma);
  else
    hipLaunchKernelGGL((markov_partials_kernel<BF16, KC, NW, NB, false>), dim3(grid),
                       dim3(NW * kWave), G::kLdsBytes, s, Uk, ldU, W1, W2p, xprev, xstride, Rg, V, r,
                       n_t, w1_rows, part, ldn, c, queue, draw, ca, gamma);
  return launch_status();
}

// One launch per group of up to 256 requests (the engine holds a group's W1
// rows in registers).
template <bool BF16, int KC>
static int launch_partials(const typename Elem<BF16>::T* Uk, long long ldU, bool vec,
                           const typename Elem<BF16>::T* W1, const typename Elem<BF16>::T* W2p,
                           const int32_t* xprev, int xstride, int R, int V, int r, int w1_rows,
                           float2* part, DrawArgs draw, const ConfArgs& ca, int gamma,
                           hipStream_t s) {
  unsigned* queue = markov_queue(part, R, V);
  const int ldn = part_ld(V);
  for (int g0 = 0; g0 < R; g0 += req_group<BF16>()) {
    const int Rg = std::min(req_group<BF16>(), R - g0);
    const int blocks = ceil_div(Rg, kTileN);
    const typename Elem<BF16>::T* Ug = Uk + (size_t)g0 * ldU;
    const int32_t* xg = xprev + (size_t)g0 * xstride;
    float2* pg = part + (size_t)g0 * ldn;
    unsigned* qg = queue + (size_t)(g0 / req_group<BF16>()) * kQueueWordsPerGroup;
    DrawArgs dg = draw;
    if (dg.u_out) {
      dg.u_out += g0;
      dg.req_ids += g0;
    }
    ConfArgs cg = ca;  // the group's rows of h and of the [R, gamma] outputs
    if (cg.h != nullptr) {
      cg.h = static_cast<const typename Elem<BF16>::T*>(cg.h) + (size_t)g0 * gamma * cg.d;
      cg.conf += (size_t)g0 * gamma;
      cg.surv += (size_t)g0 * gamma;
      if (cg.logit != nullptr) cg.logit += (size_t)g0 * gamma;
    }
    int st;
    if (partials_waves(Rg) == 4)
      st = launch_partials_cfg<BF16, KC, 4, 1>(Ug, ldU, vec, W1, W2p, xg, xstride, Rg, V, r, w1_rows, pg, qg, dg, cg, gamma, s);
    else if (blocks <= 8)
      st = launch_partials_cfg<BF16, KC, 8, 1>(Ug, ldU, vec, W1, W2p, xg, xstride, Rg, V, r, w1_rows, pg, qg, dg, cg, gamma, s);
    else if constexpr (BF16)
      st = launch_partials_cfg<BF16, KC, 8, 2>(Ug, ldU, vec, W1, W2p, xg, xstride, Rg, V, r, w1_rows, pg, qg, dg, cg, gamma, s);
    else
      st = DSPARK_ESIZE;  // unreachable: float32 groups hold at most 8 blocks
    if (st) return st;
  }
  return DSPARK_OK;
}

template <bool BF16, int KC>
static int launch_select(const typename Elem<BF16>::T* Uk, long long ldU, bool vec, bool vec_w1,
                         const typename Elem<BF16>::T* W1, const typename Elem<BF16>::T* W2p,
                         const int32_t* xprev, int xstride, int R, int V, int r,
                         const float2* part, uint64_t seed, StepArg step,
                         const uint32_t* req_ids, int k, int32_t* tok, float* p, float* lse,
                         int ostride, const float* u_pre, hipStream_t s) {
  const int n_t = n_vtiles(V), c = part_chunk(V), ldn = part_ld(V);
  unsigned* queue = markov_queue(const_cast<float2*>(part), R, V);
  const int n_queue = queue_groups(R) * kNumXcd;  // counters, kQueueStride words apart
#define DSPARK_SELECT(CM)                                                                         \
  if (vec_w1)                                                                                    \
    hipLaunchKernelGGL((markov_select_kernel<BF16, KC, CM, true>), dim3(R), dim3(kSelThreads), 0, s, Uk, \
                       ldU, W1, W2p, xprev, xstride, V, r, n_t, part, ldn, c, seed, step,         \
                       req_ids, k, tok, p, lse, ostride, queue, n_queue, u_pre);                 \
  else                                                                                           \
    hipLaunchKernelGGL((markov_select_kernel<BF16, KC, CM, false>), dim3(R), dim3(kSelThreads), 0, s, \
                       Uk, ldU, W1, W2p, xprev, xstride, V, r, n_t, part, ldn, c, seed,           \
                       step, req_ids, k, tok, p, lse, ostride, queue, n_queue, u_pre)
  // the partial row in registers, unrolled to the smallest of 8 / 10 / 12 /
  // 16 chunks that holds it (masked iterations cost as much as live ones;
  // 8 and 10 chunks are vocabularies up to 131072 and 163840)
  if (c <= 8) {
    DSPARK_SELECT(8);
  } else if (c <= 10) {
    DSPARK_SELECT(10);
  } else if (c <= 12) {
    DSPARK_SELECT(12);
  } else if (c <= 16) {
    DSPARK_SELECT(16);
  } else {
    DSPARK_SELECT(0);
  }
#undef DSPARK_SELECT
  return launch_status();
}

template <bool BF16, int KC>
static int launch_shard_select(const void* U, long long ldU, const void* W1, const void* W2p,
                               const int32_t* xprev, int xstride, const float2* part,
                               const float2* summaries, int G, int g, int v0, uint64_t seed,
                               StepArg step, const uint32_t* req_ids, int k, int R, int Vg,
                               int Vfull, int r, int32_t* tok, float* p, float* lse, int ostride,
                               hipStream_t s) {
  typedef typename Elem<BF16>::T T;
  const int n_t = n_vtiles(Vg), c = part_chunk(Vg), ldn = part_ld(Vg);
  unsigned* queue = markov_queue(const_cast<float2*>(part), R, Vg);
  const int n_queue = queue_groups(R) * kNumXcd;
  const T* Ub = static_cast<const T*>(U);
  const T* W1b = static_cast<const T*>(W1);
  const T* W2b = static_cast<const T*>(W2p);
#define DSPARK_SHSEL(CM, VW_)                                                                     \
  hipLaunchKernelGGL((markov_shard_select_kernel<BF16, KC, CM, VW_>), dim3(R), dim3(kSelThreads), 0, \
                     s, Ub, ldU, W1b, W2b, xprev, xstride, Vg, Vfull, r, n_t, part, ldn, c,        \
                     summaries, R, G, g, v0, seed, step, req_ids, k, tok, p, lse, ostride, queue,  \
                     n_queue)
  const bool vw = w1_vec_ok(W1, r);
  if (c <= 16) {
    if (vw) DSPARK_SHSEL(16, true); else DSPARK_SHSEL(16, false);
  } else {
    if (vw) DSPARK_SHSEL(0, true); else DSPARK_SHSEL(0, false);
  }
#undef DSPARK_SHSEL
  return launch_status();
}

template <bool BF16, int KC>
static int launch_markov(const void* U, const void* W1, const void* W2p, const int32_t* anchor,
                         uint64_t seed, StepArg step, const uint32_t* req_ids, int R, int gamma,
                         int V, int r, int32_t* tokens, float* p_draft, float* lse_draft,
                         float2* part, const ConfArgs& ca, hipStream_t s) {
  typedef typename Elem<BF16>::T T;
  const T* Ub = static_cast<const T*>(U);
  const T* W1b = static_cast<const T*>(W1);
  const T* W2b = static_cast<const T*>(W2p);
  const long long ldU = (long long)gamma * V;
  const bool vec_u = u_vec_ok<BF16>(U, ldU, V), vec_w1 = w1_vec_ok(W1, r);
  for (int k = 1; k <= gamma; ++k) {
    const int* xprev = (k == 1) ? anchor : tokens + (k - 2);
    const int xstride = (k == 1) ? 1 : gamma;
    const T* Uk = Ub + (size_t)(k - 1) * V;
    const DrawArgs draw{seed, step, req_ids, k, markov_u(part, R, V)};
    int st = launch_partials<BF16, KC>(Uk, ldU, vec_u && vec_w1, W1b, W2b, xprev, xstride, R, V, r,
                                       V, part, draw, ca, gamma, s);
    if (st) return st;
    st = launch_select<BF16, KC>(Uk, ldU, vec_u, vec_w1, W1b, W2b, xprev, xstride, R, V, r, part,
                                 seed, step, req_ids, k, tokens + (k - 1), p_draft + (k - 1),
                                 lse_draft + (k - 1), gamma, draw.u_out, s);
    if (st) return st;
  }
  return DSPARK_OK;
}

template <bool BF16, int KC>
static int launch_partials_api(const void* U, long long ldU, const void* W1, const void* W2p,
                               const int32_t* x_prev, int xstride, int R, int V, int r,
                               int w1_rows, float2* part, hipStream_t s) {
  typedef typename Elem<BF16>::T T;
  const bool vec = u_vec_ok<BF16>(U, ldU, V) && w1_vec_ok(W1, r);
  const DrawArgs none{0, StepArg{0, nullptr}, nullptr, 0, nullptr};
  return launch_partials<BF16, KC>(static_cast<const T*>(U), ldU, vec, static_cast<const T*>(W1),
                                   static_cast<const T*>(W2p), x_prev, xstride, R, V, r, w1_rows,
                                   part, none, ConfArgs{}, 1, s);
}

template <bool BF16, int KC>
static int launch_logits(const void* U, long long ldU, const void* W1, const void* W2p,
                         const int32_t* x_prev, int R, int V, int r, float* z, hipStream_t s) {
  typedef typename Elem<BF16>::T T;
  const int n_t = n_vtiles(V);
  const bool vec = (V % Elem<BF16>::kVec) == 0 && (ldU % Elem<BF16>::kVec) == 0 &&
                   (reinterpret_cast<uintptr_t>(U) % 16) == 0;
  dim3 grid(ceil_div(n_t, 4), ceil_div(R, kTileN));
  hipLaunchKernelGGL((markov_logits_kernel<BF16, KC>), grid, dim3(256), 0, s,
                     static_cast<const T*>(U), ldU, vec, static_cast<const T*>(W1),
                     static_cast<const T*>(W2p), x_prev, R, V, r, n_t, z);
  return launch_status();
}

}  // namespace dspark

using namespace dspark;

extern "C" size_t dspark_prepacked_w2_bytes(int r, int V, int dtype) {
  if (!dtype_ok(dtype) || r < 1 || V < 1) return 0;
  if (r > (dtype == DSPARK_BF16 ? kMaxRankBf16 : kMaxRankF32)) return 0;
  return (size_t)n_vtiles(V) * kc_instance(r) * 4 * kWave * 8 * dtype_bytes(dtype);
}

extern "C" int dspark_prepack_w2(const void* W2, int r, int V, int dtype, void* W2p,
                                 size_t W2p_bytes, void* stream) {
  if (!dtype_ok(dtype)) return DSPARK_EDTYPE;
  if (!W2 || !W2p) return DSPARK_EINVAL;
  const size_t need = dspark_prepacked_w2_bytes(r, V, dtype);
  if (need == 0) return DSPARK_ESIZE;
  if (W2p_bytes < need) return DSPARK_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int KC = kc_instance(r), n_t = n_vtiles(V);
  const long long groups = (long long)n_t * KC * 4 * kWave;
  const int grid = (int)std::min<long long>((groups + 255) / 256, 65535);
  if (dtype == DSPARK_BF16)
    hipLaunchKernelGGL(prepack_w2_kernel<uint16_t>, dim3(grid), dim3(256), 0, s,
                       static_cast<const uint16_t*>(W2), r, V, KC, n_t, static_cast<uint16_t*>(W2p));
  else
    hipLaunchKernelGGL(prepack_w2_kernel<float>, dim3(grid), dim3(256), 0, s,
                       static_cast<const float*>(W2), r, V, KC, n_t, static_cast<float*>(W2p));
  return launch_status();
}

#define DSPARK_KC_DISPATCH(BF, fn, ...)                         \
  switch (kc_instance(r)) {                                     \
    case 1: return fn<BF, 1>(__VA_ARGS__);                      \
    case 2: return fn<BF, 2>(__VA_ARGS__);                      \
    case 4: return fn<BF, 4>(__VA_ARGS__);                      \
    default: return fn<BF, 8>(__VA_ARGS__);                     \
  }

static int markov_dispatch(const void* U, const void* W1, const void* W2p, const int32_t* anchor,
                           uint64_t seed, StepArg step, const uint32_t* req_ids, int R, int gamma,
                           int V, int r, int dtype, int32_t* tokens, float* p, float* lse,
                           float2* part, const ConfArgs& ca, hipStream_t s) {
  if (resident_draft_eligible(U, W1, R, gamma, V, r, dtype))
    return resident_draft_launch(U, W1, W2p, anchor, seed, step, req_ids, R, gamma, V, r, tokens,
                                 p, lse, part, ca, s);
  if (dtype == DSPARK_BF16) {
    DSPARK_KC_DISPATCH(true, launch_markov, U, W1, W2p, anchor, seed, step, req_ids, R, gamma, V,
                       r, tokens, p, lse, part, ca, s)
  }
  switch (kc_instance(r)) {
    case 1: return launch_markov<false, 1>(U, W1, W2p, anchor, seed, step, req_ids, R, gamma, V, r, tokens, p, lse, part, ca, s);
    case 2: return launch_markov<false, 2>(U, W1, W2p, anchor, seed, step, req_ids, R, gamma, V, r, tokens, p, lse, part, ca, s);
    default: return launch_markov<false, 4>(U, W1, W2p, anchor, seed, step, req_ids, R, gamma, V, r, tokens, p, lse, part, ca, s);
  }
}

namespace dspark {
int markov_draft_checked(const void* U, const void* W1, const void* W2p, const int32_t* anchor,
                         uint64_t seed, StepArg step, const uint32_t* req_ids, int R, int gamma,
                         int V, int r, int dtype, int32_t* tokens, float* p_draft, float* lse_draft,
                         void* ws, hipStream_t s) {
  return markov_dispatch(U, W1, W2p, anchor, seed, step, req_ids, R, gamma, V, r, dtype, tokens,
                         p_draft, lse_draft, static_cast<float2*>(ws), ConfArgs{}, s);
}
}  // namespace dspark

extern "C" int dspark_markov_draft(const void* U, const void* W1, const void* W2p,
                                   const int32_t* anchor, uint64_t seed, uint64_t step,
                                   const uint64_t* step_dev, const uint32_t* req_ids, int R, int gamma, int V, int r,
                                   int dtype, int32_t* tokens, float* p_draft, float* lse_draft,
                                   void* ws, size_t ws_bytes, void* stream) {
  int st = check_sizes(R, gamma, V, r, dtype);
  if (st) return st;
  if (!U || !W1 || !W2p || !anchor || !req_ids || !tokens || !p_draft || !lse_draft)
    return DSPARK_EINVAL;
  if (!ws || ws_bytes < markov_ws_bytes(R, V)) return DSPARK_EWORKSPACE;
  return markov_draft_checked(U, W1, W2p, anchor, seed, StepArg{step, step_dev}, req_ids, R, gamma,
                              V, r, dtype, tokens, p_draft, lse_draft, ws,
                              static_cast<hipStream_t>(stream));
}

// The confidence head rides in the GEMM prologue (one wave per request, in
// workgroups 0 .. R-1) when at most a quarter of the GEMM's workgroups carry a
// request, so that the queue hands their share of tiles to the others; with
// more requests every workgroup would start late and the head runs as a
// launch of its own after the draft (the same values either way).
static bool conf_in_prologue(int R, int V, bool bf16) {
  const int group = bf16 ? req_group<true>() : req_group<false>();
  if (R > group) return false;
  return 4 * R <= partials_grid(partials_waves(R), V);
}

extern "C" int dspark_markov_draft_confidence(
    const void* U, const void* W1, const void* W2p, const int32_t* anchor, uint64_t seed,
    uint64_t step, const uint64_t* step_dev, const uint32_t* req_ids, int R, int gamma, int V,
    int r, int dtype, const void* h, const float* w, float b, const float* inv_temp, int d,
    int32_t* tokens, float* p_draft, float* lse_draft, float* conf, float* surv, float* logit,
    void* ws, size_t ws_bytes, void* stream) {
  int st = check_sizes(R, gamma, V, r, dtype);
  if (st) return st;
  if (d < 1) return DSPARK_ESIZE;
  if (!U || !W1 || !W2p || !anchor || !req_ids || !tokens || !p_draft || !lse_draft || !h || !w ||
      !conf || !surv)
    return DSPARK_EINVAL;
  if (!ws || ws_bytes < markov_ws_bytes(R, V)) return DSPARK_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool resident = resident_draft_eligible(U, W1, R, gamma, V, r, dtype);
  if (!resident && !conf_in_prologue(R, V, dtype == DSPARK_BF16)) {
    // every GEMM workgroup would carry a request: the head as a launch of its own
    st = markov_dispatch(U, W1, W2p, anchor, seed, StepArg{step, step_dev}, req_ids, R, gamma, V,
                         r, dtype, tokens, p_draft, lse_draft, static_cast<float2*>(ws),
                         ConfArgs{}, s);
    if (st) return st;
    return dspark_confidence(h, W1, anchor, tokens, w, b, inv_temp, R, gamma, d, V, r, dtype, conf,
                             surv, logit, stream);
  }
  ConfArgs ca;
  ca.h = h;
  ca.w = w;
  ca.b = b;
  ca.inv_temp = inv_temp;
  ca.d = d;
  confidence_vec_flags(h, W1, w, d, r, dtype, ca.vec_h, ca.vec_w1);
  ca.conf = conf;
  ca.surv = surv;
  ca.logit = logit;
  return markov_dispatch(U, W1, W2p, anchor, seed, StepArg{step, step_dev}, req_ids, R, gamma, V,
                         r, dtype, tokens, p_draft, lse_draft, static_cast<float2*>(ws), ca, s);
}

static int logits_dispatch(const void* U, long long ldU, const void* W1, const void* W2p,
                           const int32_t* x_prev, int R, int V, int r, int dtype, float* z,
                           hipStream_t s) {
  if (dtype == DSPARK_BF16) {
    DSPARK_KC_DISPATCH(true, launch_logits, U, ldU, W1, W2p, x_prev, R, V, r, z, s)
  }
  switch (kc_instance(r)) {
    case 1: return launch_logits<false, 1>(U, ldU, W1, W2p, x_prev, R, V, r, z, s);
    case 2: return launch_logits<false, 2>(U, ldU, W1, W2p, x_prev, R, V, r, z, s);
    default: return launch_logits<false, 4>(U, ldU, W1, W2p, x_prev, R, V, r, z, s);
  }
}

extern "C" int dspark_markov_logits(const void* U_k, long long ldU, const void* W1,
                                    const void* W2p, const int32_t* x_prev, int R, int V, int r,
                                    int dtype, float* z, void* stream) {
  int st = check_sizes(R, 1, V, r, dtype);
  if (st) return st;
  if (!U_k || !W1 || !W2p || !x_prev || !z) return DSPARK_EINVAL;
  if (ldU < V) return DSPARK_ESIZE;
  return logits_dispatch(U_k, ldU, W1, W2p, x_prev, R, V, r, dtype, z,
                         static_cast<hipStream_t>(stream));
}

static int partials_dispatch(const void* U, long long ldU, const void* W1, const void* W2p,
                             const int32_t* x_prev, int xstride, int R, int V, int r, int w1_rows,
                             int dtype, float2* part, hipStream_t s) {
  if (dtype == DSPARK_BF16) {
    DSPARK_KC_DISPATCH(true, launch_partials_api, U, ldU, W1, W2p, x_prev, xstride, R, V, r, w1_rows,
                       part, s)
  }
  switch (kc_instance(r)) {
    case 1: return launch_partials_api<false, 1>(U, ldU, W1, W2p, x_prev, xstride, R, V, r, w1_rows, part, s);
    case 2: return launch_partials_api<false, 2>(U, ldU, W1, W2p, x_prev, xstride, R, V, r, w1_rows, part, s);
    default: return launch_partials_api<false, 4>(U, ldU, W1, W2p, x_prev, xstride, R, V, r, w1_rows, part, s);
  }
}

extern "C" int dspark_markov_partials(const void* U_k, long long ldU, const void* W1,
                                      const void* W2p, const int32_t* x_prev, int xstride, int R,
                                      int V, int r, int dtype, void* part, size_t part_bytes,
                                      void* stream) {
  int st = check_sizes(R, 1, V, r, dtype);
  if (st) return st;
  if (!U_k || !W1 || !W2p || !x_prev || !part) return DSPARK_EINVAL;
  if (ldU < V || xstride < 1) return DSPARK_ESIZE;
  if (part_bytes < markov_ws_bytes(R, V)) return DSPARK_EWORKSPACE;
  return partials_dispatch(U_k, ldU, W1, W2p, x_prev, xstride, R, V, r, V, dtype,
                           static_cast<float2*>(part), static_cast<hipStream_t>(stream));
}

extern "C" int dspark_markov_shard_partials(const void* U_k, long long ldU, const void* W1,
                                            const void* W2p, const int32_t* x_prev, int xstride,
                                            int R, int V_g, int V, int r, int dtype, void* part,
                                            size_t part_bytes, void* stream) {
  int st = check_sizes(R, 1, V, r, dtype);
  if (st) return st;
  if (!U_k || !W1 || !W2p || !x_prev || !part) return DSPARK_EINVAL;
  if (V_g < 1 || V_g > V || ldU < V_g || xstride < 1) return DSPARK_ESIZE;
  if (part_bytes < markov_ws_bytes(R, V_g)) return DSPARK_EWORKSPACE;
  return partials_dispatch(U_k, ldU, W1, W2p, x_prev, xstride, R, V_g, r, V, dtype,
                           static_cast<float2*>(part), static_cast<hipStream_t>(stream));
}

template <bool BF16, int KC>
static int launch_select_api(const void* U, long long ldU, const void* W1, const void* W2p,
                             const int32_t* x_prev, int xstride, const float2* part, uint64_t seed,
                             StepArg step, const uint32_t* req_ids, int k, int R, int V, int r,
                             int32_t* tok, float* p, float* lse, int ostride, hipStream_t s) {
  typedef typename Elem<BF16>::T T;
  return launch_select<BF16, KC>(static_cast<const T*>(U), ldU, u_vec_ok<BF16>(U, ldU, V),
                                 w1_vec_ok(W1, r), static_cast<const T*>(W1),
                                 static_cast<const T*>(W2p), x_prev, xstride, R, V, r, part, seed,
                                 step, req_ids, k, tok, p, lse, ostride, nullptr, s);
}

extern "C" int dspark_markov_select(const void* U_k, long long ldU, const void* W1,
                                    const void* W2p, const int32_t* x_prev, int xstride,
                                    const void* part, uint64_t seed, uint64_t step,
                                    const uint64_t* step_dev, const uint32_t* req_ids, int k, int R, int V, int r, int dtype,
                                    int32_t* tok_out, float* p_out, float* lse_out, int ostride,
                                    void* stream) {
  int st = check_sizes(R, 1, V, r, dtype);
  if (st) return st;
  if (!U_k || !W1 || !W2p || !x_prev || !part || !req_ids || !tok_out || !p_out || !lse_out)
    return DSPARK_EINVAL;
  if (ldU < V || xstride < 1 || ostride < 1 || k < 1 || k > kMaxGamma + 1) return DSPARK_ESIZE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float2* pt = static_cast<const float2*>(part);
  const StepArg sa{step, step_dev};
#define DSPARK_SEL_ARGS U_k, ldU, W1, W2p, x_prev, xstride, pt, seed, sa, req_ids, k, R, V, r, \
                        tok_out, p_out, lse_out, ostride, s
  if (dtype == DSPARK_BF16) {
    switch (kc_instance(r)) {
      case 1: return launch_select_api<true, 1>(DSPARK_SEL_ARGS);
      case 2: return launch_select_api<true, 2>(DSPARK_SEL_ARGS);
      case 4: return launch_select_api<true, 4>(DSPARK_SEL_ARGS);
      default: return launch_select_api<true, 8>(DSPARK_SEL_ARGS);
    }
  }
  switch (kc_instance(r)) {
    case 1: return launch_select_api<false, 1>(DSPARK_SEL_ARGS);
    case 2: return launch_select_api<false, 2>(DSPARK_SEL_ARGS);
    default: return launch_select_api<false, 4>(DSPARK_SEL_ARGS);
  }
#undef DSPARK_SEL_ARGS
}

extern "C" int dspark_markov_shard_summary(const void* part, size_t part_bytes, int R, int V_g,
                                           float* summary, void* stream) {
  if (R < 1 || R > kMaxRows || V_g < 1) return DSPARK_ESIZE;
  if (!part || !summary) return DSPARK_EINVAL;
  if (part_bytes < markov_ws_bytes(R, V_g)) return DSPARK_EWORKSPACE;
  const int n_t = n_vtiles(V_g), c = part_chunk(V_g), ldn = part_ld(V_g);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float2* pt = static_cast<const float2*>(part);
  float2* out = reinterpret_cast<float2*>(summary);
  if (c <= 16)
    hipLaunchKernelGGL(markov_shard_summary_kernel<16>, dim3(R), dim3(kSelThreads), 0, s, pt, ldn,
                       c, n_t, out);
  else
    hipLaunchKernelGGL(markov_shard_summary_kernel<0>, dim3(R), dim3(kSelThreads), 0, s, pt, ldn, c,
                       n_t, out);
  return launch_status();
}

extern "C" int dspark_markov_shard_select(const void* U_k, long long ldU, const void* W1,
                                          const void* W2p, const int32_t* x_prev, int xstride,
                                          const void* part, const float* summaries, int G, int g,
                                          int v0, uint64_t seed, uint64_t step,
                                          const uint64_t* step_dev, const uint32_t* req_ids, int k,
                                          int R, int V_g, int V, int r, int dtype,
                                          int32_t* tok_out, float* p_out, float* lse_out,
                                          int ostride, void* stream) {
  int st = check_sizes(R, 1, V, r, dtype);
  if (st) return st;
  if (!U_k || !W1 || !W2p || !x_prev || !part || !summaries || !req_ids || !tok_out || !p_out ||
      !lse_out)
    return DSPARK_EINVAL;
  if (G < 1 || G > 64 || g < 0 || g >= G || V_g < 1 || v0 < 0 || (long long)v0 + V_g > V)
    return DSPARK_ESIZE;
  if (ldU < V_g || xstride < 1 || ostride < 1 || k < 1 || k > kMaxGamma + 1) return DSPARK_ESIZE;
  const StepArg sa{step, step_dev};
  const float2* pt = static_cast<const float2*>(part);
  const float2* sm = reinterpret_cast<const float2*>(summaries);
  hipStream_t s = static_cast<hipStream_t>(stream);
#define DSPARK_SHARD_ARGS U_k, ldU, W1, W2p, x_prev, xstride, pt, sm, G, g, v0, seed, sa, req_ids, \
                          k, R, V_g, V, r, tok_out, p_out, lse_out, ostride, s
  if (dtype == DSPARK_BF16) {
    switch (kc_instance(r)) {
      case 1: return launch_shard_select<true, 1>(DSPARK_SHARD_ARGS);
      case 2: return launch_shard_select<true, 2>(DSPARK_SHARD_ARGS);
      case 4: return launch_shard_select<true, 4>(DSPARK_SHARD_ARGS);
      default: return launch_shard_select<true, 8>(DSPARK_SHARD_ARGS);
    }
  }
  switch (kc_instance(r)) {
    case 1: return launch_shard_select<false, 1>(DSPARK_SHARD_ARGS);
    case 2: return launch_shard_select<false, 2>(DSPARK_SHARD_ARGS);
    default: return launch_shard_select<false, 4>(DSPARK_SHARD_ARGS);
  }
#undef DSPARK_SHARD_ARGS
}
