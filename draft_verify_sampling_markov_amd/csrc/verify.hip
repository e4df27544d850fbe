// Lossless rejection-sampling verification on gfx950.
//
// DSpark digest ("DSpark: Confidence-Scheduled Speculative Decoding with
// Semi-Autoregressive Generation", zhao9797.github.io): the target checks the
// drafted block in one forward and rejection sampling keeps the longest prefix
// that conforms; every draft probability is an exact softmax ("Architecture
// (drafter)"), which is what makes the check lossless. SGLang DSpark blog,
// "Verify modes": static verifies the whole block, compact the scheduled
// window, cap-accept the whole block while committing only the window (same
// commit as compact, plus the ceiling).
//
// Four launches, no host read-back:
//   row_partials      every packed target row, split in vocabulary chunks:
//                     (max, sum of exp) partials -- the bandwidth-bound pass
//   decide            one wave per request: merge a row's partials into its
//                     log-sum-exp, p_t(x_k), the accept test u < p_t / p_d per
//                     slot, the accepted length, and the correction job
//                     (residual at slot A+1, or bonus at slot L+1)
//   residual_partials per 64-entry vocabulary tile: recompute the draft logits
//                     of each request's job slot on the matrix cores, form
//                     q = max(0, p_t - p_d) (or p_t for a bonus), and emit
//                     per-tile sums of q and of p_t
//   residual_select   one workgroup per request: find the tile where the
//                     cumulative mass crosses u * sum, recompute that tile
//                     with the same code and finish the inverse-CDF search;
//                     write the token
#include "dspark_device.hpp"
#include "dspark_host.hpp"
#include "tile_engine.hpp"

#include <algorithm>

namespace dspark {

// vocabulary entries per row-partial workgroup, 32 per thread (measured on
// MI355X: 16384 entries over 512 threads beat 8192 over 256 by 2-8%)
constexpr int kRowChunk = 16384;
constexpr int kRowThreads = 512;

inline int n_row_chunks(int V) { return ceil_div(V, kRowChunk); }

// correction job of one request (structure of arrays in the workspace)
struct Jobs {
  int* kind;    // 0 residual, 1 bonus
  int* slot;    // 1-based slot of the correction token
  int* trow;    // packed target row of that slot
  int* xprev;   // token before the slot (anchor for slot 1)
  float* u;     // uniform of the draw
  float* lse_t; // target log-sum-exp of trow
  float* lse_d; // draft log-sum-exp of the slot (residual only)
};

// ---------------------------------------------------------------------------
// row partials
// ---------------------------------------------------------------------------

// Every load of the chunk is issued before the first value is used: addresses
// are clamped into the chunk and out-of-range values replaced afterwards (a
// branch around a load would make the compiler wait for it before the next
// one goes out). On the vector path V and the chunk bounds are multiples of
// the vector width, so a vector lies wholly inside or wholly outside.
template <bool BF16, bool VECP>
__global__ __launch_bounds__(kRowThreads) void row_partials_kernel(
    const typename Elem<BF16>::T* __restrict__ target, int V, int n_chunks,
    const int* __restrict__ cu_seqlens, int R, int rows_ws, float2* __restrict__ part) {
  typedef typename Elem<BF16>::T T;
  constexpr int VEC = Elem<BF16>::kVec;
  constexpr int PER = kRowChunk / kRowThreads;  // 32 entries per thread
  __shared__ float red[kRowThreads / kWave];
  const int row = blockIdx.y;
  if (row >= min(cu_seqlens[R], rows_ws)) return;  // block-uniform
  const int c = blockIdx.x;
  const int v_begin = c * kRowChunk;
  const int v_end = min(V, v_begin + kRowChunk);
  const T* z = target + (size_t)row * V;
  const int tid = threadIdx.x;
  float vals[PER];
  if constexpr (VECP) {
    u32x4 q[PER / VEC];
#pragma unroll
    for (int it = 0; it < PER / VEC; ++it) {
      const int v = v_begin + (it * kRowThreads + tid) * VEC;
      q[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(z + min(v, v_end - VEC)));
    }
#pragma unroll
    for (int it = 0; it < PER / VEC; ++it) {
      const bool ok = v_begin + (it * kRowThreads + tid) * VEC < v_end;
      if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vals[it * VEC + 2 * i] = ok ? __uint_as_float(q[it][i] << 16) : -INFINITY;
          vals[it * VEC + 2 * i + 1] = ok ? __uint_as_float(q[it][i] & 0xFFFF0000u) : -INFINITY;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) vals[it * VEC + i] = ok ? __uint_as_float(q[it][i]) : -INFINITY;
      }
    }
  } else {
    T raw[PER];
#pragma unroll
    for (int it = 0; it < PER; ++it) raw[it] = z[min(v_begin + it * kRowThreads + tid, v_end - 1)];
#pragma unroll
    for (int it = 0; it < PER; ++it)
      vals[it] = v_begin + it * kRowThreads + tid < v_end ? to_f32(raw[it]) : -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER; ++i) m = fmaxf(m, vals[i]);
  m = wave_max(m);
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  if (lane == 0) red[wave] = m;
  __syncthreads();
  float mb = red[0];
#pragma unroll
  for (int w = 1; w < kRowThreads / kWave; ++w) mb = fmaxf(mb, red[w]);
  __syncthreads();
  float s = 0.0f;
  if (mb != -INFINITY) {
#pragma unroll
    for (int i = 0; i < PER; ++i) s += __expf(vals[i] - mb);
  }
  s = wave_sum(s);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  if (tid == 0) {
    float sb = 0.0f;
#pragma unroll
    for (int w = 0; w < kRowThreads / kWave; ++w) sb += red[w];
    part[(size_t)row * n_chunks + c] = make_float2(mb, sb);
  }
}

// ---------------------------------------------------------------------------
// decide
// ---------------------------------------------------------------------------

// One wave per request, lane l for slot l + 1 (its packed row c0 + l). Every
// load is issued up front from clamped addresses (no branch around a load);
// one Philox block per lane gives that slot's accept, residual and bonus
// uniforms, so the correction job's uniform is a lane pick once A is known.
// CMAX > 0: the row's chunk partials (n_chunks <= CMAX) sit in registers.
template <bool BF16, int CMAX>
__global__ __launch_bounds__(256) void decide_kernel(
    const typename Elem<BF16>::T* __restrict__ target, int V, int n_chunks,
    const float2* __restrict__ part, const int* __restrict__ cu_seqlens,
    const int* __restrict__ anchor, const int* __restrict__ tokens,
    const float* __restrict__ p_draft, const float* __restrict__ lse_draft,
    const int* __restrict__ win_len, int mode, uint64_t seed, StepArg step,
    const uint32_t* __restrict__ req_ids, int R, int gamma, int rows_ws, Jobs jobs,
    int* __restrict__ accept_len,
    int* __restrict__ out_tokens, int* __restrict__ n_out, int* __restrict__ ceiling) {
  const int lane = threadIdx.x & (kWave - 1);
  const int req = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (req >= R) return;  // wave-uniform, no barriers below
  // rows of this request, clamped into the row workspace (a well-formed
  // cu_seqlens never needs the clamp)
  const int c0 = min(max(cu_seqlens[req], 0), rows_ws - 1);
  const int c1 = min(max(cu_seqlens[req + 1], c0 + 1), rows_ws);
  const int Lv = min(c1 - c0 - 1, gamma);
  const int jl = min(lane, gamma - 1);  // this lane's slot, clamped for the loads
  const int tok = tokens[(size_t)req * gamma + jl];
  const float pd = p_draft[(size_t)req * gamma + jl];
  const float lsed = lse_draft[(size_t)req * gamma + jl];
  const int anc = anchor[req];
  const uint64_t stp = step.get();
  const int wl = mode == DSPARK_VERIFY_CAP_ACCEPT ? win_len[req] : gamma;
  const int row = c0 + min(lane, Lv);
  const float zt = to_f32(target[(size_t)row * V + clamp_token(tok, V)]);
  float m = -INFINITY, S = 0.0f;
  if constexpr (CMAX > 0) {  // all partials of the row in flight at once
    float2 pv[CMAX];
#pragma unroll
    for (int c = 0; c < CMAX; ++c) pv[c] = part[(size_t)row * n_chunks + min(c, n_chunks - 1)];
#pragma unroll
    for (int c = 0; c < CMAX; ++c) m = fmaxf(m, c < n_chunks ? pv[c].x : -INFINITY);
#pragma unroll
    for (int c = 0; c < CMAX; ++c) S += c < n_chunks ? pv[c].y * __expf(pv[c].x - m) : 0.0f;
  } else {
    for (int c = 0; c < n_chunks; ++c) m = fmaxf(m, part[(size_t)row * n_chunks + c].x);
    for (int c = 0; c < n_chunks; ++c) {
      const float2 pv = part[(size_t)row * n_chunks + c];
      S += pv.y * __expf(pv.x - m);
    }
  }
  // this lane's Philox block (slot lane + 1): accept, residual and bonus words
  const U64x4 blk = philox4x64_10((uint64_t)(lane + 1), (uint64_t)req_ids[req], stp, 0ull, seed, 0ull);
  const float to24 = 5.9604644775390625e-8f;  // 2^-24
  const float u_acc = (float)(uint32_t)(blk.w[kPurposeAccept] >> 40) * to24;
  const float u_res = (float)(uint32_t)(blk.w[kPurposeResidual] >> 40) * to24;
  const float u_bon = (float)(uint32_t)(blk.w[kPurposeBonus] >> 40) * to24;
  const float lse = m + __logf(S);
  const float pt = __expf(zt - lse);
  const float ratio = pt / pd;
  const bool acc = lane < Lv && u_acc < ratio;

  const unsigned long long mask = __ballot(acc);
  const int A_full = min(__ffsll((long long)~mask) - 1, Lv);
  const int Lc = mode == DSPARK_VERIFY_CAP_ACCEPT ? min(min(max(wl, 0), gamma), Lv) : Lv;
  const int A = min(A_full, Lc);
  const bool residual = A < Lc;
  const int slot = residual ? A + 1 : Lc + 1;
  const int rel = slot - 1;  // packed row offset of the slot's target row, a lane index
  const float lse_t = readlane_f(lse, rel);
  const float u_job = readlane_f(residual ? u_res : u_bon, rel);
  const int xprev = A == 0 ? anc : __builtin_amdgcn_readlane(tok, A - 1);
  const float lse_d = residual ? readlane_f(lsed, A) : 0.0f;
  if (lane == 0) {
    jobs.kind[req] = residual ? 0 : 1;
    jobs.slot[req] = slot;
    jobs.trow[req] = c0 + rel;
    jobs.xprev[req] = xprev;
    jobs.u[req] = u_job;
    jobs.lse_t[req] = lse_t;
    jobs.lse_d[req] = lse_d;
    accept_len[req] = A;
    n_out[req] = A + 1;
    if (ceiling) ceiling[req] = A_full;
  }
  if (lane <= gamma && lane != A)
    out_tokens[(size_t)req * (gamma + 1) + lane] = lane < A ? tok : -1;
}

// ---------------------------------------------------------------------------
// residual / bonus weights
// ---------------------------------------------------------------------------

// exp(z - lse) as 2^(z log2 e + b) with b = -lse log2 e (one fused
// multiply-add before the exponential; b is rounded once per request)
__device__ __forceinline__ float shifted_exp(float z, float b) {
  return __builtin_amdgcn_exp2f(fmaf(z, kLog2e, b));
}
__device__ __forceinline__ float exp_shift(float lse) { return -lse * kLog2e; }

// q for one entry: max(0, p_t - p_d) for a residual, p_t for a bonus; bt and
// bd are exp_shift of the target and draft log-sum-exps.
__device__ __forceinline__ float corr_weight(float zt, float zd, float bt, float bd,
                                             bool residual) {
  const float pt = shifted_exp(zt, bt);
  if (!residual) return pt;
  const float pd = shifted_exp(zd, bd);
  return fmaxf(pt - pd, 0.0f);
}

// Sums over the 16 entries a lane holds of q (max(0, p_t - p_d) for a
// residual, p_t for a bonus) and of p_t, added in entry order (invalid
// entries: 0); each entry takes exactly corr_weight's operations.
// FAST (the one-block engine shape, which has registers to spare): an
// unmasked path when every lane of the wave holds 16 valid entries, and the
// masked one (a select after the exponentials) only on a ragged tile.
// Otherwise (the two-block shape, where every tile takes the masked path):
// masked entries get the exponent -inf, so both exponentials give 0 with no
// branch around them (after a select of the result the compiler branched per
// entry), and each entry is added as soon as it is formed, which keeps few
// values live.
template <bool BF16, bool FAST>
__device__ __forceinline__ void corr_tile_sums(const f32x4 acc[4], const float zt16[16],
                                               const float u16[16], int nvalid, float bt,
                                               float bd, bool residual, float& sq, float& sp) {
  sq = 0.0f;
  sp = 0.0f;
  if constexpr (FAST) {
    float q[16], pt[16];
    if (__all(nvalid >= 16)) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int idx = 4 * j + i;
          q[idx] = corr_weight(zt16[idx], acc[j][i] + u16[idx], bt, bd, residual);
          pt[idx] = shifted_exp(zt16[idx], bt);
        }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int idx = 4 * j + i;
          const bool ok = idx < nvalid;
          q[idx] = ok ? corr_weight(zt16[idx], acc[j][i] + u16[idx], bt, bd, residual) : 0.0f;
          pt[idx] = ok ? shifted_exp(zt16[idx], bt) : 0.0f;
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sq += q[i];
      sp += pt[i];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = 4 * j + i;
        const bool ok = idx < nvalid;
        const float et = ok ? fmaf(zt16[idx], kLog2e, bt) : -INFINITY;
        const float ed = ok ? fmaf(acc[j][i] + u16[idx], kLog2e, bd) : -INFINITY;
        const float ptv = __builtin_amdgcn_exp2f(et);
        sq += residual ? fmaxf(ptv - __builtin_amdgcn_exp2f(ed), 0.0f) : ptv;
        sp += ptv;
      }
  }
}

// ---------------------------------------------------------------------------
// residual partials
// ---------------------------------------------------------------------------

// Epilogue of the residual pass: per entry q = max(0, p_t - p_d) (or p_t for
// a bonus job) and p_t, summed per tile and request and stored at
// rpart[n * ldn + part_pos(t, c)]. The job fields are read
// once per kernel (prepare); a bonus job reads its target row in place of the
// U row, so the loads need no branch.
template <bool BF16, bool VEC, bool FAST>
struct ResidualEpi {
  typedef typename Elem<BF16>::T T;
  struct Pre {
    Raw16<BF16> zt, u;
  };
  struct St {
    const T* trow;
    const T* urow;
    float bt, bd;  // exp_shift of the job's target and draft log-sum-exps
    int ng;
    bool residual, active;
  };
  const T* target;
  const T* U;
  int gamma, V, R, g0;
  Jobs jobs;
  float2* rpart;
  int ldn, c;

  __device__ __forceinline__ St prepare(int n) const {
    St s;
    s.active = n < R;
    s.ng = g0 + min(n, R - 1);
    s.residual = jobs.kind[s.ng] == 0;
    s.trow = target + (size_t)jobs.trow[s.ng] * V;
    s.urow = s.residual ? U + ((size_t)s.ng * gamma + jobs.slot[s.ng] - 1) * V : s.trow;
    s.bt = exp_shift(jobs.lse_t[s.ng]);
    s.bd = exp_shift(jobs.lse_d[s.ng]);
    return s;
  }
  __device__ __forceinline__ void side_work() const {}
  __device__ __forceinline__ void load(const St& s, int v0, int nvalid, Pre& p) const {
    load16_clamped<BF16, VEC>(s.trow, v0, nvalid, V, p.zt);
    load16_clamped<BF16, VEC>(s.urow, v0, nvalid, V, p.u);
  }
  __device__ __forceinline__ void finish(const St& s, int v0, int nvalid, const f32x4 acc[4],
                                         const Pre& p, int t, int lane) const {
    float zt16[16], u16[16];
    unpack16<BF16>(p.zt, zt16);
    unpack16<BF16>(p.u, u16);
    float sq, sp;
    corr_tile_sums<BF16, FAST>(acc, zt16, u16, (s.active ? nvalid : 0), s.bt, s.bd, s.residual,
                               sq, sp);
    sq = pair_sum<false>(pair_sum<true>(sq));
    sp = pair_sum<false>(pair_sum<true>(sp));
    if ((lane >> 4) == 0 && s.active) rpart[(size_t)s.ng * ldn + part_pos(t, c)] = make_float2(sq, sp);
  }
};

template <bool BF16, int KC, int NW, int NB, bool VEC>
__global__ __launch_bounds__(NW * 64) void residual_partials_kernel(
    const typename Elem<BF16>::T* __restrict__ target, const typename Elem<BF16>::T* __restrict__ U,
    const typename Elem<BF16>::T* __restrict__ W1, const typename Elem<BF16>::T* __restrict__ W2p,
    Jobs jobs, int g0, int R, int gamma, int V, int r, int n_t, float2* __restrict__ rpart, int ldn,
    int c, unsigned* __restrict__ queue) {
  const ResidualEpi<BF16, VEC, NB == 1> epi{target, U, gamma, V, R, g0, jobs, rpart, ldn, c};
  run_tile_engine<BF16, KC, NW, NB, VEC>(W1, W2p, [&](int n) { return jobs.xprev[g0 + n]; }, R, V,
                                         r, n_t, epi, queue, V, (int)gridDim.x, (int)blockIdx.x);
}

// ---------------------------------------------------------------------------
// residual select
// ---------------------------------------------------------------------------

// One 256-thread workgroup per request, partials chunked as in the draft
// select; wave 0 recomputes the crossing tile and writes the token.
template <bool BF16, int KC, int CMAX, bool VW>
__global__ __launch_bounds__(kSelThreads) void residual_select_kernel(
    const typename Elem<BF16>::T* __restrict__ target, const typename Elem<BF16>::T* __restrict__ U,
    const typename Elem<BF16>::T* __restrict__ W1, const typename Elem<BF16>::T* __restrict__ W2p,
    Jobs jobs, int gamma, int V, int r, int n_t, const float2* __restrict__ rpart, int ldn, int c,
    int* __restrict__ out_tokens, unsigned* __restrict__ queue, int n_queue) {
  typedef typename Elem<BF16>::Frag Frag;
  __shared__ BlockSearchShared sh;
  const int n = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1);
  // the residual GEMM has finished: put its tile-queue counters back to zero
  if (n == 0 && tid < n_queue) queue[tid * kQueueStride] = 0u;
  const float2* prow = rpart + (size_t)n * ldn;
  const int t0 = tid * c;
  const int cnt = max(0, min(c, n_t - t0));
  float2 pv[CMAX > 0 ? CMAX : 1];
  if constexpr (CMAX > 0) {
#pragma unroll
    for (int i = 0; i < CMAX; ++i) pv[i] = prow[min(i, c - 1) * kSelThreads + tid];
  }
  const int x = clamp_token(jobs.xprev[n], V);
  Frag b[KC];
  load_b_row<BF16, KC, VW>(W1 + (size_t)x * r, r, lane, b);
  const float u = jobs.u[n];

  // residual mass left? (else draw from p_t)
  bool use_pt;
  WaveSearch ws;
  if constexpr (CMAX > 0) {
    float lq = 0.0f;
#pragma unroll
    for (int i = 0; i < CMAX; ++i) lq += i < cnt ? pv[i].x : 0.0f;
    use_pt = !(block_sum(lq, sh) > 0.0f);
    float w[CMAX];
#pragma unroll
    for (int i = 0; i < CMAX; ++i) w[i] = i < cnt ? (use_pt ? pv[i].y : pv[i].x) : 0.0f;
    ws = block_tile_search<CMAX>([&](int i) { return w[i]; }, t0, cnt, u, sh);
  } else {
    float lq = 0.0f;
    for (int i = 0; i < cnt; ++i) lq += prow[i * kSelThreads + tid].x;
    use_pt = !(block_sum(lq, sh) > 0.0f);
    ws = block_tile_search<0>([&](int i) {
      const float2 q = prow[i * kSelThreads + tid];
      return use_pt ? q.y : q.x;
    }, t0, cnt, u, sh);
  }
  if (tid >= kWave) return;  // wave 0 finishes; no barrier below

  // recompute the crossing tile; lane l takes entry v = 64 t + l
  const int t = min(max(ws.tstar, 0), n_t - 1);
  const bool residual = jobs.kind[n] == 0;
  const int trow = jobs.trow[n], dslot = jobs.slot[n] - 1;
  const float lse_t = jobs.lse_t[n], lse_d = jobs.lse_d[n];
  ATile<BF16, KC> at;
  load_a_tile<BF16, KC>(W2p, t, lane, at);
  const int v = t * kTileV + lane;
  const bool valid = v < V;
  const int vc = min(v, V - 1);
  const float zt = to_f32(target[(size_t)trow * V + vc]);
  const float ud = residual ? to_f32(U[((size_t)n * gamma + dslot) * V + vc]) : 0.0f;
  __builtin_amdgcn_sched_barrier(0);  // all of the tile's loads before the first product
  f32x4 acc[4];
  tile_mma_regs<BF16, KC>(at, b, acc);
  const float zd = own_entry(acc, lane) + ud;  // the same sum the residual pass formed
  const float q = corr_weight(zt, zd, exp_shift(lse_t), exp_shift(lse_d), residual);
  const float pt = shifted_exp(zt, exp_shift(lse_t));
  const float wi = valid ? (use_pt ? pt : q) : 0.0f;
  const int sel = tile_pick(wi, valid, ws.pb, ws.T, lane);
  if (lane == 0) out_tokens[(size_t)n * (gamma + 1) + jobs.slot[n] - 1] = t * kTileV + sel;
}

// ---------------------------------------------------------------------------
// analytic acceptance c* = 1 - 1/2 |p_d - p_t|_1 per verified slot
// ---------------------------------------------------------------------------

// DSpark digest, "Verification scheduling (system side)": the confidence
// head's training target is the analytic acceptance rate of a slot, one minus
// the total-variation distance between its draft and target distributions.
// With both normalisers known (the draft's stored lse, the target row's lse
// from the row partials), c* = sum_v min(p_d(v), p_t(v)) is one pass over the
// vocabulary: the draft GEMM engine recomputes every verified slot's draft
// logits, and the epilogue sums min(p_d, p_t) per 64-entry tile.
//
// One job per packed row n (the row that holds the target of slot j + 1 of
// its request, j = n - cu[r]); rows past a request's verified slots (its bonus
// row) and past the pack are inactive and point their loads at row 0.
struct AcceptJobs {
  int* out;      // r * gamma + j for an active job, -1 otherwise
  int* urow;     // draft base-logit row r * gamma + j (0 when inactive)
  int* trow;     // packed target row (0 when inactive)
  int* xprev;    // token before the slot (anchor for slot 1)
  float* lse_t;  // target log-sum-exp of trow
  float* lse_d;  // draft log-sum-exp of the slot
};

__global__ __launch_bounds__(256) void accept_jobs_kernel(
    const int* __restrict__ cu_seqlens, const int* __restrict__ anchor,
    const int* __restrict__ tokens, const float* __restrict__ lse_draft,
    const float2* __restrict__ rowpart, int n_chunks, int R, int gamma, int rows_ws,
    AcceptJobs jobs, float* __restrict__ cstar) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < R * gamma) {  // slots no packed row verifies: NaN
    const int r = i / gamma, k = i % gamma + 1;
    const int Lv = min(cu_seqlens[r + 1] - cu_seqlens[r] - 1, gamma);
    if (k > Lv) cstar[i] = __builtin_nanf("");
  }
  if (i >= rows_ws) return;
  const int M = min(cu_seqlens[R], rows_ws);
  // request of row i: the last r with cu[r] <= i
  int lo = 0, hi = R - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_seqlens[mid] <= i) lo = mid; else hi = mid - 1;
  }
  const int r = lo;
  const int j = i - cu_seqlens[r];
  const int Lv = min(cu_seqlens[r + 1] - cu_seqlens[r] - 1, gamma);
  const bool active = i < M && j >= 0 && j < Lv;
  int out = -1, xprev = 0, trow = 0;
  float lse_t = 0.0f, lse_d = 0.0f;
  if (active) {
    out = r * gamma + j;
    xprev = j == 0 ? anchor[r] : tokens[r * gamma + j - 1];
    trow = i;
    lse_d = lse_draft[out];
    float m = -INFINITY, S = 0.0f;
    for (int c = 0; c < n_chunks; ++c) m = fmaxf(m, rowpart[(size_t)i * n_chunks + c].x);
    for (int c = 0; c < n_chunks; ++c) {
      const float2 pv = rowpart[(size_t)i * n_chunks + c];
      S += pv.y * __expf(pv.x - m);
    }
    lse_t = m + __logf(S);
  }
  jobs.out[i] = out;
  jobs.urow[i] = active ? out : 0;
  jobs.trow[i] = trow;
  jobs.xprev[i] = xprev;
  jobs.lse_t[i] = lse_t;
  jobs.lse_d[i] = lse_d;
}

// Epilogue: per entry min(exp(z_d - lse_d), exp(z_t - lse_t)) with
// z_d = W1[x_prev] W2 + U (the draft pass's own sum), summed per tile and
// job and stored at cpart[n * ldn + part_pos(t, c)].
template <bool BF16, bool VEC>
struct AcceptEpi {
  typedef typename Elem<BF16>::T T;
  struct Pre {
    Raw16<BF16> zt, u;
  };
  struct St {
    const T* trow;
    const T* urow;
    float bt, bd;  // exp_shift of the slot's target and draft log-sum-exps
    int ng;
    bool active;
  };
  const T* target;
  const T* U;
  int V, R, g0;
  AcceptJobs jobs;
  float* cpart;
  int ldn, c;

  __device__ __forceinline__ St prepare(int n) const {
    St s;
    s.ng = g0 + min(n, R - 1);
    s.active = n < R && jobs.out[s.ng] >= 0;
    s.trow = target + (size_t)jobs.trow[s.ng] * V;
    s.urow = U + (size_t)jobs.urow[s.ng] * V;
    s.bt = exp_shift(jobs.lse_t[s.ng]);
    s.bd = exp_shift(jobs.lse_d[s.ng]);
    return s;
  }
  __device__ __forceinline__ void side_work() const {}
  __device__ __forceinline__ void load(const St& s, int v0, int nvalid, Pre& p) const {
    load16_clamped<BF16, VEC>(s.trow, v0, nvalid, V, p.zt);
    load16_clamped<BF16, VEC>(s.urow, v0, nvalid, V, p.u);
  }
  __device__ __forceinline__ void finish(const St& s, int v0, int nvalid, const f32x4 acc[4],
                                         const Pre& p, int t, int lane) const {
    float zt16[16], u16[16];
    unpack16<BF16>(p.zt, zt16);
    unpack16<BF16>(p.u, u16);
    const int nv = s.active ? nvalid : 0;
    float sm = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = 4 * j + i;
        const float zd = acc[j][i] + u16[idx];
        const float pd = shifted_exp(zd, s.bd), pt = shifted_exp(zt16[idx], s.bt);
        sm += idx < nv ? fminf(pd, pt) : 0.0f;
      }
    sm = pair_sum<false>(pair_sum<true>(sm));
    if ((lane >> 4) == 0 && s.active) cpart[(size_t)s.ng * ldn + part_pos(t, c)] = sm;
  }
};

template <bool BF16, int KC, int NW, int NB, bool VEC>
__global__ __launch_bounds__(NW * 64) void accept_partials_kernel(
    const typename Elem<BF16>::T* __restrict__ target, const typename Elem<BF16>::T* __restrict__ U,
    const typename Elem<BF16>::T* __restrict__ W1, const typename Elem<BF16>::T* __restrict__ W2p,
    AcceptJobs jobs, int g0, int R, int V, int r, int n_t, float* __restrict__ cpart, int ldn,
    int c, unsigned* __restrict__ queue) {
  const AcceptEpi<BF16, VEC> epi{target, U, V, R, g0, jobs, cpart, ldn, c};
  run_tile_engine<BF16, KC, NW, NB, VEC>(W1, W2p, [&](int n) { return jobs.xprev[g0 + n]; }, R, V,
                                         r, n_t, epi, queue, V, (int)gridDim.x, (int)blockIdx.x);
}

// One 256-thread workgroup per job: the tile sums in a fixed order. The
// workgroup of job 0 first puts the GEMM pass's queue counters back to zero.
__global__ __launch_bounds__(kSelThreads) void accept_reduce_kernel(
    AcceptJobs jobs, const float* __restrict__ cpart, int ldn, int c, int n_t,
    float* __restrict__ cstar, unsigned* __restrict__ queue, int n_queue) {
  __shared__ BlockSearchShared sh;
  const int n = blockIdx.x, tid = threadIdx.x;
  if (n == 0 && tid < n_queue) queue[tid * kQueueStride] = 0u;
  const int out = jobs.out[n];
  if (out < 0) return;  // workgroup-uniform
  const float* prow = cpart + (size_t)n * ldn;
  const int t0 = tid * c;
  const int cnt = max(0, min(c, n_t - t0));
  float s = 0.0f;
  for (int i = 0; i < cnt; ++i) s += prow[i * kSelThreads + tid];
  s = block_sum(s, sh);
  if (tid == 0) cstar[out] = s;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct VerifyWs {
  float2* rowpart;
  float2* rpart;  // request-major residual tile partials [R, part_ld(V)]
  unsigned* queue;  // tile-queue counters of the residual GEMM, per request group
  Jobs jobs;
};

// Row partials cover R * (gamma + 1) packed rows: no well-formed pack has more.
static size_t carve(VerifyWs* w, void* base, int R, int gamma, int V) {
  const int rows_ws = R * (gamma + 1);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const size_t o_row = take((size_t)rows_ws * n_row_chunks(V) * sizeof(float2));
  const size_t o_rp = take((size_t)R * part_ld(V) * sizeof(float2));
  const size_t o_q = take((size_t)queue_groups(R) * kQueueWordsPerGroup * 4);
  size_t o_j[7];
  for (int i = 0; i < 7; ++i) o_j[i] = take((size_t)R * 4);
  if (w && base) {
    char* b = static_cast<char*>(base);
    w->rowpart = reinterpret_cast<float2*>(b + o_row);
    w->rpart = reinterpret_cast<float2*>(b + o_rp);
    w->queue = reinterpret_cast<unsigned*>(b + o_q);
    w->jobs.kind = reinterpret_cast<int*>(b + o_j[0]);
    w->jobs.slot = reinterpret_cast<int*>(b + o_j[1]);
    w->jobs.trow = reinterpret_cast<int*>(b + o_j[2]);
    w->jobs.xprev = reinterpret_cast<int*>(b + o_j[3]);
    w->jobs.u = reinterpret_cast<float*>(b + o_j[4]);
    w->jobs.lse_t = reinterpret_cast<float*>(b + o_j[5]);
    w->jobs.lse_d = reinterpret_cast<float*>(b + o_j[6]);
  }
  return off;
}

size_t verify_ws_bytes(int R, int gamma, int V) { return carve(nullptr, nullptr, R, gamma, V); }

template <bool BF16, int KC>
static int launch_verify(const void* target, int M_cap, const int32_t* cu, const int32_t* anchor,
                         const int32_t* tokens, const float* p_draft, const float* lse_draft,
                         const void* U, const void* W1, const void* W2p, const int32_t* win_len,
                         int mode, uint64_t seed, StepArg step, const uint32_t* req_ids, int R,
                         int gamma, int V, int r, int32_t* accept_len, int32_t* out_tokens,
                         int32_t* n_out, int32_t* ceiling, const VerifyWs& ws, hipStream_t s) {
  typedef typename Elem<BF16>::T T;
  const T* tg = static_cast<const T*>(target);
  const T* Ub = static_cast<const T*>(U);
  const T* W1b = static_cast<const T*>(W1);
  const T* W2b = static_cast<const T*>(W2p);
  const int nch = n_row_chunks(V), n_t = n_vtiles(V);
  const bool vec = rows_vec_ok(target, V, V, Elem<BF16>::kVec) &&
                   rows_vec_ok(U, V, V, Elem<BF16>::kVec);
  const bool vec_w1 = w1_vec_ok(W1, r);
  const bool vec_engine = vec && vec_w1;
  const int ldn = part_ld(V), c = part_chunk(V);
  const int rows_ws = R * (gamma + 1);
  (void)M_cap;
  if (rows_vec_ok(target, V, V, Elem<BF16>::kVec))
    hipLaunchKernelGGL((row_partials_kernel<BF16, true>), dim3(nch, rows_ws), dim3(kRowThreads), 0, s,
                       tg, V, nch, cu, R, rows_ws, ws.rowpart);
  else
    hipLaunchKernelGGL((row_partials_kernel<BF16, false>), dim3(nch, rows_ws), dim3(kRowThreads), 0, s,
                       tg, V, nch, cu, R, rows_ws, ws.rowpart);
  int st = launch_status();
  if (st) return st;
  if (nch <= 16)
    hipLaunchKernelGGL((decide_kernel<BF16, 16>), dim3(ceil_div(R, 4)), dim3(256), 0, s, tg, V, nch,
                       ws.rowpart, cu, anchor, tokens, p_draft, lse_draft, win_len, mode, seed, step,
                       req_ids, R, gamma, rows_ws, ws.jobs, accept_len, out_tokens, n_out, ceiling);
  else if (nch <= 32)
    hipLaunchKernelGGL((decide_kernel<BF16, 32>), dim3(ceil_div(R, 4)), dim3(256), 0, s, tg, V, nch,
                       ws.rowpart, cu, anchor, tokens, p_draft, lse_draft, win_len, mode, seed, step,
                       req_ids, R, gamma, rows_ws, ws.jobs, accept_len, out_tokens, n_out, ceiling);
  else
    hipLaunchKernelGGL((decide_kernel<BF16, 0>), dim3(ceil_div(R, 4)), dim3(256), 0, s, tg, V, nch,
                       ws.rowpart, cu, anchor, tokens, p_draft, lse_draft, win_len, mode, seed, step,
                       req_ids, R, gamma, rows_ws, ws.jobs, accept_len, out_tokens, n_out, ceiling);
  st = launch_status();
  if (st) return st;
  const int ncu = device_cu_count();
  for (int g0 = 0; g0 < R; g0 += req_group<BF16>()) {
    const int Rg = std::min(req_group<BF16>(), R - g0);
    const int blocks = ceil_div(Rg, kTileN);
    unsigned* qg = ws.queue + (size_t)(g0 / req_group<BF16>()) * kQueueWordsPerGroup;
#define DSPARK_RES_LAUNCH(NW_, NB_, PERCU)                                                         \
    {                                                                                              \
      typedef EngineGeom<BF16, KC, NW_> G;                                                         \
      const dim3 grid(engine_grid(n_t, PERCU * ncu));                                                     \
      if (vec_engine)                                                                              \
        hipLaunchKernelGGL((residual_partials_kernel<BF16, KC, NW_, NB_, true>), grid,             \
                           dim3(NW_ * kWave), G::kLdsBytes, s, tg, Ub, W1b, W2b, ws.jobs, g0, Rg,  \
                           gamma, V, r, n_t, ws.rpart, ldn, c, qg);                               \
      else                                                                                         \
        hipLaunchKernelGGL((residual_partials_kernel<BF16, KC, NW_, NB_, false>), grid,            \
                           dim3(NW_ * kWave), G::kLdsBytes, s, tg, Ub, W1b, W2b, ws.jobs, g0, Rg,  \
                           gamma, V, r, n_t, ws.rpart, ldn, c, qg);                               \
    }
    if (blocks <= 4) DSPARK_RES_LAUNCH(4, 1, 2)
    else if (blocks <= 8) DSPARK_RES_LAUNCH(8, 1, 1)
    else if constexpr (BF16) DSPARK_RES_LAUNCH(8, 2, 1)
    else return DSPARK_ESIZE;  // unreachable: float32 groups hold at most 8 blocks
#undef DSPARK_RES_LAUNCH
    st = launch_status();
    if (st) return st;
  }
#define DSPARK_RES_SELECT(CM)                                                                     \
  if (vec_w1)                                                                                    \
    hipLaunchKernelGGL((residual_select_kernel<BF16, KC, CM, true>), dim3(R), dim3(kSelThreads), 0, s, \
                       tg, Ub, W1b, W2b, ws.jobs, gamma, V, r, n_t, ws.rpart, ldn, c,             \
                       out_tokens, ws.queue, queue_groups(R) * kNumXcd);                         \
  else                                                                                           \
    hipLaunchKernelGGL((residual_select_kernel<BF16, KC, CM, false>), dim3(R), dim3(kSelThreads), 0, s, \
                       tg, Ub, W1b, W2b, ws.jobs, gamma, V, r, n_t, ws.rpart, ldn, c,             \
                       out_tokens, ws.queue, queue_groups(R) * kNumXcd)
  // the partial row in registers, unrolled to the smallest of 8 / 10 / 12 /
  // 16 chunks that holds it (masked iterations cost as much as live ones;
  // 8 and 10 chunks are vocabularies up to 131072 and 163840)
  if (c <= 8) {
    DSPARK_RES_SELECT(8);
  } else if (c <= 10) {
    DSPARK_RES_SELECT(10);
  } else if (c <= 12) {
    DSPARK_RES_SELECT(12);
  } else if (c <= 16) {
    DSPARK_RES_SELECT(16);
  } else {
    DSPARK_RES_SELECT(0);
  }
#undef DSPARK_RES_SELECT
  return launch_status();
}

// Analytic-acceptance workspace: row partials and jobs for R * (gamma + 1)
// packed rows, their tile sums and the tile-queue counters.
struct AcceptWs {
  float2* rowpart;
  float* cpart;
  unsigned* queue;
  AcceptJobs jobs;
};

static size_t carve_accept(AcceptWs* w, void* base, int R, int gamma, int V) {
  const int rows_ws = R * (gamma + 1);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const size_t o_row = take((size_t)rows_ws * n_row_chunks(V) * sizeof(float2));
  const size_t o_cp = take((size_t)rows_ws * part_ld(V) * sizeof(float));
  const size_t o_q = take((size_t)queue_groups(rows_ws) * kQueueWordsPerGroup * 4);
  size_t o_j[6];
  for (int i = 0; i < 6; ++i) o_j[i] = take((size_t)rows_ws * 4);
  if (w && base) {
    char* b = static_cast<char*>(base);
    w->rowpart = reinterpret_cast<float2*>(b + o_row);
    w->cpart = reinterpret_cast<float*>(b + o_cp);
    w->queue = reinterpret_cast<unsigned*>(b + o_q);
    w->jobs.out = reinterpret_cast<int*>(b + o_j[0]);
    w->jobs.urow = reinterpret_cast<int*>(b + o_j[1]);
    w->jobs.trow = reinterpret_cast<int*>(b + o_j[2]);
    w->jobs.xprev = reinterpret_cast<int*>(b + o_j[3]);
    w->jobs.lse_t = reinterpret_cast<float*>(b + o_j[4]);
    w->jobs.lse_d = reinterpret_cast<float*>(b + o_j[5]);
  }
  return off;
}

size_t accept_ws_bytes(int R, int gamma, int V) { return carve_accept(nullptr, nullptr, R, gamma, V); }

template <bool BF16, int KC>
static int launch_accept(const void* target, const int32_t* cu, const int32_t* anchor,
                         const int32_t* tokens, const float* lse_draft, const void* U,
                         const void* W1, const void* W2p, int R, int gamma, int V, int r,
                         float* cstar, const AcceptWs& ws, hipStream_t s) {
  typedef typename Elem<BF16>::T T;
  const T* tg = static_cast<const T*>(target);
  const T* Ub = static_cast<const T*>(U);
  const T* W1b = static_cast<const T*>(W1);
  const T* W2b = static_cast<const T*>(W2p);
  const int nch = n_row_chunks(V), n_t = n_vtiles(V);
  const bool vec = rows_vec_ok(target, V, V, Elem<BF16>::kVec) &&
                   rows_vec_ok(U, V, V, Elem<BF16>::kVec) && w1_vec_ok(W1, r);
  const int ldn = part_ld(V), c = part_chunk(V);
  const int rows_ws = R * (gamma + 1);
  if (rows_vec_ok(target, V, V, Elem<BF16>::kVec))
    hipLaunchKernelGGL((row_partials_kernel<BF16, true>), dim3(nch, rows_ws), dim3(kRowThreads), 0, s,
                       tg, V, nch, cu, R, rows_ws, ws.rowpart);
  else
    hipLaunchKernelGGL((row_partials_kernel<BF16, false>), dim3(nch, rows_ws), dim3(kRowThreads), 0, s,
                       tg, V, nch, cu, R, rows_ws, ws.rowpart);
  int st = launch_status();
  if (st) return st;
  hipLaunchKernelGGL(accept_jobs_kernel, dim3(ceil_div(rows_ws, 256)), dim3(256), 0, s, cu, anchor,
                     tokens, lse_draft, ws.rowpart, nch, R, gamma, rows_ws, ws.jobs, cstar);
  st = launch_status();
  if (st) return st;
  const int ncu = device_cu_count();
  for (int g0 = 0; g0 < rows_ws; g0 += req_group<BF16>()) {
    const int Rg = std::min(req_group<BF16>(), rows_ws - g0);
    const int blocks = ceil_div(Rg, kTileN);
    unsigned* qg = ws.queue + (size_t)(g0 / req_group<BF16>()) * kQueueWordsPerGroup;
#define DSPARK_ACC_LAUNCH(NW_, NB_, PERCU)                                                         \
    {                                                                                              \
      typedef EngineGeom<BF16, KC, NW_> G;                                                         \
      const dim3 grid(engine_grid(n_t, PERCU * ncu));                                                     \
      if (vec)                                                                                     \
        hipLaunchKernelGGL((accept_partials_kernel<BF16, KC, NW_, NB_, true>), grid,               \
                           dim3(NW_ * kWave), G::kLdsBytes, s, tg, Ub, W1b, W2b, ws.jobs, g0, Rg,  \
                           V, r, n_t, ws.cpart, ldn, c, qg);                                      \
      else                                                                                         \
        hipLaunchKernelGGL((accept_partials_kernel<BF16, KC, NW_, NB_, false>), grid,              \
                           dim3(NW_ * kWave), G::kLdsBytes, s, tg, Ub, W1b, W2b, ws.jobs, g0, Rg,  \
                           V, r, n_t, ws.cpart, ldn, c, qg);                                      \
    }
    if (blocks <= 4) DSPARK_ACC_LAUNCH(4, 1, 2)
    else if (blocks <= 8) DSPARK_ACC_LAUNCH(8, 1, 1)
    else if constexpr (BF16) DSPARK_ACC_LAUNCH(8, 2, 1)
    else return DSPARK_ESIZE;  // unreachable: float32 groups hold at most 8 blocks
#undef DSPARK_ACC_LAUNCH
    st = launch_status();
    if (st) return st;
  }
  hipLaunchKernelGGL(accept_reduce_kernel, dim3(rows_ws), dim3(kSelThreads), 0, s, ws.jobs, ws.cpart,
                     ldn, c, n_t, cstar, ws.queue, queue_groups(rows_ws) * kNumXcd);
  return launch_status();
}

}  // namespace dspark

using namespace dspark;

extern "C" int dspark_verify(const void* target_packed, int M_cap, const int32_t* cu_seqlens,
                             const int32_t* anchor, const int32_t* tokens, const float* p_draft,
                             const float* lse_draft, const void* U, const void* W1,
                             const void* W2p, const int32_t* win_len, int mode, uint64_t seed,
                             uint64_t step, const uint64_t* step_dev, const uint32_t* req_ids,
                             int R, int gamma, int V, int r, int dtype, int32_t* accept_len,
                             int32_t* out_tokens, int32_t* n_out, int32_t* ceiling_len, void* ws,
                             size_t ws_bytes, void* stream) {
  int st = check_sizes(R, gamma, V, r, dtype);
  if (st) return st;
  if (mode < DSPARK_VERIFY_STATIC || mode > DSPARK_VERIFY_CAP_ACCEPT) return DSPARK_EINVAL;
  if (!target_packed || !cu_seqlens || !anchor || !tokens || !p_draft || !lse_draft || !U || !W1 ||
      !W2p || !req_ids || !accept_len || !out_tokens || !n_out)
    return DSPARK_EINVAL;
  if (mode == DSPARK_VERIFY_CAP_ACCEPT && !win_len) return DSPARK_EINVAL;
  if (M_cap < R * (gamma + 1)) return DSPARK_ESIZE;
  if (!ws || ws_bytes < verify_ws_bytes(R, gamma, V)) return DSPARK_EWORKSPACE;
  VerifyWs w;
  carve(&w, ws, R, gamma, V);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const StepArg sa{step, step_dev};
#define DSPARK_VERIFY_ARGS                                                                        \
  target_packed, M_cap, cu_seqlens, anchor, tokens, p_draft, lse_draft, U, W1, W2p, win_len, mode, \
      seed, sa, req_ids, R, gamma, V, r, accept_len, out_tokens, n_out, ceiling_len, w, s
  if (dtype == DSPARK_BF16) {
    switch (kc_instance(r)) {
      case 1: return launch_verify<true, 1>(DSPARK_VERIFY_ARGS);
      case 2: return launch_verify<true, 2>(DSPARK_VERIFY_ARGS);
      case 4: return launch_verify<true, 4>(DSPARK_VERIFY_ARGS);
      default: return launch_verify<true, 8>(DSPARK_VERIFY_ARGS);
    }
  }
  switch (kc_instance(r)) {
    case 1: return launch_verify<false, 1>(DSPARK_VERIFY_ARGS);
    case 2: return launch_verify<false, 2>(DSPARK_VERIFY_ARGS);
    default: return launch_verify<false, 4>(DSPARK_VERIFY_ARGS);
  }
#undef DSPARK_VERIFY_ARGS
}

extern "C" int dspark_analytic_accept(const void* target_packed, int M_cap,
                                      const int32_t* cu_seqlens, const int32_t* anchor,
                                      const int32_t* tokens, const float* lse_draft, const void* U,
                                      const void* W1, const void* W2p, int R, int gamma, int V,
                                      int r, int dtype, float* cstar, void* ws, size_t ws_bytes,
                                      void* stream) {
  int st = check_sizes(R, gamma, V, r, dtype);
  if (st) return st;
  if (!target_packed || !cu_seqlens || !anchor || !tokens || !lse_draft || !U || !W1 || !W2p ||
      !cstar)
    return DSPARK_EINVAL;
  if (M_cap < R * (gamma + 1)) return DSPARK_ESIZE;
  if (!ws || ws_bytes < accept_ws_bytes(R, gamma, V)) return DSPARK_EWORKSPACE;
  AcceptWs w;
  carve_accept(&w, ws, R, gamma, V);
  hipStream_t s = static_cast<hipStream_t>(stream);
#define DSPARK_ACCEPT_ARGS \
  target_packed, cu_seqlens, anchor, tokens, lse_draft, U, W1, W2p, R, gamma, V, r, cstar, w, s
  if (dtype == DSPARK_BF16) {
    switch (kc_instance(r)) {
      case 1: return launch_accept<true, 1>(DSPARK_ACCEPT_ARGS);
      case 2: return launch_accept<true, 2>(DSPARK_ACCEPT_ARGS);
      case 4: return launch_accept<true, 4>(DSPARK_ACCEPT_ARGS);
      default: return launch_accept<true, 8>(DSPARK_ACCEPT_ARGS);
    }
  }
  switch (kc_instance(r)) {
    case 1: return launch_accept<false, 1>(DSPARK_ACCEPT_ARGS);
    case 2: return launch_accept<false, 2>(DSPARK_ACCEPT_ARGS);
    default: return launch_accept<false, 4>(DSPARK_ACCEPT_ARGS);
  }
#undef DSPARK_ACCEPT_ARGS
}
