// Persistent, double-buffered engine for the Markov bias GEMM
// [R, r] x [r, V] on the gfx950 matrix cores, shared by the draft pass and the
// verify residual pass.
//
// Work split. The vocabulary tiles (64 entries each) are cut into eight
// contiguous ranges, one per XCD: workgroup b runs on XCD b % 8 (the
// dispatcher deals workgroups to the XCDs round-robin), so each XCD's L2 sees
// one contiguous stretch of the vocabulary and writes the partial rows of that
// stretch. Inside its XCD's range, workgroup j takes tiles j, gx + j and
// 2 gx + j (gx workgroups on the XCD), then claims further tiles one at a
// time from the XCD's queue counter (an atomic add issued a step before the
// tile's loads), so workgroups that run faster take more tiles and the
// workgroups of a launch finish together. The counters sit 256 bytes apart
// (atomics on one line serialise) and are put back to zero by the kernel that
// consumes the partials, before it reads them. The 16-request blocks of the request group
// are dealt to the waves round-robin, NB per wave; a wave keeps the gathered
// W1 rows of its blocks (the B operand) in registers for the whole kernel. The
// pre-packed W2 tile (the A operand) is staged in LDS, double buffered, and
// fetched two tiles ahead into two rotating register sets; the epilogue's
// per-request rows (U, target) are also fetched two tiles ahead. The
// steady-state loop is straight-line code: prefetch addresses are clamped to
// valid tiles instead of guarded, so no branch forces the compiler to drain
// the loads early. Every accumulator receives its rank chunks in increasing
// order, exactly as tile_mma() / tile_mma_regs() in dspark_device.hpp do, so
// a later recompute of one tile gives bit-identical logits.
//
// The epilogue policy supplies (all const, no branch around a load):
//   struct St;                     // per-lane request state, set up once
//   struct Pre;                    // prefetched per-lane rows of one tile
//   St prepare(int n)              // request n of the lane (may be >= R)
//   void load(const St&, int v0, int nvalid, Pre&)            // issue loads
//   void finish(const St&, int v0, int nvalid, const f32x4 acc[4],
//               const Pre&, int t, int lane)                  // consume, write
//   void side_work()                // once, in the prologue, loads in flight
#pragma once

#include "dspark_device.hpp"

namespace dspark {

constexpr int kNumXcd = 8;  // XCDs of an MI355X; only the tile order depends on it

template <bool BF16, int KC, int NW>
struct EngineGeom {
  typedef typename Elem<BF16>::Frag Frag;
  static constexpr int kTileFrags = KC * 4 * kWave;               // frags per W2 tile
  static constexpr int kThreads = NW * kWave;
  static constexpr int kPer = (kTileFrags + kThreads - 1) / kThreads;  // frags per thread
  static constexpr size_t kLdsBytes = 2 * (size_t)kTileFrags * sizeof(Frag);
  // fragment k of thread tid in a tile copy; when the tile has fewer
  // fragments than threads, surplus threads repeat one (same value, same
  // slot), which keeps the copy free of branches
  static __device__ __forceinline__ int slot(int k, int tid) {
    return (k * kThreads + tid) % kTileFrags;
  }
};

// Gather the B operand (W1 rows of the wave's blocks) into registers. With
// VEC (W1 16-byte aligned, r a multiple of 8) the loads are unconditional:
// addresses are clamped into the row and out-of-range values zeroed after the
// load, so the prologue has no branch that would drain the loads in flight.
template <bool BF16, int KC, int NB, bool VEC, typename TokFn>
__device__ __forceinline__ void gather_b(const typename Elem<BF16>::T* __restrict__ W1, TokFn tok,
                                         int R, int r, int w1_rows, int wave, int nw, int lane,
                                         typename Elem<BF16>::Frag b[NB][KC]) {
  typedef typename Elem<BF16>::T T;
  typedef typename Elem<BF16>::Frag Frag;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = (wave + nw * nb) * kTileN + (lane & 15);
    const bool ok = n < R;
    const int x = clamp_token(tok(min(n, R - 1)), w1_rows);
    const T* row = W1 + (size_t)x * r;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int k0 = kc * kChunkK + 8 * (lane >> 4);
      if constexpr (VEC) {
        const Frag f = *reinterpret_cast<const Frag*>(row + min(k0, r - 8));
        b[nb][kc] = (ok && k0 < r) ? f : Frag{};
      } else {
        T tmp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) tmp[e] = (ok && k0 + e < r) ? row[k0 + e] : (T)0;
        b[nb][kc] = *reinterpret_cast<const Frag*>(tmp);
      }
    }
  }
}

// Queue counters: one per XCD, kQueueStride words apart; a launch serving
// request group g uses the counters at queue + g * kNumXcd * kQueueStride.
constexpr int kQueueStride = 64;  // 256 bytes
constexpr int kQueueWordsPerGroup = kNumXcd * kQueueStride;
constexpr int kStaticTiles = 3;   // tiles per workgroup dealt before the queue

// Tile range [lo, hi) of this workgroup's XCD (split in proportion to the
// workgroups each XCD runs), the XCD's workgroup count gx and this
// workgroup's index j among them.
struct XcdShare {
  int lo, hi, gx, j;
};
__device__ __forceinline__ XcdShare xcd_share(int n_t) {
  const int G = gridDim.x, x = blockIdx.x % kNumXcd;
  const int first = x * (G / kNumXcd) + min(x, G % kNumXcd);
  XcdShare s;
  s.gx = G / kNumXcd + (x < G % kNumXcd ? 1 : 0);
  s.j = blockIdx.x / kNumXcd;
  s.lo = (int)((long long)n_t * first / G);
  s.hi = (int)((long long)n_t * (first + s.gx) / G);
  return s;
}

// One step of the pipelined tile loop, straight-line code (no branch around
// any load, so the compiler's in-order load counters let the prefetches stay
// in flight): issue W2 of tile t2 into `w_issue`; multiply tile t out of `cur`;
// hand the epilogue its rows for t (prefetched two steps ago into `u`); issue
// the rows of t2 into `u`; store `w_ready` (W2 issued one step ago) into
// `nxt`. The caller ends the step with a barrier. t2 is the tile two steps
// ahead, clamped into the range.
template <bool BF16, int KC, int NW, int NB, class Epi>
__device__ __forceinline__ void engine_step(
    int t, int t2, int V, const typename Elem<BF16>::Frag* __restrict__ src,
    const typename Elem<BF16>::Frag* cur, typename Elem<BF16>::Frag* nxt,
    typename Elem<BF16>::Frag (&w_ready)[EngineGeom<BF16, KC, NW>::kPer],
    typename Elem<BF16>::Frag (&w_issue)[EngineGeom<BF16, KC, NW>::kPer],
    typename Epi::Pre (&u)[NB], const typename Elem<BF16>::Frag (&b)[NB][KC],
    const typename Epi::St (&st)[NB], const Epi& epi) {
  typedef EngineGeom<BF16, KC, NW> Geo;
  typedef typename Elem<BF16>::Frag Frag;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int g = lane >> 4;
  {
    const Frag* s = src + (size_t)t2 * Geo::kTileFrags;
#pragma unroll
    for (int k = 0; k < Geo::kPer; ++k) w_issue[k] = s[Geo::slot(k, tid)];
  }
  f32x4 acc[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[nb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    Frag a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = cur[(kc * 4 + j) * kWave + lane];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) mma_step<BF16>(acc[nb][j], a[j], b[nb][kc]);
  }
  const int v0 = t * kTileV + 16 * g;
  const int v0n = t2 * kTileV + 16 * g;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    epi.finish(st[nb], v0, min(16, V - v0), acc[nb], u[nb], t, lane);
    epi.load(st[nb], v0n, min(16, V - v0n), u[nb]);
  }
#pragma unroll
  for (int k = 0; k < Geo::kPer; ++k) nxt[Geo::slot(k, tid)] = w_ready[k];
}

// queue: this launch's kQueueWordsPerGroup counters (zero on entry). w1_rows:
// rows of W1 (token ids are clamped into them); V: vocabulary columns of this
// launch (fewer than w1_rows for one shard of a vocabulary-sharded draft).
template <bool BF16, int KC, int NW, int NB, bool VEC, class Epi, typename TokFn>
__device__ __forceinline__ void run_tile_engine(const typename Elem<BF16>::T* __restrict__ W1,
                                                const typename Elem<BF16>::T* __restrict__ W2p,
                                                TokFn tok, int R, int V, int r, int n_t,
                                                const Epi& epi, unsigned* __restrict__ queue,
                                                int w1_rows) {
  typedef EngineGeom<BF16, KC, NW> Geo;
  typedef typename Elem<BF16>::Frag Frag;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_grab[2];
  Frag* buf0 = reinterpret_cast<Frag*>(smem);
  Frag* buf1 = buf0 + Geo::kTileFrags;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int g = lane >> 4, nl = lane & 15;
  const Frag* src = reinterpret_cast<const Frag*>(W2p);
  const XcdShare xs = xcd_share(n_t);  // hi > lo: the grid has at most n_t workgroups
  unsigned* counter = queue + (blockIdx.x % kNumXcd) * kQueueStride;
  const int qbase = xs.lo + kStaticTiles * xs.gx;  // first tile the queue hands out
  auto clampt = [&](int t) { return min(t, xs.hi - 1); };
  int tc = xs.lo + xs.j, tn = tc + xs.gx, tnn = tn + xs.gx;  // current, next, next-but-one
  if (tc >= xs.hi) return;  // workgroup-uniform; no barrier passed yet

  // prologue: tile tc into LDS, W2 of tn and the rows of tc and tn in flight;
  // the first tile's loads go out before the (token -> W1 row) gather
  Frag wA[Geo::kPer], wB[Geo::kPer];
  typename Epi::Pre uA[NB], uB[NB];
  Frag first[Geo::kPer];
  {
    const Frag* s = src + (size_t)tc * Geo::kTileFrags;
#pragma unroll
    for (int i = 0; i < Geo::kPer; ++i) first[i] = s[Geo::slot(i, tid)];
  }
  Frag b[NB][KC];
  gather_b<BF16, KC, NB, VEC>(W1, tok, R, r, w1_rows, wave, NW, lane, b);
  typename Epi::St st[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) st[nb] = epi.prepare((wave + NW * nb) * kTileN + nl);
#pragma unroll
  for (int i = 0; i < Geo::kPer; ++i) buf0[Geo::slot(i, tid)] = first[i];
  {
    const Frag* s = src + (size_t)clampt(tn) * Geo::kTileFrags;
#pragma unroll
    for (int i = 0; i < Geo::kPer; ++i) wA[i] = s[Geo::slot(i, tid)];
  }
  {
    const int v0 = tc * kTileV + 16 * g, v1 = clampt(tn) * kTileV + 16 * g;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      epi.load(st[nb], v0, min(16, V - v0), uA[nb]);
      epi.load(st[nb], v1, min(16, V - v1), uB[nb]);
    }
  }
  epi.side_work();
  __syncthreads();

  // steady state: each step claims the tile three steps ahead (the atomic
  // returns while the step multiplies) and publishes it before the barrier.
  // A workgroup's tiles increase, so the first one past the range ends it.
  for (;;) {
    unsigned grab = 0;
    if (tid == 0) grab = atomicAdd(counter, 1u);
    engine_step<BF16, KC, NW, NB>(tc, clampt(tnn), V, src, buf0, buf1, wA, wB, uA, b, st, epi);
    if (tid == 0) s_grab[0] = qbase + (int)grab;
    __syncthreads();
    tc = tn;
    tn = tnn;
    tnn = max(s_grab[0], tn + 1);
    if (tc >= xs.hi) break;
    if (tid == 0) grab = atomicAdd(counter, 1u);
    engine_step<BF16, KC, NW, NB>(tc, clampt(tnn), V, src, buf1, buf0, wB, wA, uB, b, st, epi);
    if (tid == 0) s_grab[1] = qbase + (int)grab;
    __syncthreads();
    tc = tn;
    tn = tnn;
    tnn = max(s_grab[1], tn + 1);
    if (tc >= xs.hi) break;
  }
}

}  // namespace dspark
