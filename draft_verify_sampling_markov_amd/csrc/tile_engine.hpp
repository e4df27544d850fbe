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
// pre-packed W2 tile (the A operand) is staged in LDS, double buffered; each
// step issues the next tile's W2 and epilogue rows (U, target) before it
// multiplies, and prefetch addresses are clamped to valid tiles instead of
// guarded. Every accumulator receives its rank chunks in increasing
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
//   void side_work()                // once, in the prologue
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
// xtok[nb]: the token of the lane's request in block nb (read beforehand, so
// that the row loads wait on the token loads alone).
template <bool BF16, int KC, int NB, bool VEC>
__device__ __forceinline__ void gather_b(const typename Elem<BF16>::T* __restrict__ W1,
                                         const int (&xtok)[NB], int R, int r, int w1_rows,
                                         int wave, int nw, int lane,
                                         typename Elem<BF16>::Frag b[NB][KC]) {
  typedef typename Elem<BF16>::T T;
  typedef typename Elem<BF16>::Frag Frag;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = (wave + nw * nb) * kTileN + (lane & 15);
    const bool ok = n < R;
    const int x = clamp_token(xtok[nb], w1_rows);
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
__device__ __forceinline__ XcdShare xcd_share(int n_t, int G, int b) {
  const int x = b % kNumXcd;
  const int first = x * (G / kNumXcd) + min(x, G % kNumXcd);
  XcdShare s;
  s.gx = G / kNumXcd + (x < G % kNumXcd ? 1 : 0);
  s.j = b / kNumXcd;
  s.lo = (int)((long long)n_t * first / G);
  s.hi = (int)((long long)n_t * (first + s.gx) / G);
  return s;
}

// s_waitcnt with only the vector-memory count set: wait until at most n of
// this wave's vector memory operations are outstanding (they retire in issue
// order). The other counters are left at their maximum.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// queue: this engine's kQueueWordsPerGroup counters (zero on entry). w1_rows:
// rows of W1 (token ids are clamped into them); V: vocabulary columns of this
// launch (fewer than w1_rows for one shard of a vocabulary-sharded draft).
// G workgroups run this engine, gb is this one's index among them; workgroup
// gb runs on XCD gb % 8 (the launch keeps gb and blockIdx.x equal modulo 8).
//
// The loop is one step per tile, all of whose global loads go out at the
// step's start: the W2 tile and the epilogue rows of the NEXT tile, and the
// queue claim of the tile three steps ahead. The step then multiplies the current tile
// out of LDS and runs its epilogue (one global store per block), waits until
// only those stores are outstanding, moves the next tile's W2 into the other
// LDS buffer and its rows into the epilogue's registers, and ends with a
// barrier. Nothing a step loads is still in flight when the next one starts,
// so the loads of a step overlap its own multiply and epilogue.
template <bool BF16, int KC, int NW, int NB, bool VEC, class Epi, typename TokFn>
__device__ __forceinline__ void run_tile_engine(const typename Elem<BF16>::T* __restrict__ W1,
                                                const typename Elem<BF16>::T* __restrict__ W2p,
                                                TokFn tok, int R, int V, int r, int n_t,
                                                const Epi& epi, unsigned* __restrict__ queue,
                                                int w1_rows, int G, int gb) {
  typedef EngineGeom<BF16, KC, NW> Geo;
  typedef typename Elem<BF16>::Frag Frag;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_grab[2];
  Frag* cur = reinterpret_cast<Frag*>(smem);
  Frag* nxt = cur + Geo::kTileFrags;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int g = lane >> 4, nl = lane & 15;
  const Frag* src = reinterpret_cast<const Frag*>(W2p);
  const XcdShare xs = xcd_share(n_t, G, gb);  // hi > lo: at most n_t workgroups per engine
  unsigned* counter = queue + (gb % kNumXcd) * kQueueStride;
  const int qbase = xs.lo + kStaticTiles * xs.gx;  // first tile the queue hands out
  auto clampt = [&](int t) { return min(t, xs.hi - 1); };
  int tc = xs.lo + xs.j, tn = tc + xs.gx, tnn = tn + xs.gx;  // current, next, next-but-one
  if (tc >= xs.hi) return;  // workgroup-uniform; no barrier passed yet

  // prologue: the lane's tokens, then W2 and rows of tile tc, then the
  // (token -> W1 row) gather, which waits on the token loads alone
  int xtok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) xtok[nb] = tok(min((wave + NW * nb) * kTileN + nl, R - 1));
  Frag wq[Geo::kPer];
  typename Epi::Pre uc[NB], un[NB];
  {
    const Frag* s = src + (size_t)tc * Geo::kTileFrags;
#pragma unroll
    for (int i = 0; i < Geo::kPer; ++i) wq[i] = s[Geo::slot(i, tid)];
  }
  typename Epi::St st[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) st[nb] = epi.prepare((wave + NW * nb) * kTileN + nl);
  {
    const int v0 = tc * kTileV + 16 * g;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) epi.load(st[nb], v0, min(16, V - v0), uc[nb]);
  }
  Frag b[NB][KC];
  gather_b<BF16, KC, NB, VEC>(W1, xtok, R, r, w1_rows, wave, NW, lane, b);
  epi.side_work();
  wait_vm<0>();
#pragma unroll
  for (int i = 0; i < Geo::kPer; ++i) cur[Geo::slot(i, tid)] = wq[i];
  __syncthreads();

  // steady state. Each step claims the tile three steps ahead (the atomic
  // returns while the step multiplies) and publishes it before the barrier.
  // A workgroup's tiles increase, so the first one past the range ends it.
  int par = 0;
  for (;;) {
    unsigned grab = 0;
    if (tid == 0) grab = atomicAdd(counter, 1u);
    {
      const int tl = clampt(tn);
      const Frag* s = src + (size_t)tl * Geo::kTileFrags;
#pragma unroll
      for (int k = 0; k < Geo::kPer; ++k) wq[k] = s[Geo::slot(k, tid)];
      const int v0n = tl * kTileV + 16 * g;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) epi.load(st[nb], v0n, min(16, V - v0n), un[nb]);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the multiply

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
    const int v0 = tc * kTileV + 16 * g;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) epi.finish(st[nb], v0, min(16, V - v0), acc[nb], uc[nb], tc, lane);

    // the step's loads (and the claim) are in once at most its NB stores are
    // outstanding
    wait_vm<NB>();
#pragma unroll
    for (int k = 0; k < Geo::kPer; ++k) nxt[Geo::slot(k, tid)] = wq[k];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) uc[nb] = un[nb];
    if (tid == 0) s_grab[par] = qbase + (int)grab;
    __syncthreads();
    Frag* t_ = cur;
    cur = nxt;
    nxt = t_;
    tc = tn;
    tn = tnn;
    tnn = max(s_grab[par], tn + 1);
    par ^= 1;
    if (tc >= xs.hi) break;
  }
}

}  // namespace dspark
