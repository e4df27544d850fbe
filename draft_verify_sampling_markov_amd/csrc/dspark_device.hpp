// Device-side building blocks shared by the DSpark kernels (gfx950 / CDNA4).
//
// - element access for float32 and bfloat16 storage
// - Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11), written from its
//   published definition
// - deterministic wave reductions (fixed butterfly order)
// - the Markov bias tile: a 64-vocabulary x 16-request block of
//   W1[x_prev] . W2 on the matrix cores (v_mfma_f32_16x16x32_bf16 for bf16,
//   v_mfma_f32_16x16x4_f32 for f32)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

constexpr int kWave = 64;
constexpr int kTileV = 64;     // vocabulary entries per Markov tile
constexpr int kTileN = 16;     // requests per Markov tile
constexpr int kChunkK = 32;    // rank entries per matrix-core step
constexpr int kLdsPad = 8;     // elements of padding per W1 row in LDS

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// storage types
// ---------------------------------------------------------------------------

template <bool BF16> struct Elem;
template <> struct Elem<true> {
  typedef uint16_t T;       // bfloat16 bit pattern
  typedef bf16x8 Frag;      // 8 values = one matrix-core operand
  static constexpr int kVec = 8;  // elements per 16-byte load
};
template <> struct Elem<false> {
  typedef float T;
  typedef f32x8 Frag;
  static constexpr int kVec = 4;
};

__device__ __forceinline__ float to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ float to_f32(float f) { return f; }

// 16 consecutive elements p[0..15] as float; `n` of them are in range
// (n >= 16: all). `vec` says p is 16-byte aligned for vector loads.
template <bool BF16>
__device__ __forceinline__ void load16(const typename Elem<BF16>::T* __restrict__ p, int n, bool vec,
                                       float out[16]) {
  if (vec && n >= 16) {
    if constexpr (BF16) {
      const u32x4* q = reinterpret_cast<const u32x4*>(p);
      u32x4 a = __builtin_nontemporal_load(q);
      u32x4 b = __builtin_nontemporal_load(q + 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(a[i] << 16);
        out[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
        out[8 + 2 * i] = __uint_as_float(b[i] << 16);
        out[8 + 2 * i + 1] = __uint_as_float(b[i] & 0xFFFF0000u);
      }
    } else {
      const f32x4* q = reinterpret_cast<const f32x4*>(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 a = __builtin_nontemporal_load(q + i);
        out[4 * i] = a[0];
        out[4 * i + 1] = a[1];
        out[4 * i + 2] = a[2];
        out[4 * i + 3] = a[3];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) out[i] = (i < n) ? to_f32(p[i]) : 0.0f;
  }
}


// 16 consecutive elements kept as raw 16-byte words (bf16: 2 words holding
// 8 values each; f32: 4 words), so a prefetch costs 8 or 16 VGPRs.
template <bool BF16>
struct Raw16 {
  u32x4 w[BF16 ? 2 : 4];
};

template <bool BF16>
__device__ __forceinline__ void load16_raw(const typename Elem<BF16>::T* __restrict__ p, int n,
                                           bool vec, Raw16<BF16>& r) {
  constexpr int NW = BF16 ? 2 : 4;
  if (vec && n >= 16) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < NW; ++i) r.w[i] = __builtin_nontemporal_load(q + i);
  } else {
    uint32_t bits[4 * NW];
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t lo = (2 * i < n) ? p[2 * i] : 0u;
        const uint32_t hi = (2 * i + 1 < n) ? p[2 * i + 1] : 0u;
        bits[i] = lo | (hi << 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) bits[i] = (i < n) ? __float_as_uint(p[i]) : 0u;
    }
#pragma unroll
    for (int i = 0; i < NW; ++i)
      r.w[i] = u32x4{bits[4 * i], bits[4 * i + 1], bits[4 * i + 2], bits[4 * i + 3]};
  }
}

// Branch-free load of 16 elements row[v0 .. v0+16) for the engine's
// pipelined epilogues. Every address stays inside the row [0, V): with VEC
// (16-byte aligned rows, V a multiple of the vector width) word i reads from
// v0 + VEC * min(i, words_valid - 1), and a lane past the end reads from the
// row start; without VEC each element is read from min(v0 + i, V - 1). Entries
// at or beyond nvalid hold arbitrary row values and must be masked by the
// caller. The loads carry no nontemporal hint: these rows are read once, but
// on MI355X the plain cached loads measured faster here, as the tile
// pipeline issues them beside the re-read W2 stream.
template <bool BF16, bool VEC>
__device__ __forceinline__ void load16_clamped(const typename Elem<BF16>::T* __restrict__ row,
                                               int v0, int nvalid, int V, Raw16<BF16>& r) {
  constexpr int W = BF16 ? 2 : 4;
  constexpr int PER = Elem<BF16>::kVec;
  if constexpr (VEC) {
    const int base = nvalid > 0 ? v0 : 0;
    const int nv = nvalid > 0 ? min(W, (nvalid + PER - 1) / PER) : 1;
    const u32x4* q = reinterpret_cast<const u32x4*>(row + base);
#pragma unroll
    for (int i = 0; i < W; ++i) r.w[i] = q[min(i, nv - 1)];
  } else {
    uint32_t bits[4 * W];
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t lo = row[min(v0 + 2 * i, V - 1)];
        const uint32_t hi = row[min(v0 + 2 * i + 1, V - 1)];
        bits[i] = lo | (hi << 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) bits[i] = __float_as_uint(row[min(v0 + i, V - 1)]);
    }
#pragma unroll
    for (int i = 0; i < W; ++i)
      r.w[i] = u32x4{bits[4 * i], bits[4 * i + 1], bits[4 * i + 2], bits[4 * i + 3]};
  }
}

constexpr float kLog2e = 1.44269504088896340736f;

// The value lane l ^ 16 (ROW = true) or l ^ 32 (ROW = false) holds, with the
// gfx950 lane-swap instructions: v_permlane16_swap with both operands x gives
// every lane the pair (row 2i, row 2i + 1) of its 32-lane half, in that
// order, and v_permlane32_swap the pair (lanes 0-31, lanes 32-63); the partner
// is the element that is not the lane's own. Plain VALU, where a shuffle
// through the LDS crossbar (ds_bpermute) waits on an LDS round trip.
template <bool ROW>
__device__ __forceinline__ float lane_partner(float x) {
  const unsigned u = __float_as_uint(x);
  const unsigned lane = __lane_id();
  if constexpr (ROW) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
  }
}

// Reduce x over the lane pair {l, l ^ 16} (ROW) or {l, l ^ 32}: both lanes
// get the same value, formed in the same operand order (the lower lane's
// value first), so sums are bit-identical across the pair.
template <bool ROW>
__device__ __forceinline__ float pair_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = ROW ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                     : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
template <bool ROW>
__device__ __forceinline__ float pair_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = ROW ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                     : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Softmax partial (m, s) of one request's 64 tile entries, 16 masked logits
// (-inf = masked) in each of the four lanes l, l ^ 16, l ^ 32, l ^ 48, without
// branches: m is the max over the 64 entries (over the lane's 16, then over
// the four lanes), s = sum of 2^(z log2 e - m log2 e) over the lane's 16 with
// the exponent formed by one fused multiply-add (v_exp_f32 computes 2^x), then
// summed over the four lanes; m log2 e is rounded once per tile, which scales
// the tile's terms alike by at most 2^(ulp(m log2 e) / 2). All four lanes end
// with the same (m, s). m = -inf (all masked) gives s = 0.
__device__ __forceinline__ void softmax16_merge4(const float z[16], float& m_out, float& s_out) {
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, z[i]);
  m = pair_max<true>(m);
  m = pair_max<false>(m);
  const float mref = (m == -INFINITY) ? 0.0f : m;
  const float mb = -mref * kLog2e;
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += __builtin_amdgcn_exp2f(fmaf(z[i], kLog2e, mb));
  s = pair_sum<true>(s);
  s = pair_sum<false>(s);
  m_out = m;
  s_out = s;
}

template <bool BF16>
__device__ __forceinline__ void unpack16(const Raw16<BF16>& r, float out[16]) {
  if constexpr (BF16) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[8 * h + 2 * i] = __uint_as_float(r.w[h][i] << 16);
        out[8 * h + 2 * i + 1] = __uint_as_float(r.w[h][i] & 0xFFFF0000u);
      }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) out[4 * h + i] = __uint_as_float(r.w[h][i]);
  }
}

template <bool BF16>
__device__ __forceinline__ void zero16(Raw16<BF16>& r) {
#pragma unroll
  for (int i = 0; i < (BF16 ? 2 : 4); ++i) r.w[i] = u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// Philox4x64-10
// ---------------------------------------------------------------------------

constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;  // golden ratio
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;  // sqrt(3) - 1

struct U64x4 { uint64_t w[4]; };

__device__ __forceinline__ U64x4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                               uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint64_t hi0 = __umul64hi(kPhiloxM0, c0), lo0 = kPhiloxM0 * c0;
    const uint64_t hi1 = __umul64hi(kPhiloxM1, c2), lo1 = kPhiloxM1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  U64x4 r;
  r.w[0] = c0;
  r.w[1] = c1;
  r.w[2] = c2;
  r.w[3] = c3;
  return r;
}

enum { kPurposeDraft = 0, kPurposeAccept = 1, kPurposeResidual = 2, kPurposeBonus = 3 };

// The Philox step of a call: a launch argument, or, when dev is set, a word in
// device memory read when the kernel runs, so that a launch recorded once (a
// captured graph) follows a step counter the device advances.
struct StepArg {
  uint64_t value;
  const uint64_t* dev;
  __device__ __forceinline__ uint64_t get() const { return dev != nullptr ? *dev : value; }
};

// Uniform in [0, 1 - 2^-24] for slot k of request req_id: word `purpose` of the
// Philox block with counter (k, req_id, step, 0) and key (seed, 0).
__device__ __forceinline__ float slot_uniform(uint64_t seed, uint64_t step, uint32_t req_id, int k,
                                              int purpose) {
  const U64x4 b = philox4x64_10((uint64_t)k, (uint64_t)req_id, step, 0ull, seed, 0ull);
  const uint32_t top = (uint32_t)(b.w[purpose] >> 40);
  return (float)top * 5.9604644775390625e-8f;  // 2^-24, exact
}

// ---------------------------------------------------------------------------
// wave reductions (fixed order, deterministic)
// ---------------------------------------------------------------------------

// Cross-lane steps use DPP row operations (gfx9-family encodings): the
// quad permutes swap lanes 1 and 2 apart, the mirrors reverse a half-row / a
// row, row_shr:n shifts within a 16-lane row, row_bcast:15 / :31 carry the
// last lane of a row / of lanes 0-31 into the following rows, wave_shr:1
// shifts the whole wave by one lane. Lanes a step does not write keep `old`.
enum : int {
  kDppXor1 = 0xB1,          // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,          // quad_perm [2,3,0,1]
  kDppRowShr1 = 0x111,
  kDppRowShr2 = 0x112,
  kDppRowShr4 = 0x114,
  kDppRowShr8 = 0x118,
  kDppWaveShr1 = 0x138,
  kDppRowMirror = 0x140,
  kDppRowHalfMirror = 0x141,
  kDppRowBcast15 = 0x142,
  kDppRowBcast31 = 0x143,
};

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Largest value over the 64 lanes, returned to every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v, v));
  v = fmaxf(v, dpp_f<kDppXor2>(v, v));
  v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v, v));
  v = fmaxf(v, dpp_f<kDppRowMirror>(v, v));
  v = fmaxf(v, dpp_f<kDppRowBcast15, 0xA>(v, v));
  v = fmaxf(v, dpp_f<kDppRowBcast31, 0xC>(v, v));
  return readlane_f(v, kWave - 1);
}
__device__ __forceinline__ int wave_max_int(int v) {
  v = max(v, dpp_i<kDppXor1>(v, v));
  v = max(v, dpp_i<kDppXor2>(v, v));
  v = max(v, dpp_i<kDppRowHalfMirror>(v, v));
  v = max(v, dpp_i<kDppRowMirror>(v, v));
  v = max(v, dpp_i<kDppRowBcast15, 0xA>(v, v));
  v = max(v, dpp_i<kDppRowBcast31, 0xC>(v, v));
  return __builtin_amdgcn_readlane(v, kWave - 1);
}
// Sum over the 64 lanes in a fixed order, returned to every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppXor1>(0.0f, v);
  v += dpp_f<kDppXor2>(0.0f, v);
  v += dpp_f<kDppRowHalfMirror>(0.0f, v);
  v += dpp_f<kDppRowMirror>(0.0f, v);
  v += dpp_f<kDppRowBcast15, 0xA>(0.0f, v);
  v += dpp_f<kDppRowBcast31, 0xC>(0.0f, v);
  return readlane_f(v, kWave - 1);
}
// Inclusive prefix sum over the 64 lanes (Hillis-Steele within rows, then the
// row carries; fixed order).
__device__ __forceinline__ float wave_inclusive_scan(float v, int /*lane*/) {
  v += dpp_f<kDppRowShr1>(0.0f, v);
  v += dpp_f<kDppRowShr2>(0.0f, v);
  v += dpp_f<kDppRowShr4>(0.0f, v);
  v += dpp_f<kDppRowShr8>(0.0f, v);
  v += dpp_f<kDppRowBcast15, 0xA>(0.0f, v);
  v += dpp_f<kDppRowBcast31, 0xC>(0.0f, v);
  return v;
}
// The value of the previous lane (0 for lane 0).
__device__ __forceinline__ float wave_shift_up1(float v) { return dpp_f<kDppWaveShr1>(0.0f, v); }

// Integer versions (exact, so the order does not matter for the result).
__device__ __forceinline__ uint32_t wave_inclusive_scan_u32(uint32_t v) {
  v += (uint32_t)dpp_i<kDppRowShr1>(0, (int)v);
  v += (uint32_t)dpp_i<kDppRowShr2>(0, (int)v);
  v += (uint32_t)dpp_i<kDppRowShr4>(0, (int)v);
  v += (uint32_t)dpp_i<kDppRowShr8>(0, (int)v);
  v += (uint32_t)dpp_i<kDppRowBcast15, 0xA>(0, (int)v);
  v += (uint32_t)dpp_i<kDppRowBcast31, 0xC>(0, (int)v);
  return v;
}
__device__ __forceinline__ int wave_min_int(int v) {
  v = min(v, dpp_i<kDppXor1>(v, v));
  v = min(v, dpp_i<kDppXor2>(v, v));
  v = min(v, dpp_i<kDppRowHalfMirror>(v, v));
  v = min(v, dpp_i<kDppRowMirror>(v, v));
  v = min(v, dpp_i<kDppRowBcast15, 0xA>(v, v));
  v = min(v, dpp_i<kDppRowBcast31, 0xC>(v, v));
  return __builtin_amdgcn_readlane(v, kWave - 1);
}

// (largest th, then smallest k) over the 64 lanes, returned to every lane.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ void argmax_step(unsigned long long& th, int& k) {
  const int lo = (int)(uint32_t)th, hi = (int)(uint32_t)(th >> 32);
  const uint32_t olo = (uint32_t)dpp_i<CTRL, ROW_MASK>(lo, lo);
  const uint32_t ohi = (uint32_t)dpp_i<CTRL, ROW_MASK>(hi, hi);
  const int ok = dpp_i<CTRL, ROW_MASK>(k, k);
  const unsigned long long ot = ((unsigned long long)ohi << 32) | olo;
  const bool better = ot > th || (ot == th && ok < k);
  th = better ? ot : th;
  k = better ? ok : k;
}
__device__ __forceinline__ void wave_argmax_u64(unsigned long long& th, int& k) {
  argmax_step<kDppXor1>(th, k);
  argmax_step<kDppXor2>(th, k);
  argmax_step<kDppRowHalfMirror>(th, k);
  argmax_step<kDppRowMirror>(th, k);
  argmax_step<kDppRowBcast15, 0xA>(th, k);
  argmax_step<kDppRowBcast31, 0xC>(th, k);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)th, kWave - 1);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(th >> 32), kWave - 1);
  th = ((unsigned long long)hi << 32) | lo;
  k = __builtin_amdgcn_readlane(k, kWave - 1);
}

// Dot product of `len` stored elements with float weights, by one wave: 16-byte
// loads when `vec` (len a multiple of the vector width, rows and weights
// aligned). All of a lane's loads, of the elements and of their weights, go
// out from clamped addresses before the first product (a load under a bounds
// branch would wait for the sums before it); the products are then summed in
// chunk and element order.
template <bool BF16>
__device__ __forceinline__ float wave_dot(const typename Elem<BF16>::T* __restrict__ x,
                                          const float* __restrict__ w, int len, bool vec, int lane) {
  constexpr int VEC = Elem<BF16>::kVec;
  constexpr int WV = VEC / 4;  // weight vectors of four per chunk
  float acc = 0.0f;
  if (vec) {
    const int nv = len / VEC;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    const f32x4* wv = reinterpret_cast<const f32x4*>(w);
    constexpr int U = 8;  // chunks per lane and round: 4096 bfloat16 elements per wave
    for (int base = 0; base < nv; base += U * kWave) {
      u32x4 q[U];
      f32x4 wt[U][WV];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        if (base + i * kWave < nv) {  // wave-uniform: chunk groups past the end are not loaded
          const int c = min(base + i * kWave + lane, nv - 1);
          q[i] = xv[c];
#pragma unroll
          for (int t = 0; t < WV; ++t) wt[i][t] = wv[(size_t)c * WV + t];
        }
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        if (base + i * kWave + lane < nv) {
          if constexpr (BF16) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc += __uint_as_float(q[i][e] << 16) * wt[i][(2 * e) / 4][(2 * e) % 4];
              acc += __uint_as_float(q[i][e] & 0xFFFF0000u) * wt[i][(2 * e + 1) / 4][(2 * e + 1) % 4];
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc += __uint_as_float(q[i][e]) * wt[i][0][e];
          }
        }
      }
    }
  } else {
    for (int i = lane; i < len; i += kWave) acc += to_f32(x[i]) * w[i];
  }
  return wave_sum(acc);
}

// The confidence head's logit for one slot, by one wave: w . [h_k ; W1[x_{k-1}]] + b
// (the hidden-state dot, then the W1-row dot, each a fixed-order wave sum).
template <bool BF16>
__device__ __forceinline__ float conf_logit(const typename Elem<BF16>::T* __restrict__ h_row,
                                            const typename Elem<BF16>::T* __restrict__ w1_row,
                                            const float* __restrict__ w, float b, int d, int r,
                                            bool vec_h, bool vec_w1, int lane) {
  const float zh = wave_dot<BF16>(h_row, w, d, vec_h, lane);
  const float ze = wave_dot<BF16>(w1_row, w + d, r, vec_w1, lane);
  return zh + ze + b;
}

// Inputs of the confidence head for a draft call that also scores its slots
// (h == nullptr: it does not). Layouts as dspark_confidence's.
struct ConfArgs {
  const void* h;          // [R, gamma, d] hidden states, storage type
  const float* w;         // [d + r]
  float b;
  const float* inv_temp;  // [gamma] or nullptr
  int d;
  bool vec_h, vec_w1;     // 16-byte loads allowed (alignment and lengths checked on the host)
  float* conf;            // [R, gamma]
  float* surv;            // [R, gamma]
  float* logit;           // [R, gamma] or nullptr
};

// Merge two (max, sum of exp(z - max)) softmax partials.
__device__ __forceinline__ void softmax_merge(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) {
    m = mm;
    s = 0.0f;
    return;
  }
  s = s * __expf(m - mm) + s2 * __expf(m2 - mm);
  m = mm;
}

__device__ __forceinline__ int clamp_token(int x, int V) { return x < 0 ? 0 : (x >= V ? V - 1 : x); }

// ---------------------------------------------------------------------------
// Markov bias tile on the matrix cores
// ---------------------------------------------------------------------------
//
// Pre-packed W2 layout (written by the prepack kernel): for tile t (64
// vocabulary entries), rank chunk kc (32 ranks), sub-tile j (0..3) and lane l:
// 8 consecutive elements
//     W2p[(((t * KC + kc) * 4 + j) * 64 + l) * 8 + e] = W2[kc*32 + 8*(l/16) + e, v]
//     v = 64 t + 16 (rho / 4) + 4 j + (rho % 4),  rho = l % 16
// (zero outside r x V). With the matrix-core output layout (lane l holds
// column l % 16 and rows 4 (l/16) .. 4 (l/16) + 3 of each 16 x 16 sub-tile),
// lane l of a 16-request tile then ends up holding the 16 consecutive
// vocabulary entries v = 64 t + 16 (l/16) + [0, 16) of request l % 16, entry
// 4 j + i in acc[j][i].
//
// The W1 rows of the tile's 16 requests sit in LDS, row n at lds + n * ldw,
// with ldw = KC * 32 + kLdsPad elements (padding spreads rows over banks).
// Lane l reads ranks kc*32 + 8 (l/16) .. +8 of row l % 16.
//
// For float32 the 32-rank chunk is eight 16x16x4 steps; in step s, lane l
// contributes rank kc*32 + 8 (l/16) + s on both operands, so the two operands
// stay matched.

template <bool BF16, int KC>
struct ATile {
  typename Elem<BF16>::Frag a[KC][4];
};

template <bool BF16, int KC>
__device__ __forceinline__ void load_a_tile(const typename Elem<BF16>::T* __restrict__ W2p, int t,
                                            int lane, ATile<BF16, KC>& at) {
  typedef typename Elem<BF16>::Frag Frag;
  const Frag* base = reinterpret_cast<const Frag*>(W2p) + (size_t)t * KC * 4 * kWave;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
#pragma unroll
    for (int j = 0; j < 4; ++j) at.a[kc][j] = base[(kc * 4 + j) * kWave + lane];
}

template <bool BF16>
__device__ __forceinline__ void mma_step(f32x4& acc, const typename Elem<BF16>::Frag& a,
                                         const typename Elem<BF16>::Frag& b) {
  if constexpr (BF16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
  }
}

// acc[j] = sum over ranks of W2-tile x W1-rows for the 16 requests whose rows
// start at lds_rows (row stride ldw).
template <bool BF16, int KC>
__device__ __forceinline__ void tile_mma(const ATile<BF16, KC>& at,
                                         const typename Elem<BF16>::T* lds_rows, int ldw, int lane,
                                         f32x4 acc[4]) {
  typedef typename Elem<BF16>::Frag Frag;
  const typename Elem<BF16>::T* brow = lds_rows + (lane & 15) * ldw + 8 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const Frag b = *reinterpret_cast<const Frag*>(brow + kc * kChunkK);
#pragma unroll
    for (int j = 0; j < 4; ++j) mma_step<BF16>(acc[j], at.a[kc][j], b);
  }
}

// ---------------------------------------------------------------------------
// W1 row staging: rows of `count` requests whose tokens are xprev[n*xstride]
// ---------------------------------------------------------------------------

template <bool BF16>
__device__ __forceinline__ void stage_rows(const typename Elem<BF16>::T* __restrict__ W1,
                                           const int* __restrict__ xprev, int xstride, int count,
                                           int rows, int r, int V, int kpad, int ldw,
                                           typename Elem<BF16>::T* lds) {
  typedef typename Elem<BF16>::T T;
  constexpr int VEC = Elem<BF16>::kVec;
  const int tid = threadIdx.x, nth = blockDim.x;
  if ((r % VEC) == 0) {
    const int per_row = kpad / VEC;
    const int total = rows * per_row;
    for (int idx = tid; idx < total; idx += nth) {
      const int n = idx / per_row, c = idx - n * per_row;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (n < count && c * VEC < r) {
        const int tok = clamp_token(xprev[(size_t)n * xstride], V);
        v = *reinterpret_cast<const u32x4*>(W1 + (size_t)tok * r + c * VEC);
      }
      *reinterpret_cast<u32x4*>(lds + n * ldw + c * VEC) = v;
    }
  } else {
    const int total = rows * kpad;
    for (int idx = tid; idx < total; idx += nth) {
      const int n = idx / kpad, k = idx - n * kpad;
      T v = (T)0;
      if (n < count && k < r) v = W1[(size_t)clamp_token(xprev[(size_t)n * xstride], V) * r + k];
      lds[n * ldw + k] = v;
    }
  }
}

// z values of one tile for the lane's request (lane & 15) and entries
// v0 + [0, 16), v0 = 64 t + 16 (lane >> 4); invalid entries get -inf.
template <bool BF16>
__device__ __forceinline__ void tile_logits(const f32x4 acc[4], const float u16[16], int nvalid,
                                            bool active, float z[16]) {
  // every lane of the wave holds 16 valid entries of an active request (all
  // tiles but the last, when R fills the blocks): no masks
  if (__all(active && nvalid >= 16)) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) z[4 * j + i] = acc[j][i] + u16[4 * j + i];
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = 4 * j + i;
      const float val = acc[j][i] + u16[idx];
      z[idx] = (active && idx < nvalid) ? val : -INFINITY;
    }
}



// ---------------------------------------------------------------------------
// workgroup inverse-CDF tile search
// ---------------------------------------------------------------------------
//
// One workgroup of kSelThreads threads per request. Thread p owns the c
// consecutive tiles [p c, p c + cnt) (cnt <= c; c = ceil(n_t / kSelThreads))
// with weights w(i), i < cnt. The group forms S = sum of all weights (thread
// sums in tile order, a fixed-order scan over the lanes of each wave, then the
// wave totals in wave order) and T = u S, finds the first thread whose
// inclusive prefix exceeds T, and that thread walks its tiles to the first one
// where the running sum crosses T (ABS: T = u as given). Result (in every thread): the crossing
// tile and the mass before it (pb). When rounding leaves no crossing, the
// result is the last tile with positive weight and pb = -inf, which makes the
// in-tile search end at that tile's last positive entry. CMAX > 0: the
// weights sit in registers (w(i) is called with compile-time i < CMAX);
// CMAX == 0: a rolled loop (weights re-read).

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;

struct WaveSearch {
  int tstar;
  float pb, S, T;
};

struct BlockSearchShared {
  float red[kSelWaves];
  float wsum[kSelWaves];
  int wlast[kSelWaves];
  int wfirst[kSelWaves];
  int tstar;
  float pb;
};

// Largest value over the workgroup (every thread gets it); one barrier.
__device__ __forceinline__ float block_max(float v, BlockSearchShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  v = wave_max(v);
  if (lane == 0) sh.red[wave] = v;
  __syncthreads();
  float m = sh.red[0];
#pragma unroll
  for (int q = 1; q < kSelWaves; ++q) m = fmaxf(m, sh.red[q]);
  return m;
}

// Sum over the workgroup in a fixed order (every thread gets it); one barrier.
__device__ __forceinline__ float block_sum(float v, BlockSearchShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  v = wave_sum(v);
  if (lane == 0) sh.red[wave] = v;
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < kSelWaves; ++q) s += sh.red[q];
  return s;
}

template <int CMAX, bool ABS = false, typename WFn>
__device__ __forceinline__ WaveSearch block_tile_search(WFn w, int t0, int cnt, float u,
                                                        BlockSearchShared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  float ls = 0.0f;
  if constexpr (CMAX > 0) {
#pragma unroll
    for (int i = 0; i < CMAX; ++i)
      if (i < cnt) ls += w(i);
  } else {
    for (int i = 0; i < cnt; ++i) ls += w(i);
  }
  float incl = wave_inclusive_scan(ls, lane);
  if (lane == kWave - 1) sh.wsum[wave] = incl;
  __syncthreads();
  float off = 0.0f, S = 0.0f;
#pragma unroll
  for (int q = 0; q < kSelWaves; ++q) {
    if (q < wave) off += sh.wsum[q];
    S += sh.wsum[q];
  }
  WaveSearch r;
  r.S = S;
  r.T = ABS ? u : u * S;  // ABS: u is the threshold itself, not a fraction of S
  const float prev = wave_shift_up1(incl) + off;
  incl += off;
  const unsigned long long pm = __ballot(incl > r.T);
  if (lane == 0) sh.wfirst[wave] = pm ? wave * kWave + __ffsll((long long)pm) - 1 : 0x7fffffff;
  __syncthreads();
  int pstar = 0x7fffffff;
#pragma unroll
  for (int q = 0; q < kSelWaves; ++q) pstar = min(pstar, sh.wfirst[q]);
  // -1 below: rounding left no crossing (or the crossing thread holds no
  // positive weight); the result is then the workgroup's last positive tile
  int tstar = -1;
  r.pb = -INFINITY;
  if (pstar != 0x7fffffff) {  // uniform over the workgroup
    if (tid == pstar) {
      float cum = prev, pbv = -INFINITY;
      int found = -1, last = -1;
      if constexpr (CMAX > 0) {
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
      } else {
        for (int i = 0; i < cnt && found < 0; ++i) {
          const float wi = w(i);
          const float cn = cum + wi;
          if (cn > r.T) {
            found = t0 + i;
            pbv = cum;
          }
          if (wi > 0.0f) last = t0 + i;
          cum = cn;
        }
      }
      sh.tstar = found >= 0 ? found : last;
      sh.pb = found >= 0 ? pbv : -INFINITY;
    }
    __syncthreads();
    tstar = sh.tstar;
    r.pb = sh.pb;
  }
  if (tstar < 0) {  // uniform (read from shared memory, or pstar absent)
    int last = -1;
    if constexpr (CMAX > 0) {
#pragma unroll
      for (int i = 0; i < CMAX; ++i)
        if (i < cnt && w(i) > 0.0f) last = t0 + i;
    } else {
      for (int i = 0; i < cnt; ++i)
        if (w(i) > 0.0f) last = t0 + i;
    }
    const int wl = wave_max_int(last);
    if (lane == 0) sh.wlast[wave] = wl;
    __syncthreads();
    int glast = -1;
#pragma unroll
    for (int q = 0; q < kSelWaves; ++q) glast = max(glast, sh.wlast[q]);
    tstar = glast;
    r.pb = -INFINITY;
  }
  r.tstar = tstar;
  return r;
}

// B operand of a tile product whose 16 columns all hold one W1 row: lane l
// holds ranks kc*32 + 8 (l/16) .. +8 of `row` for every chunk kc (zero past r).
// VW: row 16-byte aligned and r a multiple of 8 (one vector load per chunk).
// Both paths are branch-free (clamped addresses, masked values), so the loads
// of all chunks stay in flight together.
template <bool BF16, int KC, bool VW>
__device__ __forceinline__ void load_b_row(const typename Elem<BF16>::T* __restrict__ row, int r,
                                           int lane, typename Elem<BF16>::Frag b[KC]) {
  typedef typename Elem<BF16>::T T;
  typedef typename Elem<BF16>::Frag Frag;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const int k0 = kc * kChunkK + 8 * (lane >> 4);
    if constexpr (VW) {
      const Frag f = *reinterpret_cast<const Frag*>(row + min(k0, r - 8));
      b[kc] = k0 < r ? f : Frag{};
    } else {
      T tmp[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const T v = row[min(k0 + e, r - 1)];
        tmp[e] = (k0 + e < r) ? v : (T)0;
      }
      b[kc] = *reinterpret_cast<const Frag*>(tmp);
    }
  }
}

// acc[j] = W2-tile x B over all rank chunks, B held in registers; the same
// accumulation order as tile_mma() and the GEMM engine.
template <bool BF16, int KC>
__device__ __forceinline__ void tile_mma_regs(const ATile<BF16, KC>& at,
                                              const typename Elem<BF16>::Frag (&b)[KC],
                                              f32x4 acc[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
#pragma unroll
    for (int j = 0; j < 4; ++j) mma_step<BF16>(acc[j], at.a[kc][j], b[kc]);
}

// The product entry lane l of a one-row tile product needs for tile entry l,
// acc[(l / 4) % 4][l % 4] (layout above), taken with exact 0/1 weights rather
// than an indexed read: the compiler turns indexed picks out of small arrays
// into LDS arrays addressed through the dispatch packet, a read of host memory.
// Exact for finite products (adds of zero).
__device__ __forceinline__ float own_entry(const f32x4 acc[4], int lane) {
  const int j = (lane >> 2) & 3, i = lane & 3;
  float r = 0.0f;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) r = fmaf(acc[jj][ii], (jj == j && ii == i) ? 1.0f : 0.0f, r);
  return r;
}

// Position of tile t's partial in a request's partial row, chunked for the
// select workgroup: thread p's tiles [p c, p c + c) load as c coalesced
// workgroup-wide reads, tile p c + i at i * kSelThreads + p. Rows hold
// kSelThreads * c partials.
__device__ __forceinline__ int part_pos(int t, int c) { return (t % c) * kSelThreads + t / c; }

// In-tile inverse-CDF search by one wave: lane i holds weight e_i of entry
// v = 64 t + i (0 outside the vocabulary). Returns the lane of the first entry
// whose cumulative weight pb + sum_{j <= i} e_j exceeds T, else the last lane
// with positive weight.
__device__ __forceinline__ int tile_pick(float e, bool valid, float pb, float T, int lane) {
  const float sc = wave_inclusive_scan(e, lane);
  const bool cross = valid && (pb + sc > T);
  const unsigned long long cm = __ballot(cross);
  if (cm) return __ffsll((long long)cm) - 1;
  const unsigned long long pm = __ballot(e > 0.0f);
  return pm ? 63 - __clzll((long long)pm) : 0;
}

}  // namespace dspark
