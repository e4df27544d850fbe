// Host-side helpers shared by the C ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dspark.h"

namespace dspark {

constexpr int kMaxGamma = 16;
constexpr int kMaxRows = 4096;      // R * (gamma + 1)
constexpr int kMaxRankBf16 = 256;
constexpr int kMaxRankF32 = 128;
constexpr int kMaxTiers = 32;
// Requests whose W1 rows one GEMM launch holds in registers: 16 blocks of 16
// for bfloat16 (two per wave), 8 blocks for float32, whose 8-float operands
// would not fit twice per wave.
template <bool BF16> constexpr int req_group() { return BF16 ? 256 : 128; }

inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Request groups a workspace keeps tile-queue counters for (enough for either
// dtype).
inline int queue_groups(int R) { return ceil_div(R, 128); }

inline int rank_chunks(int r) { return ceil_div(r, 32); }
// KC rounded up to the instantiated set {1, 2, 4, 8}.
inline int kc_instance(int r) {
  const int kc = rank_chunks(r);
  return kc <= 1 ? 1 : kc <= 2 ? 2 : kc <= 4 ? 4 : 8;
}
inline int n_vtiles(int V) { return ceil_div(V, 64); }
// Request-major tile partial rows: c = ceil(n_t / 256) tiles per thread of the
// 256-thread select workgroup, rows of 256 c partials (tile t at
// part_pos(t, c), see dspark_device.hpp).
constexpr int kSelThreadsHost = 256;
inline int part_chunk(int V) { return ceil_div(n_vtiles(V), kSelThreadsHost); }
inline int part_ld(int V) { return kSelThreadsHost * part_chunk(V); }

// Vector paths: rows 16-byte aligned with V and the row stride multiples of
// the vector width; W1 16-byte aligned with r a multiple of 8.
inline bool rows_vec_ok(const void* p, long long ld, int V, int vec_elems) {
  return (V % vec_elems) == 0 && (ld % vec_elems) == 0 && (reinterpret_cast<uintptr_t>(p) % 16) == 0;
}
inline bool w1_vec_ok(const void* W1, int r) {
  return (r % 8) == 0 && (reinterpret_cast<uintptr_t>(W1) % 16) == 0;
}

inline bool dtype_ok(int dt) { return dt == DSPARK_F32 || dt == DSPARK_BF16; }
inline size_t dtype_bytes(int dt) { return dt == DSPARK_BF16 ? 2 : 4; }

// Compute units of the current device (cached per device id).
int device_cu_count();

// Workgroups for a persistent tile-engine launch over n_t tiles with at most
// max_g resident: one per tile up to max_g, else max_g. The tile queues hand
// the tiles of a last, partial round to whichever workgroups are ahead, so
// every resident slot is used (2374 tiles on 256 slots: 256 workgroups, not
// the 238 that would make every round full, which measured slower).
inline int engine_grid(int n_t, int max_g) {
  if (n_t <= max_g) return n_t > 0 ? n_t : 1;
  return max_g;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? DSPARK_OK : DSPARK_EHIP; }

// Check the launch that was just enqueued.
inline int launch_status() { return hip_status(hipGetLastError()); }

// Sizes shared by several calls.
inline int check_sizes(int R, int gamma, int V, int r, int dt) {
  if (!dtype_ok(dt)) return DSPARK_EDTYPE;
  if (R < 1 || gamma < 1 || V < 1 || r < 1) return DSPARK_ESIZE;
  if (gamma > kMaxGamma) return DSPARK_ESIZE;
  if ((long long)R * (gamma + 1) > kMaxRows) return DSPARK_ESIZE;
  if (r > (dt == DSPARK_BF16 ? kMaxRankBf16 : kMaxRankF32)) return DSPARK_ESIZE;
  if ((long long)V * (long long)R * (gamma + 1) > (1ll << 40)) return DSPARK_ESIZE;
  return DSPARK_OK;
}

// Workspace layout pieces (bytes, 256-aligned).
size_t markov_ws_bytes(int R, int V);
// Start of the draft workspace's bookkeeping tail (tile-queue counters, draft
// uniforms, hand-off block); the tile partials lie before it.
size_t markov_tail_offset(int R, int V);
// Zero-fill n bytes at p on stream s (the kernel behind dspark_workspace_init).
int zero_fill(void* p, size_t n, hipStream_t s);
// Hand-off block of a draft workspace (resident-W2 kernel): call epoch, exit
// counter and error word, per-unit ready words and per-request tagged tokens.
constexpr size_t kResidentBarBytes = 4096;
constexpr size_t kResidentErrByte = 512;  // the error word's offset in the block
size_t resident_bar_offset(int R, int V);

// The resident-W2 draft (resident.hip): whether a call of these sizes,
// pointers and dtype takes it, and the launch (bfloat16, rank chunk count 8).
struct StepArg;
struct ConfArgs;
bool resident_draft_eligible(const void* U, const void* W1, int R, int gamma, int V, int r,
                             int dtype);
// dspark_markov_draft after its argument checks (ws: a draft workspace for R, V).
int markov_draft_checked(const void* U, const void* W1, const void* W2p, const int32_t* anchor,
                         uint64_t seed, StepArg step, const uint32_t* req_ids, int R, int gamma,
                         int V, int r, int dtype, int32_t* tokens, float* p_draft, float* lse_draft,
                         void* ws, hipStream_t s);
int resident_draft_launch(const void* U, const void* W1, const void* W2p, const int32_t* anchor,
                          uint64_t seed, StepArg step, const uint32_t* req_ids, int R, int gamma,
                          int V, int r, int32_t* tokens, float* p_draft, float* lse_draft,
                          void* ws, const ConfArgs& ca, hipStream_t s);
// 16-byte load flags of the confidence head's two dot products (alignment and
// lengths of h, the W1 rows and the weight vector)
void confidence_vec_flags(const void* h, const void* W1, const float* w, int d, int r, int dtype,
                          bool& vec_h, bool& vec_w1);
size_t verify_ws_bytes(int R, int gamma, int V);
size_t accept_ws_bytes(int R, int gamma, int V);

}  // namespace dspark
