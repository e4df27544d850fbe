// dspark_markov_draft for callers that cannot allocate (code under graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the draft's
// workspace is a file-scope device array instead of a caller buffer.
//
// The array is the same workspace dspark_markov_draft takes (tile partials,
// tile-queue counters, draft uniforms, the resident kernel's hand-off block),
// at most kNoAllocScratchBytes. Each device the library runs on holds its own
// copy until the process ends; its address is looked up once per device with
// hipGetSymbolAddress and kept. Every call zero-fills the workspace's
// bookkeeping tail first (a fill kernel on the caller's stream), since the
// previous call may have had other sizes and left partials where this call's
// counters lie. All calls on one device share the array: calls that overlap
// on one device (two streams, or two threads) race and give undefined
// outputs.
#include "dspark_device.hpp"
#include "dspark_host.hpp"

namespace dspark {
namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;  // 8 MiB: R = 256 at V = 163840
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

void* g_scratch[kMaxDevices] = {nullptr};

// The device address of this device's scratch array (nullptr on failure).
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace
}  // namespace dspark

using namespace dspark;

extern "C" size_t dspark_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int dspark_markov_draft_noalloc(const void* U, const void* W1, const void* W2p,
                                           const int32_t* anchor, uint64_t seed, uint64_t step,
                                           const uint64_t* step_dev, const uint32_t* req_ids,
                                           int R, int gamma, int V, int r, int dtype,
                                           int32_t* tokens, float* p_draft, float* lse_draft,
                                           void* stream) {
  int st = check_sizes(R, gamma, V, r, dtype);
  if (st) return st;
  if (!U || !W1 || !W2p || !anchor || !req_ids || !tokens || !p_draft || !lse_draft)
    return DSPARK_EINVAL;
  const size_t need = markov_ws_bytes(R, V);
  if (need > kNoAllocScratchBytes) return DSPARK_EWORKSPACE;
  void* ws = scratch_ptr();
  if (ws == nullptr) return DSPARK_EHIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t tail = markov_tail_offset(R, V);
  st = zero_fill(static_cast<char*>(ws) + tail, need - tail, s);
  if (st) return st;
  return markov_draft_checked(U, W1, W2p, anchor, seed, StepArg{step, step_dev}, req_ids, R, gamma,
                              V, r, dtype, tokens, p_draft, lse_draft, ws, s);
}
