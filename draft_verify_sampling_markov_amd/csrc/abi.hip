// C ABI utilities: status strings, workspace sizing and initialisation.
#include "dspark_host.hpp"

#include <algorithm>

using namespace dspark;

extern "C" const char* dspark_status_string(int status) {
  switch (status) {
    case DSPARK_OK: return "DSPARK_OK: success";
    case DSPARK_EINVAL: return "DSPARK_EINVAL: null pointer or invalid argument";
    case DSPARK_EDTYPE: return "DSPARK_EDTYPE: unknown dtype";
    case DSPARK_ETIER: return "DSPARK_ETIER: capture tiers must be 1..32 positive ascending values";
    case DSPARK_ESIZE: return "DSPARK_ESIZE: size outside the supported limits";
    case DSPARK_EWORKSPACE: return "DSPARK_EWORKSPACE: workspace missing or too small";
    case DSPARK_EHIP: return "DSPARK_EHIP: HIP runtime or launch failure";
    default: return "DSPARK: unknown status";
  }
}

extern "C" size_t dspark_workspace_bytes(int call, int R, int gamma, int V, int r) {
  if (R < 1 || gamma < 1 || gamma > kMaxGamma || V < 1 || r < 1) return 0;
  if ((long long)R * (gamma + 1) > kMaxRows) return 0;
  switch (call) {
    case DSPARK_CALL_MARKOV_DRAFT: return markov_ws_bytes(R, V);
    case DSPARK_CALL_VERIFY: return verify_ws_bytes(R, gamma, V);
    case DSPARK_CALL_ANALYTIC_ACCEPT: return accept_ws_bytes(R, gamma, V);
    default: return 0;
  }
}

// Zero-fill, 16 bytes per thread where the buffer allows (a kernel rather than
// a memset, so the call may sit in a captured graph).
__global__ void workspace_zero_kernel(unsigned char* __restrict__ p, size_t n) {
  const size_t n16 = (reinterpret_cast<uintptr_t>(p) % 16) == 0 ? n / 16 : 0;
  uint4* q = reinterpret_cast<uint4*>(p);
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    q[i] = make_uint4(0u, 0u, 0u, 0u);
  for (size_t i = n16 * 16 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    p[i] = 0;
}

int dspark::zero_fill(void* p, size_t n, hipStream_t s) {
  if (n == 0) return DSPARK_OK;
  const size_t per_block = 256 * 16;
  const int grid = (int)std::min<size_t>((n + per_block - 1) / per_block, 4096);
  hipLaunchKernelGGL(workspace_zero_kernel, dim3(grid), dim3(256), 0, s,
                     static_cast<unsigned char*>(p), n);
  return launch_status();
}

extern "C" int dspark_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return DSPARK_EINVAL;
  return zero_fill(ws, ws_bytes, static_cast<hipStream_t>(stream));
}

extern "C" size_t dspark_workspace_status_offset(int R, int V) {
  if (R < 1 || R > kMaxRows || V < 1) return 0;
  return resident_bar_offset(R, V) + kResidentErrByte;  // the resident kernel's error word
}
