// C ABI utilities: status strings and workspace sizing.
#include "dspark_host.hpp"

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
    default: return 0;
  }
}
