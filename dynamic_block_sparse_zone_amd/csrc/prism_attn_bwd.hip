// Sparse attention backward (placeholder until the gfx950 kernels land).
#include "prism_common.h"
#include "prism_kernels.h"

namespace prism {
bool launch_attn_bwd(const PlanDev&, const BwdDev&, const void*, const void*, const float*,
                     const void*, void*, void*, void*, hipStream_t) {
  return false;
}
}  // namespace prism
