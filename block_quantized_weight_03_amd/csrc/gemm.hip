// Small-M / prefill GEMM (not yet implemented in this revision).
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mnb {
uint64_t gemm_ws_bytes(const Sizes&, int64_t) { return 0; }
hipError_t launch_gemm(const Sizes&, const mnb_plan&, int64_t, const float*, float*, void*,
                       hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace mnb
