// INT3 QMoE (not yet implemented in this revision).
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mnb {
uint64_t qmoe_ws_bytes(const Sizes&, const Sizes&, int, int64_t) { return 0; }
hipError_t launch_qmoe(const Sizes&, const mnb_plan&, const Sizes&, const mnb_plan&, int, int64_t,
                       const uint16_t*, const float*, uint16_t*, void*, hipStream_t,
                       const QmoeDebug*) {
  return hipErrorNotSupported;
}
}  // namespace mnb
