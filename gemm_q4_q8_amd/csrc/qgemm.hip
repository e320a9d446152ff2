// Prefill GEMM (in progress).
#include "q4q8_dev.h"
#include "q4q8_internal.h"

namespace q4q8 {
hipError_t launch_qgemm(int, int, int, const void*, int64_t, int64_t, const void*, int64_t, int64_t, void*, int64_t,
                        hipStream_t, const LaunchEvents&) {
  return hipErrorNotSupported;
}
}  // namespace q4q8
