// Mixture-of-experts path (in progress).
#include "q4q8_dev.h"
#include "q4q8_internal.h"

namespace q4q8 {
hipError_t launch_moe_route(const float*, int, int, int, int32_t*, float*, int32_t*, int32_t*, int32_t*, hipStream_t) {
  return hipErrorNotSupported;
}
size_t moe_workspace_bytes(int, int, int, int, int, int) { return 256; }
hipError_t launch_moe_qgemm(int, int, const void*, const void*, const void*, int, int, int, const void*, int, int,
                            const float*, const int32_t*, const int32_t*, float*, void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace q4q8
