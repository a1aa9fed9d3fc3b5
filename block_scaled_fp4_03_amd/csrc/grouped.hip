// grouped.hip -- grouped GEMM (placeholder until the grouped kernel lands).
#include "fp4_device.h"
#include "fp4_launch.h"

namespace fp4 {

size_t gemm_grouped_workspace(int64_t, int64_t, int64_t, int32_t) { return 0; }

hipError_t launch_gemm_grouped(const uint8_t*, const uint8_t*, int64_t, const int32_t*, const int32_t*, int32_t,
                               const uint8_t*, const uint8_t*, const float*, const float*, void*, int64_t, int64_t,
                               int64_t, int, int, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace fp4
