// gemm_nv.hip -- NVFP4 GEMM (placeholder until the FP16-decode kernel lands).
#include "fp4_device.h"
#include "fp4_launch.h"

namespace fp4 {

size_t gemm_nv_workspace(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm_nv(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, const float*, const float*,
                          void*, int64_t, int64_t, int64_t, int, void*, size_t, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace fp4
