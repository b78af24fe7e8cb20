// grouped_gemm.hip -- grouped GEMM kernels (in progress).
#include "pqm_device.hpp"
#include "pqm_internal.hpp"

namespace pqm {
hipError_t launch_grouped_gemm(int, int, const void *, const uint8_t *, const float *,
                               const void *, const uint8_t *, const float *, int64_t,
                               const int64_t *, int64_t, int64_t, int64_t, int64_t, void *,
                               int, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace pqm
