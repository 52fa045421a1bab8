// Stand-ins for the kernel launchers, for the host-only build of the C ABI layer that the
// sanitizer test runs the argument-validation tests against (tests/test_sanitizers.py).
// Those tests never get past validation to a launch; if one did, the call would fail with
// HBL_ERR_HIP instead of touching a GPU.
#include "hbl_internal.h"

namespace hbl {

hipError_t launch_wquant(const float*, int64_t, int64_t, uint8_t*, float*, double*, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_actquant(const void*, int, int64_t, int64_t, int, const float*, float, int, int, uint8_t*, float*,
                           hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_decode_fused(const void*, int, int64_t, int64_t, int, const float*, float, int, const uint8_t*,
                               const float*, int64_t, uint8_t*, float*, float*, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_gemm(const uint8_t*, const float*, const uint8_t*, const float*, int64_t, int64_t, int64_t, int,
                       int32_t*, float*, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_gemm_swiglu(const uint8_t*, const float*, const uint8_t*, const float*, const float*, int64_t, int64_t,
                              int64_t, int, int, void*, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_gemm_f6f4(const uint8_t*, const float*, const uint8_t*, const float*, int64_t, int64_t, int64_t,
                            int32_t*, float*, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_weights_fp4(const uint8_t*, int64_t, int64_t, uint8_t*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_qkv_quant(const void*, int, int64_t, int64_t, int, uint8_t*, float*, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_qkv_dequant(const uint8_t*, const float*, int64_t, int64_t, int, float*, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_swiglu(const float*, const float*, int64_t, float*, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace hbl
