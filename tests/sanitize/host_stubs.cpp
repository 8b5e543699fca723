// Host-only stand-ins for the kernel launchers, for a build of the C ABI's
// validation code under AddressSanitizer and UndefinedBehaviorSanitizer on a
// machine without a GPU.  Every launcher reports hipErrorNoDevice, so a call
// that passes validation returns MXQ_EHIP instead of launching anything.
#include "mxq_kernels.h"

namespace mxq {

hipError_t launch_mxfp8_row(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, uint8_t*,
                            bool, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_mxfp8_tile(int, const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t,
                             uint8_t*, uint8_t*, int64_t, uint8_t*, bool, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_nvfp4_tensor_scale(const uint16_t*, int64_t, int64_t, int64_t, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_nvfp4_row(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, uint8_t*,
                            float*, int, bool, int, uint64_t, uint32_t, uint32_t, hipStream_t, uint32_t*) {
  return hipErrorNoDevice;
}
hipError_t launch_zero_u32(uint32_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_nvfp4_tile16(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, uint8_t*,
                               float*, int, int, uint64_t, uint32_t, uint32_t, uint16_t*, int64_t,
                               uint8_t*, int64_t, uint8_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_nvfp4_col(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, uint8_t*,
                            float*, int, bool, bool, bool, uint32_t, uint64_t, uint32_t, uint32_t,
                            hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_nvfp4_tensor_scale_rht(const uint16_t*, int64_t, int64_t, int64_t, uint32_t, float*,
                                         hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_dq_mxfp8(const uint8_t*, int64_t, const uint8_t*, int64_t, int64_t, bool, bool, int,
                           uint16_t*, int64_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_dq_nvfp4(const uint8_t*, int64_t, const uint8_t*, const float*, int64_t, int64_t,
                           bool, int, bool, uint16_t*, int64_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_swiglu(const uint16_t*, int64_t, int64_t, int64_t, uint16_t*, int64_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_gemm_fp8s(const Fp8sArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gemm(int, bool, const GemmArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gemm_swiglu_q(const GemmArgs&, uint8_t*, int64_t, uint8_t*, float*, bool, hipStream_t) {
  return hipErrorNoDevice;
}
void gemm_set_tile(int) {}

}  // namespace mxq
