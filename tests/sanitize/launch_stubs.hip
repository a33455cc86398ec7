// launch_stubs.hip -- test infrastructure for the host-sanitizer build of the
// planner and argument validation (tests/test_host_sanitizers.py): the kernel
// launch functions the library's host code calls, without any kernel.  Every
// one reports a launch failure; the sanitizer driver only exercises paths that
// return before a launch (argument validation, dg_select_config).
#include "../../moe_grouped_gemm_x128_amd/csrc/dg_kernel.h"

namespace dg {

hipError_t launch(int, const TileShape&, const Params&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_splitk_reduce(int, const Params&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_swiglu_quantize(const uint16_t*, uint8_t*, float*, int, int, int, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_quantize(int, const float*, uint8_t*, float*, int, int, int, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace dg
