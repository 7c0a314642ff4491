// Two-stage PISA selection (placeholder until the stage kernels land).
#include "pisa_launch.h"

namespace pisa {

bool select_two_stage_supported(const LaunchShape&) { return false; }
size_t select_two_stage_ws_bytes(const LaunchShape&) { return 0; }
hipError_t launch_select_two_stage(const LaunchShape&, const void*, const void*, const float*,
                                   int32_t*, float*, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace pisa
