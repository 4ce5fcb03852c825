// Stand-ins for the device side of the library, linked with api.cpp into the
// host-only sanitizer build of the C ABI. The calls the driver makes all fail
// validation before reaching a launcher, so every launcher reports an error
// and runs nothing; the size queries return fixed sizes.
#include "../../sequence_chunked_exact_amd/csrc/launch.h"

namespace ca {

hipError_t launch_fwd(const Shape&, const void*, const void*, const void*, void*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_bwd(const Shape&, const void*, const void*, const void*, const void*, const float*, const void*,
                      float, float*, float*, float*, float*, size_t, hipStream_t, bool, const NextStats&) {
  return hipErrorNotSupported;
}
hipError_t scratch_address(void**) { return hipErrorNotSupported; }
hipError_t launch_accumulate(float*, const float*, int, int, int, int, int, int, float, hipStream_t) {
  return hipErrorNotSupported;
}
size_t proj_bwd_ws_bytes(const ProjShape&, bool have_wt) { return have_wt ? 2048 : 4096; }
size_t proj_wt_bytes(const ProjShape&) { return 2048; }
hipError_t launch_proj_wt(const ProjShape&, const void*, const void*, const void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_proj_fwd(const ProjShape&, const void*, const void*, const void*, const void*, void*, void*, void*,
                           hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_proj_bwd(const ProjShape&, const void*, const void*, const void*, const void*, const float*,
                           const float*, const float*, float*, float*, float*, float*, void*, hipStream_t,
                           const void*) {
  return hipErrorNotSupported;
}
hipError_t launch_residual_fwd(const ResidualShape&, const void*, const void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_residual_bwd(const ResidualShape&, const float*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
size_t head_ws_bytes(const HeadShape&) { return 4096; }
hipError_t launch_head_transpose(const HeadShape&, const void*, void*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_head_sft(const HeadShape&, const void*, const void*, const void*, const int*, const float*, float,
                           float*, float*, float*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_zero(float*, size_t, hipStream_t) { return hipErrorNotSupported; }

}  // namespace ca
