// The kernel launchers, for the host-side sanitizer build: every call the
// host driver makes must fail its argument checks before a launch, so
// reaching any of these is an error.  Test infrastructure only.
#include <cstdio>
#include <cstdlib>

#include "../../mixed_precision_sharded_amd/csrc/kernels.h"

namespace {
[[noreturn]] void reached(const char* what)
{
    std::fprintf(stderr, "a call reached the launcher %s\n", what);
    std::abort();
}
}  // namespace

namespace mps {
hipError_t launch_grad_norm(const WorkspaceView&, bool, int, int, double*, double, double, float*,
                            hipStream_t) { reached("grad_norm"); }
hipError_t launch_grad_norm_partials(const WorkspaceView&, bool, int, int, const int32_t*,
                                     hipStream_t) { reached("grad_norm_partials"); }
hipError_t launch_clip_coef(const double*, double, double, float*, hipStream_t) { reached("clip"); }
hipError_t launch_adamw_step(const WorkspaceView&, bool, bool, int, const float*, const double*,
                             int32_t*, const HyperParams&, hipStream_t) { reached("adamw_step"); }
hipError_t launch_clipped_step(const WorkspaceView&, bool, bool, int, int, double, double, int, double*,
                               float*, int32_t*, const HyperParams&, hipStream_t) { reached("clipped"); }
hipError_t fused_grid_limit(bool, int*) { reached("fused_grid_limit"); }
hipError_t launch_fused_step(const WorkspaceView&, bool, int, int, double, double, int, double*,
                             float*, int32_t*, const HyperParams&, uint32_t, hipStream_t) { reached("fused"); }
hipError_t launch_fused_status(WorkspaceHeader*, uint32_t*, hipStream_t) { reached("fused_status"); }
hipError_t scratch_address(int, void**) { reached("scratch_address"); }
hipError_t launch_adamw8_step(const WorkspaceView&, const QuantEntry*, bool, int, const float*,
                              const double*, int32_t*, const HyperParams&, hipStream_t) { reached("adamw8"); }
hipError_t launch_adamw8_clipped(const WorkspaceView&, const QuantEntry*, bool, int, int, double,
                                 double, int, double*, float*, int32_t*, const HyperParams&,
                                 hipStream_t) { reached("adamw8_clipped"); }
hipError_t launch_quantize(const float*, int64_t, bool, uint8_t*, uint8_t*, hipStream_t) { reached("quantize"); }
hipError_t launch_dequantize(const uint8_t*, const uint8_t*, int64_t, bool, float*, hipStream_t) { reached("dequantize"); }
}  // namespace mps
