// Pipelined MFMA kernels for aligned fp16/bf16 problems (not built yet).
#include "gemm_internal.h"

namespace dgr {
hipError_t launch_mfma16(const Config&, const LaunchArgs&) { return hipErrorNotSupported; }
}  // namespace dgr
