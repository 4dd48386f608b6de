// Attention backward (placeholder until the recomputation kernels land).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
hipError_t launch_bwd(const BwdArgs&) { return hipErrorNotSupported; }
}  // namespace fa
