// ssm_bwd.hip -- fused reverse-mode pass (placeholder until the kernels land).
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {
bool bwd_variant_exists(const BwdKey&) { return false; }
hipError_t launch_bwd(const BwdKey&, const BwdParams&, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace ssm
