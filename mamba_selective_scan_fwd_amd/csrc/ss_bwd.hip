// ss_bwd.hip -- selective-scan backward (placeholder until the kernels land).
#include "ss_device.h"
#include "ss_internal.h"

namespace ss {
hipError_t launch_bwd(const BwdParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ss
