// attn_bwd.hip -- backward pass (placeholder until the kernels land).
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

hipError_t launch_bwd(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace attn
