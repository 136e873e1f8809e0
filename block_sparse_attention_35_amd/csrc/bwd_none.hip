// Backward kernels of the none mask family (see bwd_kernels.h).
#include "bwd_kernels.h"

namespace bsattn {

hipError_t launch_backward_none(int32_t dtype, const BwdArgs& a, hipStream_t stream) {
  return launch_backward_family<ATTN_MASK_NONE>(dtype, a, stream);
}

}  // namespace bsattn
