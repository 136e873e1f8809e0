// Backward kernels of the sliding mask family (see bwd_kernels.h).
#include "bwd_kernels.h"

namespace bsattn {

hipError_t launch_backward_sliding(int32_t dtype, const BwdArgs& a, hipStream_t stream) {
  return launch_backward_family<ATTN_MASK_SLIDING_WINDOW>(dtype, a, stream);
}

}  // namespace bsattn
