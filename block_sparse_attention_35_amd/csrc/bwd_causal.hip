// Backward kernels of the causal mask family (see bwd_kernels.h).
#include "bwd_kernels.h"

namespace bsattn {

hipError_t launch_backward_causal(int32_t dtype, const BwdArgs& a, hipStream_t stream) {
  return launch_backward_family<ATTN_MASK_CAUSAL>(dtype, a, stream);
}

}  // namespace bsattn
