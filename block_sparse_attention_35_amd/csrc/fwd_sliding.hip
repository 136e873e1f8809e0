// Forward kernels of the sliding mask family (the rule families of the
// BlockMask kinds; see fwd_kernels.h).
#include "fwd_kernels.h"

namespace bsattn {

hipError_t launch_forward_sliding(int32_t dtype, const FwdArgs& a, hipStream_t stream) {
  return launch_family<ATTN_MASK_SLIDING_WINDOW>(dtype, a, stream);
}

}  // namespace bsattn
