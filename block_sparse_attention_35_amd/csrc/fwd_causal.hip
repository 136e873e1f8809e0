// Forward kernels of the causal mask family (the rule families of the
// BlockMask kinds; see fwd_kernels.h).
#include "fwd_kernels.h"

namespace bsattn {

hipError_t launch_forward_causal(int32_t dtype, const FwdArgs& a, hipStream_t stream) {
  return launch_family<ATTN_MASK_CAUSAL>(dtype, a, stream);
}

}  // namespace bsattn
