// Forward kernels of user-supplied bit-packed masks (the CUSTOM BlockMask
// kind; see fwd_kernels.h).
#include "fwd_kernels.h"

namespace bsattn {

hipError_t launch_forward_custom(int32_t dtype, const FwdArgs& a, hipStream_t stream) {
  return launch_family<ATTN_MASK_CUSTOM>(dtype, a, stream);
}

}  // namespace bsattn
