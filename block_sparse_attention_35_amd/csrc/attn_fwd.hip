// Forward dispatch over the mask families; the kernels are instantiated in
// fwd_none.hip, fwd_causal.hip, fwd_sliding.hip, fwd_document.hip and
// fwd_custom.hip.
#include "bsattn.h"
#include "internal.h"

namespace bsattn {

hipError_t launch_forward_none(int32_t dtype, const FwdArgs& a, hipStream_t stream);
hipError_t launch_forward_causal(int32_t dtype, const FwdArgs& a, hipStream_t stream);
hipError_t launch_forward_sliding(int32_t dtype, const FwdArgs& a, hipStream_t stream);
hipError_t launch_forward_document(int32_t dtype, const FwdArgs& a, hipStream_t stream);
hipError_t launch_forward_custom(int32_t dtype, const FwdArgs& a, hipStream_t stream);

hipError_t launch_forward(int32_t dtype, const FwdArgs& a, hipStream_t stream) {
  if ((int64_t)a.B * a.H * a.m.nq == 0) return hipSuccess;
  switch (a.m.kind) {
    case ATTN_MASK_NONE: return launch_forward_none(dtype, a, stream);
    case ATTN_MASK_CAUSAL: return launch_forward_causal(dtype, a, stream);
    case ATTN_MASK_SLIDING_WINDOW: return launch_forward_sliding(dtype, a, stream);
    case ATTN_MASK_DOCUMENT: return launch_forward_document(dtype, a, stream);
    case ATTN_MASK_CUSTOM: return launch_forward_custom(dtype, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bsattn
