// Backward dispatch: D and the logsumexp in log2 units, the transposed
// BlockMask and its work plan, then the dK/dV and dQ kernels of the mask family (instantiated
// in bwd_none.hip, bwd_causal.hip, bwd_sliding.hip, bwd_document.hip and
// bwd_custom.hip).
#include "bwd_kernels.h"

namespace bsattn {

hipError_t launch_backward_none(int32_t dtype, const BwdArgs& a, hipStream_t stream);
hipError_t launch_backward_causal(int32_t dtype, const BwdArgs& a, hipStream_t stream);
hipError_t launch_backward_sliding(int32_t dtype, const BwdArgs& a, hipStream_t stream);
hipError_t launch_backward_document(int32_t dtype, const BwdArgs& a, hipStream_t stream);
hipError_t launch_backward_custom(int32_t dtype, const BwdArgs& a, hipStream_t stream);

hipError_t launch_backward(int32_t dtype, const BwdArgs& a, hipStream_t stream) {
  const dim3 block(kThreads);
  const int64_t rows = (int64_t)a.f.B * a.f.H * a.f.L;
  // D and lse2 (one workgroup per 32 rows) and the transposed BlockMask (one
  // per kv block) in one launch.
  const int64_t blocks = (int64_t)a.f.m.nk + (rows + kThreads / 8 - 1) / (kThreads / 8);
  if (blocks > 0) {
    const dim3 grid((unsigned)blocks);
    if (dtype == ATTN_BF16)
      hipLaunchKernelGGL(bwd_prep_transpose_kernel<__bf16>, grid, block, 0, stream, a);
    else if (dtype == ATTN_F16)
      hipLaunchKernelGGL(bwd_prep_transpose_kernel<_Float16>, grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL(bwd_prep_transpose_kernel<float>, grid, block, 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the dK/dV work plan over kv blocks and their query-block lists
  e = launch_plan(a.f.m.nk, a.f.m.nq, a.tq_num, a.tq_idx, a.tf_num, a.tf_idx, a.tplan, stream);
  if (e != hipSuccess) return e;
  switch (a.f.m.kind) {
    case ATTN_MASK_NONE: return launch_backward_none(dtype, a, stream);
    case ATTN_MASK_CAUSAL: return launch_backward_causal(dtype, a, stream);
    case ATTN_MASK_SLIDING_WINDOW: return launch_backward_sliding(dtype, a, stream);
    case ATTN_MASK_DOCUMENT: return launch_backward_document(dtype, a, stream);
    case ATTN_MASK_CUSTOM: return launch_backward_custom(dtype, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bsattn
