// Internal declarations shared by the host entry points and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace bsattn {

constexpr int kBlock = 128;   // BlockMask granularity and query/key tile size
constexpr int kHeadDim = 64;  // the one head dimension with kernels

// Everything the forward kernels need from a BlockMask.
struct MaskView {
  const int32_t* kv_num;
  const int32_t* kv_idx;
  const int32_t* full_num;
  const int32_t* full_idx;
  const int32_t* schedule;
  const int32_t* doc;
  int32_t nq, nk, kind, window;
};

// Arguments of one forward call, validated on the host.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int32_t B, H, L, S;
  // element strides: batch, head, sequence (the head-dim stride is 1)
  int64_t q_sb, q_sh, q_sl;
  int64_t k_sb, k_sh, k_sl;
  int64_t v_sb, v_sh, v_sl;
  int64_t o_sb, o_sh, o_sl;
  MaskView m;
  float scale;
  float softcap;  // > 0 only when the soft-cap score_mod is on
};

// Enqueue the block classification and the query-block schedule.
hipError_t launch_block_mask(int32_t kind, int32_t window, const int32_t* doc, int32_t q_len,
                             int32_t kv_len, int32_t nq, int32_t nk, int32_t* kv_num,
                             int32_t* kv_idx, int32_t* full_num, int32_t* full_idx,
                             int32_t* schedule, hipStream_t stream);

// Enqueue the fused forward. dtype is ATTN_F32 / ATTN_BF16 / ATTN_F16.
hipError_t launch_forward(int32_t dtype, const FwdArgs& a, hipStream_t stream);

}  // namespace bsattn
