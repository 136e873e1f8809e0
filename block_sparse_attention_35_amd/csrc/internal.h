// Internal declarations shared by the host entry points and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace bsattn {

constexpr int kBlock = 128;   // BlockMask granularity and query/key tile size
constexpr int kMaxChunks = 2; // work items a query block may be split into
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
  // Split work items (see the work plan): ticket counters [nq][B*H] and
  // partial results, one slot per (query block, chunk, batch*head).
  int32_t split;
  int32_t* counters;
  float* partials;
};

// Partial result of one split item: the 4 waves' O^T accumulators in
// register order ([wave][32 registers][64 lanes]), then the running max and
// the sum of each of the 128 rows. Slots are [query block][chunk][B*H].
constexpr int64_t kSlotFloats = 4 * 32 * 64 + 2 * kBlock;
// Long query blocks are split only when there are few work items.
constexpr int64_t kSplitMaxItems = 2048;

inline bool use_split(int32_t dtype, int64_t bh, int32_t nq) {
  return dtype != 0 /* ATTN_F32 */ && nq > 0 && bh * nq <= kSplitMaxItems;
}
inline size_t counters_bytes(int64_t bh, int32_t nq) {
  return ((size_t)(bh * nq) * sizeof(int32_t) + 255) & ~(size_t)255;
}
inline size_t workspace_bytes(int32_t dtype, int64_t bh, int32_t nq) {
  if (!use_split(dtype, bh, nq)) return 0;
  return counters_bytes(bh, nq) + (size_t)nq * kMaxChunks * (size_t)bh * kSlotFloats * sizeof(float);
}

// Enqueue the block classification and the query-block schedule.
hipError_t launch_block_mask(int32_t kind, int32_t window, const int32_t* doc, int32_t q_len,
                             int32_t kv_len, int32_t nq, int32_t nk, int32_t* kv_num,
                             int32_t* kv_idx, int32_t* full_num, int32_t* full_idx,
                             int32_t* schedule, hipStream_t stream);

// Enqueue the fused forward. dtype is ATTN_F32 / ATTN_BF16 / ATTN_F16.
hipError_t launch_forward(int32_t dtype, const FwdArgs& a, hipStream_t stream);

}  // namespace bsattn
