// Internal declarations shared by the host entry points and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace bsattn {

constexpr int kBlock = 128;   // BlockMask granularity and query/key tile size
constexpr int kMaxChunks = 2; // work items a query block may be split into
constexpr int kHeadDim = 64;  // the one head dimension with kernels

// The kernels' form of a mask kind: one of the rule families NONE, CAUSAL,
// SLIDING_WINDOW, DOCUMENT (or CUSTOM, a bit-packed user mask), evaluated at
// the shifted query position
// p = i + q_off. The bottom-right kinds shift by S - L; the bidirectional
// document kind shifts by kNoCausal, so that the causal part j <= p always
// holds (positions stay below 2^22, so p cannot overflow).
constexpr int32_t kNoCausal = 1 << 30;
struct MaskForm {
  int32_t kind;
  int32_t q_off;
};
inline MaskForm mask_form(int32_t kind, int32_t q_len, int32_t kv_len) {
  switch (kind) {
    case 4 /* ATTN_MASK_CAUSAL_LOWER_RIGHT */: return {1, kv_len - q_len};
    case 5 /* ATTN_MASK_SLIDING_WINDOW_LOWER_RIGHT */: return {2, kv_len - q_len};
    case 6 /* ATTN_MASK_DOCUMENT_BIDIRECTIONAL */: return {3, kNoCausal};
    // 7, ATTN_MASK_CUSTOM: its own family (the pair test reads the bits)
    default: return {kind, 0};
  }
}

// Everything the forward kernels need from a BlockMask.
struct MaskView {
  const int32_t* kv_num;
  const int32_t* kv_idx;
  const int32_t* full_num;
  const int32_t* full_idx;
  const int32_t* schedule;
  const int32_t* doc;
  const uint32_t* bits;  // CUSTOM: [L][bits_w] bit-packed mask
  int32_t bits_w;        // words per mask row, 4 * nk
  int32_t nq, nk;
  int32_t kind;   // rule family (MaskForm::kind)
  int32_t window;
  int32_t q_off;  // query position offset (MaskForm::q_off)
};

// Arguments of one forward call, validated on the host.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int32_t B, H, L, S;
  int32_t kv_group;  // query heads per K/V head (GQA); K/V head = h / kv_group
  // Key padding: batch entry b keeps keys [key_start[b], key_end[b]) (device
  // int32 [B], clamped to [0, S]); a null array means 0, respectively S.
  const int32_t* key_start;
  const int32_t* key_end;
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
  // Split-KV (kv_split_count > 0): every query block's visit list is cut into
  // kv_split contiguous chunks, one work item each; the items leave row-major
  // partial results and a second kernel merges them.
  int32_t kv_split;
  // Packed rows (pack_split > 0): the L x G query rows of each K/V head form
  // one 32-row tile; the visit list is cut into pack_split chunks, merged
  // from partial results when there is more than one.
  int32_t pack_split;
  // Chained items (chain > 0): a grid of that many resident workgroups,
  // each walking the plan entries of one batch*head (sliding windows).
  int32_t chain;
  // Plan entries per query block a launch provides workgroups for:
  // kMaxChunks, or 1 when the plan cannot split (plan_never_splits).
  int32_t items_per_qb;
};

// The work plan splits a query block only when it visits more than
// max(kPlanMinSplit, ceil(max_n / 2)) kv blocks, so a plan never splits when
// no query block can visit more than kPlanMinSplit blocks: at most that many
// kv blocks in all, or a sliding window of at most kPlanMinSplit - 1 blocks
// (W <= 1920: its query blocks touch at most 16 kv blocks). Such launches
// need one workgroup per query block instead of kMaxChunks.
constexpr int32_t kPlanMinSplit = 16;
inline bool plan_never_splits(int32_t form_kind, int32_t window, int32_t nk) {
  return nk <= kPlanMinSplit ||
         (form_kind == 2 /* ATTN_MASK_SLIDING_WINDOW */ && window <= (kPlanMinSplit - 1) * kBlock);
}

// Sliding windows with at most this many kv blocks per query block (W <=
// 1920: never split by the plan) run as chained items when there are at
// least kChainMinItems work items; the grid holds kChainSlots workgroups
// (two per compute unit), rounded down to a multiple of B*H.
constexpr int32_t kChainMaxWindow = 15 * kBlock;
constexpr int64_t kChainMinItems = 1024;
constexpr int64_t kChainSlots = 512;
// (The chained kernel copies a first block for every item, block 0 for an
// item without live blocks, so it needs at least one key.)
inline int32_t chain_grid(int32_t dtype, int32_t form_kind, int32_t window, bool padded, int64_t bh, int32_t nq,
                          int32_t kv_len) {
  if (dtype == 0 /* ATTN_F32 */ || form_kind != 2 /* ATTN_MASK_SLIDING_WINDOW */ || padded || kv_len < 1) return 0;
  if (window > kChainMaxWindow || bh * nq < kChainMinItems) return 0;
  const int64_t per_head = bh >= kChainSlots ? 1 : kChainSlots / bh;
  return (int32_t)(bh * (per_head < nq ? per_head : nq));
}

// Partial result of one split item: the 4 waves' O^T accumulators in
// register order ([wave][32 registers][64 lanes]) -- for split-KV items the
// rows' O row-major ([128 rows][64]) -- then the running max and the sum of
// each of the 128 rows. Two-way split items keep one slot per (query block,
// B*H), the partial of whichever chunk finishes first: [query block][B*H];
// split-KV items one per chunk: [query block][chunk][B*H].
constexpr int64_t kSlotFloats = 4 * 32 * 64 + 2 * kBlock;
// Long query blocks are split only when there are few work items.
constexpr int64_t kSplitMaxItems = 2048;

inline bool use_split(int32_t dtype, int64_t bh, int32_t nq) {
  return dtype != 0 /* ATTN_F32 */ && nq > 0 && bh * nq <= kSplitMaxItems;
}
// The ticket counters, [query block][B*H], take a region of fixed size (the
// most a splitting call can use), so the partial results always start at
// the same offset: a workspace shared by calls of different shapes then
// never sees an earlier call's partial results where a later call keeps its
// counters, and every call leaves all counters at zero.
constexpr size_t kCountersBytes = kSplitMaxItems * sizeof(int32_t);
// Split-KV for shapes with few query blocks (decode: a few queries against a
// long key sequence): with B*H*nq items the GPU would idle, so each query
// block's kv blocks are cut into k chunks, k chosen from the shape alone
// (about kKvSplitTarget items, at least two kv blocks per chunk, at most
// kKvSplitMax), when that gives more than the two-way split of the plan.
constexpr int64_t kKvSplitTarget = 512;
constexpr int32_t kKvSplitMax = 64;
inline int32_t kv_split_count(int32_t dtype, int64_t bh, int32_t nq, int32_t nk) {
  if (dtype == 0 /* ATTN_F32 */ || nq <= 0 || bh <= 0) return 0;
  int64_t k = (kKvSplitTarget + bh * nq - 1) / (bh * nq);
  k = k < kKvSplitMax ? k : kKvSplitMax;
  k = k < nk / 2 ? k : nk / 2;
  return k >= 3 ? (int32_t)k : 0;
}
inline size_t workspace_bytes(int32_t dtype, int64_t bh, int32_t nq, int32_t nk) {
  const int32_t ks = kv_split_count(dtype, bh, nq, nk);
  if (ks > 0) return kCountersBytes + (size_t)nq * ks * (size_t)bh * kSlotFloats * sizeof(float);
  if (!use_split(dtype, bh, nq)) return 0;
  return kCountersBytes + (size_t)nq * (size_t)bh * kSlotFloats * sizeof(float);
}

// Packed rows: when the L queries of the G = H / H_kv query heads sharing a
// K/V head number at most kPackRows, one work item per (batch, K/V head,
// chunk) computes them all from one read of the K/V head. The chunk count
// aims at kPackTarget work items (two per CU, the most the kernel's LDS
// allows: each keeps one block of copies in flight per wave, so two
// workgroups per CU double the bytes in flight) with at least two kv blocks
// each, and
// is capped by the partial slots that fit in the workspace the shape asks
// for (the formula above, which does not depend on H_kv or L); with one chunk
// the items write the output directly. Slot: O [32][64] row-major, then the
// rows' maxima [32] and sums [32].
constexpr int kPackRows = 32;
constexpr int64_t kPackSlotFloats = kPackRows * kHeadDim + 2 * kPackRows;
constexpr int64_t kPackTarget = 512;
inline bool use_packed(int32_t dtype, int32_t L, int32_t G) {
  return dtype != 0 /* ATTN_F32 */ && L >= 1 && G >= 1 && (int64_t)L * G <= kPackRows;
}
inline int32_t packed_split_count(int64_t bhk, int32_t nk, size_t ws_bytes) {
  int64_t k = (kPackTarget + bhk - 1) / bhk;
  k = k < kKvSplitMax ? k : kKvSplitMax;
  k = k < nk / 2 ? k : nk / 2;
  const int64_t slots = ws_bytes > kCountersBytes
                            ? (int64_t)((ws_bytes - kCountersBytes) / sizeof(float)) / kPackSlotFloats
                            : 0;
  k = k < slots / bhk ? k : slots / bhk;
  return k >= 2 ? (int32_t)k : 1;
}

// Enqueue the block classification and the query-block schedule.
// kind is the rule family and q_off the query offset (mask_form).
// bits: the CUSTOM kind's bit-packed mask ([q_len][4 nk] words).
hipError_t launch_block_mask(int32_t kind, int32_t q_off, int32_t window, const int32_t* doc,
                             const uint32_t* bits, int32_t q_len, int32_t kv_len, int32_t nq,
                             int32_t nk, int32_t* kv_num, int32_t* kv_idx, int32_t* full_num,
                             int32_t* full_idx, int32_t* schedule, hipStream_t stream);

// Enqueue the packing of a dense byte mask into the CUSTOM bit layout.
hipError_t launch_pack_mask(const uint8_t* dense, int64_t row_stride, int32_t q_len, int32_t kv_len,
                            uint32_t* bits, hipStream_t stream);

// Enqueue the fused forward. dtype is ATTN_F32 / ATTN_BF16 / ATTN_F16.
hipError_t launch_forward(int32_t dtype, const FwdArgs& a, hipStream_t stream);

// Everything the backward kernels take (host-validated; every tensor
// contiguous [B, heads, len, 64]).
struct BwdArgs {
  FwdArgs f;          // q, k, v, o, lse, sizes, strides, mask, scale, soft-cap, padding
  const void* dout;   // [B, H, L, E], q's strides
  void* dq;           // [B, H, L, E], q's strides
  void* dk;           // [B, H_kv, S, E], k's strides
  void* dv;           // [B, H_kv, S, E], v's strides
  float* D;           // [B*H, L]: dO . O
  float* lse2;        // [B*H, L]: lse * log2 e (+inf for rows without a live key)
  int32_t* tq_num;    // [nk]: partial query blocks of kv block kb
  int32_t* tq_idx;    // [nk][nq]: their indices, ascending
  int32_t* tf_num;    // [nk]: full query blocks of kv block kb
  int32_t* tf_idx;    // [nk][nq]
  // Work plan of the dK/dV kernel ([4 + 8 nk], the forward plan's format
  // over kv blocks and their query-block lists); the dQ kernel follows the
  // forward's plan (f.m.schedule). A split item leaves its fp32 partial
  // accumulators, and the later of the two merges (ticket counters).
  int32_t* tplan;
  int32_t split_kv;      // dK/dV items may split (f.split for dQ)
  int32_t* counters_kv;  // [nk][B*H_kv]
  float* part_kv;        // [nk][2][B*H_kv] x kBwdKvSlot
  int32_t* counters_q;   // [nq][B*H]
  float* part_q;         // [nq][2][B*H] x kBwdQSlot
};

// Backward workspace, each region on a 256-byte boundary: the dK/dV and dQ
// ticket counters first, at fixed offsets (kSplitMaxItems int32 each, so a
// workspace shared by calls of different shapes always finds its counters
// where the previous call left them at zero), then D and lse2 ([B*H*L]
// floats each), the transposed BlockMask (tq_num, tf_num [nk]; tq_idx,
// tf_idx [nk*nq]), the dK/dV plan [4 + 8 nk], and, when items may split (at
// most kSplitMaxItems items), the partial slots: dK/dV [nk][2][B*H_kv] of
// kBwdKvSlot floats, dQ [nq][2][B*H] of kBwdQSlot floats (the 4 waves'
// accumulators in register order).
constexpr int64_t kBwdQSlot = 4 * 32 * 64;
constexpr int64_t kBwdKvSlot = 2 * 4 * 32 * 64;
inline size_t bwd_align(size_t n) { return (n + 255) & ~(size_t)255; }
struct BwdLayout {
  size_t counters_kv, counters_q, D, lse2, tq_num, tf_num, tq_idx, tf_idx, tplan, part_kv, part_q, total;
  bool split_kv, split_q;
};
inline BwdLayout bwd_layout(int64_t bh, int64_t bhk, int32_t L, int32_t nq, int32_t nk) {
  BwdLayout w{};
  size_t o = 0;
  auto take = [&](size_t n) { const size_t at = o; o += bwd_align(n); return at; };
  w.counters_kv = take(kCountersBytes);
  w.counters_q = take(kCountersBytes);
  w.D = take((size_t)bh * L * sizeof(float));
  w.lse2 = take((size_t)bh * L * sizeof(float));
  w.tq_num = take((size_t)nk * sizeof(int32_t));
  w.tf_num = take((size_t)nk * sizeof(int32_t));
  w.tq_idx = take((size_t)nk * nq * sizeof(int32_t));
  w.tf_idx = take((size_t)nk * nq * sizeof(int32_t));
  w.tplan = take((size_t)(4 + 8 * (int64_t)nk) * sizeof(int32_t));
  w.split_kv = bhk * nk <= kSplitMaxItems;
  w.split_q = bh * nq <= kSplitMaxItems;
  w.part_kv = take(w.split_kv ? (size_t)nk * 2 * bhk * kBwdKvSlot * sizeof(float) : 0);
  w.part_q = take(w.split_q ? (size_t)nq * 2 * bh * kBwdQSlot * sizeof(float) : 0);
  w.total = o;
  return w;
}
inline size_t bwd_workspace_bytes(int64_t bh, int64_t bhk, int32_t L, int32_t nq, int32_t nk) {
  return bwd_layout(bh, bhk, L, nq, nk).total;
}

// Enqueue the work plan (plan_kernel) over n_rows rows of blocks whose
// partial / full block lists have n_cols columns.
hipError_t launch_plan(int32_t nrows, int32_t ncols, const int32_t* part_num, const int32_t* part_idx,
                       const int32_t* full_num, const int32_t* full_idx, int32_t* plan, hipStream_t stream);

// Enqueue the backward (bf16 / fp16): D and lse2, the transposed BlockMask,
// then the dK/dV and dQ kernels.
hipError_t launch_backward(int32_t dtype, const BwdArgs& a, hipStream_t stream);

}  // namespace bsattn
