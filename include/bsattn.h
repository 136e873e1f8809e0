/*
 * bsattn.h -- C ABI of the block-sparse fused attention forward for AMD
 * MI355X (gfx950).
 *
 * Two operations make up the path:
 *
 *   attn_build_block_mask  turns a mask rule into a 128x128 BlockMask: for
 *                          every query block, the ascending list of "partial"
 *                          kv blocks (some but not all pairs live; the rule is
 *                          evaluated per element there) and of "full" kv blocks
 *                          (every pair live; no per-element rule), plus the
 *                          order in which the forward visits query blocks.
 *                          Fully masked blocks appear in neither list and are
 *                          never touched. Mask rules: "FlexAttention on Apple
 *                          Silicon: block masks" (dreaming.press), sections
 *                          "Mask 1" to "Mask 3"; 128x128 blocks and block
 *                          skipping: "FlexAttention on MPS vs SDPA" (qiita,
 *                          kiarina), data-flow section.
 *
 *   attn_forward           O = softmax(Q K^T * scale + mask bias [+ score_mod]) V
 *                          and the per-row logsumexp, fused: the L x S score
 *                          table never leaves registers/LDS. Definition: "SDPA
 *                          replaces hand-written attention" (qiita, GeneLab_999),
 *                          section 1, the Attention equation; online softmax
 *                          over tiles: same page, section 2 (only a running max
 *                          and running sum are kept), and "FlashAttention"
 *                          (service-dock), exactness of tiled softmax;
 *                          score_mod soft-cap: block-mask page, section "Bonus".
 *
 * Conventions for every entry point:
 *  - Memory: the caller owns every buffer. Pointers documented as "device"
 *    must be device memory of the current HIP device; the library never
 *    allocates, frees or synchronises, and only enqueues work on `stream`
 *    (a hipStream_t; NULL means the default stream). Results are visible
 *    after the caller synchronises with that stream.
 *  - Errors: every call returns an attn_status. Arguments are validated on
 *    the host before anything is enqueued; on a validation failure nothing is
 *    enqueued and no output is touched. A combination the library has no
 *    kernel for returns ATTN_ERR_UNSUPPORTED; there is no fallback path.
 *    attn_last_error() returns a message for the calling thread's last
 *    failure. No exception or abort crosses this interface.
 *  - Thread safety: calls may be made from several host threads; calls that
 *    write the same BlockMask arrays or outputs concurrently race.
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define ATTN_OK 0
#define ATTN_ERR_INVALID_ARGUMENT (-1) /* a null pointer, bad size, stride or alignment */
#define ATTN_ERR_UNSUPPORTED (-2)      /* valid, but no kernel for it (e.g. head dim != 64) */
#define ATTN_ERR_HIP (-3)              /* the HIP runtime reported an error at launch */
typedef int32_t attn_status;

/* Element types of q, k, v and o. */
#define ATTN_F32 0
#define ATTN_BF16 1
#define ATTN_F16 2

/* Mask rules; each returns "live" for query position i and key position j.
 *   NONE             every pair is live
 *   CAUSAL           i >= j
 *   SLIDING_WINDOW   i >= j && i - j < window   (the window holds `window`
 *                    keys including the query's own position)
 *   DOCUMENT         i >= j && document_id[i] == document_id[j]
 * Positions are absolute and start at 0 for both queries and keys, also
 * when q_len != kv_len (upper-left alignment).
 * Variants:
 *   CAUSAL_LOWER_RIGHT          p >= j, with p = i + (kv_len - q_len)
 *   SLIDING_WINDOW_LOWER_RIGHT  p >= j && p - j < window, same p
 *   DOCUMENT_BIDIRECTIONAL      document_id[i] == document_id[j]
 * The lower-right kinds align the causal triangle to the bottom-right corner
 * (the last query sees every key), the form chunked or cached-key inference
 * needs when q_len != kv_len ("SDPA replaces hand-written attention" (qiita,
 * GeneLab_999), section 4, pitfall 3, causal_lower_right); with q_len >
 * kv_len the first q_len - kv_len rows see no key. DOCUMENT_BIDIRECTIONAL is
 * the block-diagonal document mask without the causal part. */
#define ATTN_MASK_NONE 0
#define ATTN_MASK_CAUSAL 1
#define ATTN_MASK_SLIDING_WINDOW 2
#define ATTN_MASK_DOCUMENT 3
#define ATTN_MASK_CAUSAL_LOWER_RIGHT 4
#define ATTN_MASK_SLIDING_WINDOW_LOWER_RIGHT 5
#define ATTN_MASK_DOCUMENT_BIDIRECTIONAL 6
/* CUSTOM: a user-supplied boolean mask M [q_len][kv_len], live iff M[i][j]
 * (True keeps the pair: the boolean attn_mask convention of "SDPA replaces
 * hand-written attention" (qiita, GeneLab_999), section 4, pitfall 1; the
 * dense form the pages hand to SDPA, "FlexAttention on MPS vs SDPA" (qiita,
 * kiarina), setup notes), held bit-packed on the device: row i is
 * attn_mask_words(kv_len) = 4 * ceil(kv_len / 128) uint32 words, bit b of
 * word w is M[i][32 w + b] (so one 16-byte group of a row covers one 128-key
 * block); bits past kv_len are ignored. Built with
 * attn_build_block_mask_custom, not attn_build_block_mask. */
#define ATTN_MASK_CUSTOM 7

/* score_mod applied to each scaled score s before the mask:
 *   NONE      s
 *   SOFTCAP   softcap * tanh(s / softcap)   */
#define ATTN_SCORE_NONE 0
#define ATTN_SCORE_SOFTCAP 1

/* The only block size: 128 x 128. */
#define ATTN_BLOCK_SIZE 128
/* Largest number of kv blocks per query block the mask builder supports. */
#define ATTN_MAX_KV_BLOCKS 16384

/*
 * A BlockMask. The caller allocates the five int32 device arrays (sizes from
 * attn_num_blocks) and sets the pointers; attn_build_block_mask fills the
 * arrays and every other field. One BlockMask serves every batch and head
 * (the rule does not depend on them) and any number of attn_forward calls.
 *
 *   kv_num_blocks[nq]          number of partial kv blocks of query block qb
 *   kv_indices[nq * nk]        row qb: its partial kv block indices, ascending,
 *                              then 0 up to nk entries
 *   full_kv_num_blocks[nq]     number of full kv blocks of query block qb
 *   full_kv_indices[nq * nk]   row qb: its full kv block indices, ascending,
 *                              then 0 up to nk entries
 *   schedule[4 + 8 * nq]       work plan of the forward: schedule[0] is the
 *                              number of work items, schedule[1] the split
 *                              length C = max(16, ceil(max_n / 2)) (max_n the
 *                              largest number n of live kv blocks of any query
 *                              block), schedule[2..3] are 0, and
 *                              schedule[4 + 4r .. 4r + 7] describes the r-th
 *                              item: {qb | chunk << 20 | (k - 1) << 22, full
 *                              blocks of qb, partial blocks of qb, kv block
 *                              index of the item's first visited block}
 *                              (entries past the last item hold -1). A query
 *                              block with n > C is k = 2 items, chunk 0 its
 *                              first C visited blocks and chunk 1 the rest (in
 *                              the order full blocks then partial blocks);
 *                              others are one item (k = 1). Items are ordered
 *                              by decreasing number of blocks visited, ties by
 *                              2 qb + chunk.
 * with nq = ceil(q_len / 128) and nk = ceil(kv_len / 128). A block is full only
 * if all 128 x 128 of its positions are in range and live, so the blocks at a
 * ragged end are at most partial.
 */
typedef struct attn_block_mask {
  /* set by the caller: device arrays */
  int32_t* kv_num_blocks;
  int32_t* kv_indices;
  int32_t* full_kv_num_blocks;
  int32_t* full_kv_indices;
  int32_t* schedule;
  /* filled by attn_build_block_mask */
  int32_t q_len;
  int32_t kv_len;
  int32_t block_size;
  int32_t num_q_blocks;
  int32_t num_kv_blocks;
  int32_t kind;
  int32_t window;
  const int32_t* document_id; /* device, borrowed: must stay valid while the mask is used */
  const uint32_t* mask_bits;  /* CUSTOM: device bit-packed mask, borrowed likewise */
} attn_block_mask;

/* ceil(len / block_size) for len >= 0 and block_size == 128; -1 otherwise. */
int32_t attn_num_blocks(int32_t len, int32_t block_size);

/*
 * Length in int32 entries of the `schedule` array a BlockMask over q_len
 * queries and kv_len keys needs: 4 + 8 * ceil(q_len / 128) (a 4-entry header
 * and at most two 4-entry item descriptors per query block, as laid out
 * above). The work plan is this library's own: the pages fix only that the
 * kernel's cost should follow the live blocks ("FlexAttention on Apple
 * Silicon: block masks", closing section on block skipping) and that work is
 * spread over parallel units ("Flash Attention 2 and the IO bottleneck",
 * differences between FlashAttention 1 and 2). -1 for a negative length or
 * block_size != 128. kv_len does not change the length; it is taken so the
 * call names the mask's whole shape.
 */
int32_t attn_block_mask_schedule_len(int32_t q_len, int32_t kv_len, int32_t block_size);

/*
 * Build a BlockMask for `kind` over q_len queries and kv_len keys.
 *   window        the two SLIDING_WINDOW kinds: >= 1; ignored (and stored as
 *                 0) otherwise
 *   document_id   the two DOCUMENT kinds: device int32[max(q_len, kv_len)];
 *                 ignored otherwise
 *   block_size    must be 128
 *   bm            host struct with the five array pointers set (non-null
 *                 unless the array has no elements)
 * Errors: INVALID_ARGUMENT for a null bm/array, q_len or kv_len < 0, a bad
 * window, a missing document_id or an unknown kind (CUSTOM included: it has
 * its own builder); UNSUPPORTED for block_size != 128 or more than
 * ATTN_MAX_KV_BLOCKS kv blocks.
 */
attn_status attn_build_block_mask(int32_t kind, int32_t window, const int32_t* document_id,
                                  int32_t q_len, int32_t kv_len, int32_t block_size,
                                  attn_block_mask* bm, void* stream);

/* 32-bit words per row of a bit-packed CUSTOM mask: 4 * ceil(kv_len / 128)
 * for kv_len >= 0; -1 otherwise. */
int32_t attn_mask_words(int32_t kv_len);

/*
 * Pack a dense boolean mask into the CUSTOM bit layout (asynchronous on
 * `stream`).
 *   dense       device bytes, row i at dense + i * row_stride, byte j nonzero
 *               = the pair (i, j) is live (a torch.bool or uint8 tensor)
 *   row_stride  bytes between rows, >= kv_len
 *   bits        device uint32 [q_len * attn_mask_words(kv_len)], 16-byte
 *               aligned, written in full (bits past kv_len are 0)
 * Errors: INVALID_ARGUMENT for null pointers with a non-empty mask, negative
 * sizes, row_stride < kv_len or misaligned bits; HIP for a failed launch.
 */
attn_status attn_pack_mask(const uint8_t* dense, int64_t row_stride, int32_t q_len, int32_t kv_len,
                           uint32_t* bits, void* stream);

/*
 * Build a BlockMask of kind CUSTOM from a bit-packed mask (asynchronous on
 * `stream`). Every 128 x 128 block is classified from its bits: no live
 * in-range pair -> skipped, all 128 x 128 pairs in range and live -> full,
 * else partial ("FlexAttention on Apple Silicon: block masks", closing
 * section: only fully masked blocks can be skipped). The work plan is the
 * same as attn_build_block_mask's.
 *   bits   device uint32 [q_len * attn_mask_words(kv_len)], 16-byte
 *          aligned; stored in
 *          bm->mask_bits and read again by attn_forward, so it must stay
 *          valid and unchanged while the mask is used
 *   q_len, kv_len, block_size, bm  as for attn_build_block_mask
 * Errors: those of attn_build_block_mask, and INVALID_ARGUMENT for null bits
 * with q_len * kv_len > 0 or misaligned bits.
 */
attn_status attn_build_block_mask_custom(const uint32_t* bits, int32_t q_len, int32_t kv_len,
                                         int32_t block_size, attn_block_mask* bm, void* stream);

/*
 * Bytes of device workspace attn_forward needs for this problem (0 when it
 * needs none, and always for ATTN_F32). It depends on dtype, B * H and the
 * mask's block counts nq = num_q_blocks, nk = num_kv_blocks only:
 *   with k = min(64, ceil(1024 / (B * H * nq)), nk / 2) >= 3: split-KV, every
 *     query block's visit list cut into k chunks whose partial results a
 *     second kernel merges: 8192 + nq * k * B * H * 8448 * 4 bytes;
 *   else, with B * H * nq <= 2048: long query blocks split into two work
 *     items; the first to finish leaves its partial result, the other merges
 *     (ticket counters): 8192 + nq * B * H * 8448 * 4 bytes;
 *   else 0.
 * Layout: 8192 bytes of int32 ticket counters, then fp32 partial slots.
 * When the L queries of the H / H_kv query heads sharing a K/V head number
 * at most 32 (decode), the forward instead packs them into one tile per K/V
 * head and cuts the visit list into as many chunks (of 32 * 64 + 64 floats
 * each) as the same area holds, up to its own target; with one chunk it
 * writes the output directly.
 * Errors: INVALID_ARGUMENT for a null bm or bytes, or B, H < 1.
 */
attn_status attn_forward_workspace_size(int32_t dtype, int32_t B, int32_t H,
                                        const attn_block_mask* bm, size_t* bytes);

/*
 * Fused block-sparse attention forward.
 *   q  device [B, H, L, E], k device [B, H, S, E], v device [B, H, S, E],
 *   o  device [B, H, L, E] output, all of element type `dtype`;
 *   q_strides, k_strides, v_strides, o_strides: host int64[4], the element
 *   strides of the four dimensions (batch, head, sequence, head dim), or NULL
 *   for the contiguous layout. The head-dim stride must be 1; base pointers
 *   and the other strides must keep every row 16-byte aligned. The sequence
 *   strides of k and v may be at most 2^24 elements (ATTN_ERR_UNSUPPORTED
 *   otherwise).
 *   lse  device fp32 [B, H, L] contiguous, natural-log logsumexp of each row's
 *        scores after scale, score_mod and mask; may be NULL. It is the log
 *        of the normaliser O is divided by, whose terms are the probabilities
 *        as rounded for the P.V product (relative rounding <= 2^-8 for bf16,
 *        2^-11 for fp16), so it carries that rounding.
 *   q, k, v, o may be NULL only when they have no elements.
 *   bm   a BlockMask built for q_len == L and kv_len == S.
 *   score_mod ATTN_SCORE_NONE or ATTN_SCORE_SOFTCAP (then softcap > 0).
 *   scale  multiplier of q.k (pass 1/sqrt(E) for the usual attention).
 *   workspace  device memory of at least attn_forward_workspace_size bytes,
 *        256-byte aligned, owned by the caller; may be NULL when that size is
 *        0. Its first use must see it zero-filled; every call leaves the
 *        counters at zero again, so it can be reused by later calls of any
 *        shape (each needs it to be large enough). Calls that share a
 *        workspace must not run concurrently.
 * A row whose every key is masked gets O = 0 and lse = -inf.
 * Arithmetic: products in fp32 (MFMA) from the input type, fp32 softmax
 * statistics and accumulation; probabilities are rounded to the input type
 * (round to nearest even) before the P.V product for bf16/fp16; O is rounded
 * to the output type with round to nearest even.
 * Errors: INVALID_ARGUMENT for null pointers, sizes < 0 (B, H >= 1), a mask
 * built for other lengths, bad strides/alignment, a bad score_mod/softcap or
 * a scale that is not finite and > 0, a missing, misaligned or too small
 * workspace; UNSUPPORTED for E != 64 or an unknown dtype; HIP for a failed
 * launch.
 */
attn_status attn_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                         int32_t dtype, int32_t B, int32_t H, int32_t L, int32_t S, int32_t E,
                         const int64_t* q_strides, const int64_t* k_strides,
                         const int64_t* v_strides, const int64_t* o_strides,
                         const attn_block_mask* bm, int32_t score_mod, float softcap, float scale,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_forward for grouped-query attention: H query heads share H_kv K/V
 * heads, H a multiple of H_kv, query head h reading K/V head h / (H / H_kv)
 * (consecutive query heads share one K/V head: "SDPA replaces hand-written
 * attention" (qiita, GeneLab_999), section 5, enable_gqa). k and v are
 * [B, H_kv, S, E]; everything else, including the workspace size (which
 * depends on H, not H_kv), is as for attn_forward, which is this call with
 * H_kv = H.
 * Errors: those of attn_forward, and INVALID_ARGUMENT for H_kv < 1 or H not a
 * multiple of H_kv.
 */
attn_status attn_forward_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                             int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t L, int32_t S,
                             int32_t E, const int64_t* q_strides, const int64_t* k_strides,
                             const int64_t* v_strides, const int64_t* o_strides,
                             const attn_block_mask* bm, int32_t score_mod, float softcap,
                             float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_forward_gqa with key padding: batch entry b keeps only keys
 * key_start[b] <= j < key_end[b], ANDed with the mask rule (the padded keys of
 * a batch take no weight; a row left with no key gets O = 0, lse = -inf).
 * "SDPA replaces hand-written attention" (qiita, GeneLab_999), section 4,
 * pitfall 1 (a boolean mask's True keeps the pair, so padding is dropped) and
 * section 5 (the padding mask ANDed with the causal mask; left padding).
 *   key_start, key_end  device int32[B], or NULL for 0, respectively S;
 *        entries are clamped to [0, S] (and key_end to >= key_start). Read by
 *        the kernels; the caller keeps them valid until the call completes.
 * Blocks of the BlockMask with no kept key are skipped; blocks a padding
 * boundary cuts take the per-element test. Everything else, and the errors,
 * as for attn_forward_gqa (with both pointers NULL it is attn_forward_gqa).
 */
attn_status attn_forward_padded(const void* q, const void* k, const void* v, void* o, float* lse,
                                int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t L,
                                int32_t S, int32_t E, const int64_t* q_strides,
                                const int64_t* k_strides, const int64_t* v_strides,
                                const int64_t* o_strides, const attn_block_mask* bm,
                                int32_t score_mod, float softcap, float scale,
                                const int32_t* key_start, const int32_t* key_end, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * attn_forward_padded without a workspace argument and without any device
 * allocation, for callers that cannot allocate: code recorded under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The split
 * work items' partial results and ticket counters live in a fixed scratch
 * array of 64 MiB that the library holds on each GPU it runs on until the
 * process ends; every call clears the counters first (with a kernel on
 * `stream`, so a captured call clears them on every replay). All other
 * arguments, the results (bit-identical to attn_forward_padded's) and the
 * errors are as for attn_forward_padded, plus UNSUPPORTED when the shape
 * needs more scratch than 64 MiB (attn_forward_workspace_size tells; at most
 * about 69 MB, for bf16/fp16 work with B*H*nq near 2048).
 * Every call on one GPU shares that GPU's scratch: calls that overlap in
 * time on one GPU (on different streams, or from different threads) race
 * and must be serialised by the caller.
 */
attn_status attn_forward_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t L,
                                 int32_t S, int32_t E, const int64_t* q_strides,
                                 const int64_t* k_strides, const int64_t* v_strides,
                                 const int64_t* o_strides, const attn_block_mask* bm,
                                 int32_t score_mod, float softcap, float scale,
                                 const int32_t* key_start, const int32_t* key_end, void* stream);

/*
 * Bytes of device workspace attn_backward needs (always > 0): two fixed 8 KiB
 * regions of ticket counters, D and lse2 (B*H*q_len floats each), the
 * BlockMask transposed ([nk] counts and [nk * nq] indices, twice), the dK/dV
 * work plan (4 + 8 nk ints), and, when there are few work items (B*H_kv*nk
 * <= 2048, resp. B*H*nq <= 2048), fp32 partial slots for the two-way split
 * of long items (nk * 2 * B*H_kv slots of 16384 floats, nq * 2 * B*H slots
 * of 8192 floats); each region 256-byte aligned.
 * Errors: INVALID_ARGUMENT for a null bm or bytes, B, H, H_kv < 1 or H not a
 * multiple of H_kv.
 */
attn_status attn_backward_workspace_size(int32_t B, int32_t H, int32_t H_kv, const attn_block_mask* bm,
                                         size_t* bytes);

/*
 * Backward of attn_forward_padded (fp32 / bf16 / fp16): the gradients dq, dk, dv of
 * sum(dout * o) with respect to q, k and v, the attention matrix recomputed
 * from the forward's logsumexp instead of stored ("Flash Attention 2 and the
 * IO bottleneck" (tcdigital), section on recomputation in backpropagation).
 * With P the forward's probabilities and s' its (soft-capped) scaled scores:
 *   dv_j = sum_i P_ij dout_i;  dS_ij = P_ij (dout_i . v_j - dout_i . o_i) mod'
 *   dq_i = scale sum_j dS_ij k_j;  dk_j = scale sum_i dS_ij q_i
 * with mod' = 1 - (s'/softcap)^2 under the soft-cap (1 otherwise); a K/V head
 * shared by several query heads gets the sum over them. Masked pairs, padded
 * keys and rows without a live key contribute nothing.
 *   q, o, dout, dq  device [B, H, L, E];  k, v, dk, dv  device [B, H_kv, S, E];
 *        all contiguous, 16-byte aligned, element type dtype (ATTN_F32,
 *        ATTN_BF16 or ATTN_F16); dq, dk, dv are written in full.
 *   lse  device fp32 [B, H, L]: the forward's logsumexp for these arguments
 *        (o too must be the forward's output).
 *   bm, score_mod, softcap, scale, key_start, key_end: as for the forward.
 *   workspace  device memory of at least attn_backward_workspace_size bytes,
 *        256-byte aligned, owned by the caller; its first use must see it
 *        zero-filled, and every call leaves its counters at zero, so it can be
 *        reused by later calls of any shape. Calls sharing a workspace must
 *        not run concurrently.
 * Arithmetic: products on MFMA from the input type, P and dS rounded to the
 * input type for their products (kept in fp32 for ATTN_F32), fp32
 * accumulation; deterministic (no
 * atomics on the gradients: the same inputs give the same bits).
 * Errors: INVALID_ARGUMENT as for the forward (null pointers, sizes, a mask
 * built for other lengths, score_mod/softcap/scale, workspace); UNSUPPORTED
 * for an unknown dtype, E != 64, or too many work items; HIP for a
 * failed launch.
 */
attn_status attn_backward(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t L, int32_t S,
                          int32_t E, const attn_block_mask* bm, int32_t score_mod, float softcap,
                          float scale, const int32_t* key_start, const int32_t* key_end,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* attn_status_string(attn_status status);

/* Detail of the calling thread's last failed call ("" if none). The pointer
 * stays valid until the thread's next call into this library. */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H */
