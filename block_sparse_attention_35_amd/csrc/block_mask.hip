// BlockMask construction on the GPU.
//
// A 128x128 block (qb, kb) is classified from the mask rule: no live pair ->
// skipped, every pair live (and the whole block in range) -> full, otherwise
// partial. Rules: "FlexAttention on Apple Silicon: block masks", sections
// "Mask 1: causal", "Mask 2: sliding-window causal", "Mask 3: document-packed";
// only fully masked blocks may be skipped (same page, closing section); 128x128
// blocks: "FlexAttention on MPS vs SDPA", data-flow section.
//
// Causal and sliding-window blocks are classified in closed form: all pair
// offsets d = p - j of a block, p = i + q_off the query position the rule
// sees (q_off = 0, or S - L for the bottom-right kinds), form the integer
// interval [q0 + q_off - k1, q1 + q_off - k0], and a pair is live iff
// 0 <= d < W (W = infinity for causal), so the block is skipped iff the two
// intervals are disjoint and full iff the first lies inside the second. Document blocks whose queries share one id and whose
// keys share one id follow the causal rule (or are skipped when the ids
// differ); the rest are classified exactly by evaluating every in-range pair
// cooperatively (ids may be in any order).
//
// CUSTOM blocks are classified from the bit-packed user mask: a block is
// skipped when none of its in-range bits is set and full when all 128 x 128
// are in range and set.
//
// Kernel 1 (one workgroup per query block) writes the classes to LDS, then
// compacts them in ascending kb order with wave ballots and writes the counts,
// the index lists and the zero padding. Kernel 2 writes the work plan (items
// ranked by cost). For the interval rules one kernel does both.
#include <algorithm>

#include "internal.h"

#include "bsattn.h"

namespace bsattn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

enum : uint8_t { kSkip = 0, kPartial = 1, kFull = 2 };

__device__ inline uint8_t classify_interval(int64_t q0, int64_t q1, int64_t k0, int64_t k1,
                                            int64_t window, bool whole) {
  const int64_t dmin = q0 - k1, dmax = q1 - k0;
  if (dmax < 0 || dmin > window - 1) return kSkip;
  if (dmin >= 0 && dmax <= window - 1 && whole) return kFull;
  return kPartial;
}

// Classes of query block qb's kv blocks into cls (LDS, [nk] bytes), then the
// compacted lists and counts of the block.
__device__ __forceinline__ void classify_block(
    int qb, int32_t kind, int32_t q_off, int32_t window, const int32_t* __restrict__ doc,
    const uint32_t* __restrict__ bits, int32_t q_len, int32_t kv_len,
    int32_t nk, uint8_t* cls, int32_t* __restrict__ kv_num, int32_t* __restrict__ kv_idx,
    int32_t* __restrict__ full_num, int32_t* __restrict__ full_idx) {
  __shared__ __attribute__((aligned(16))) int32_t doc_q[kBlock];
  __shared__ int32_t qd_id[kBlock], qd_last[kBlock];  // distinct query ids, last row of each
  __shared__ int32_t qd_n;
  __shared__ int32_t wave_counts[2][kWaves];

  const int tid = threadIdx.x;
  const int64_t q0 = (int64_t)qb * kBlock;
  const int64_t q1 = min<int64_t>(q_len, q0 + kBlock) - 1;
  const bool q_whole = (q1 - q0 + 1) == kBlock;

  if (kind == ATTN_MASK_DOCUMENT) {
    // Shortcut, exact: when every in-range query of the block has one id and
    // every in-range key of a kv block has one id, a pair is live iff its
    // causal condition holds and the two ids are equal, so the class follows
    // from the causal interval rule (or is skip for different ids). A block
    // that mixes ids can never be full; for those, every in-range pair is
    // evaluated (ids may be in any order). Wave w takes kv blocks w, w + 4,
    // ..., sixteen at a time, each lane two keys of each (coalesced loads,
    // all in flight); the first batch is issued before the query side is
    // prepared, and each block is classified from the keys in registers,
    // with no workgroup barrier per block.
    const int wave = tid >> 6, lane = tid & 63;
    constexpr int kBatch = 16;
    int32_t d0[kBatch], d1[kBatch];  // keys k0 + lane and k0 + 64 + lane of block base + 4u
    auto load_batch = [&](int base) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int kb = base + u * kWaves;
        d0[u] = d1[u] = 0;
        if (kb < nk) {
          // keys past kv_len repeat the block's last key (an in-range id)
          const int64_t k0 = (int64_t)kb * kBlock;
          const int64_t k1 = min<int64_t>(kv_len, k0 + kBlock) - 1;
          d0[u] = doc[min<int64_t>(k0 + lane, k1)];
          d1[u] = doc[min<int64_t>(k0 + 64 + lane, k1)];
        }
      }
    };
    load_batch(wave);
    if (tid < kBlock) doc_q[tid] = (q0 + tid <= q1) ? doc[q0 + tid] : 0;
    __syncthreads();
    const int32_t q_id = doc_q[0];
    const bool q_uniform = __syncthreads_and(tid >= kBlock || q0 + tid > q1 || doc_q[tid] == q_id);
    const int n_rows = (int)(q1 - q0 + 1);
    // The distinct ids of the block's queries, each with its last row: a key
    // with id d at position j has a live pair in the block iff some query
    // row i with id d has j <= i + q_off, i.e. iff j <= (last row of d) +
    // q0 + q_off.
    if (tid == 0) {
      qd_n = q_uniform ? 1 : 0;
      qd_id[0] = q_id;
      qd_last[0] = n_rows - 1;
    }
    __syncthreads();
    if (!q_uniform && tid < n_rows) {
      const int32_t id = doc_q[tid];
      bool last = true;
      // every row, four per LDS read (all threads read the same words)
#pragma unroll 8
      for (int r4 = 0; r4 < kBlock / 4; ++r4) {
        const int4 x = reinterpret_cast<const int4*>(doc_q)[r4];
        const int r = 4 * r4;
        last &= !((r > tid) & (r < n_rows) & (x.x == id));
        last &= !((r + 1 > tid) & (r + 1 < n_rows) & (x.y == id));
        last &= !((r + 2 > tid) & (r + 2 < n_rows) & (x.z == id));
        last &= !((r + 3 > tid) & (r + 3 < n_rows) & (x.w == id));
      }
      if (last) {
        const int at = atomicAdd(&qd_n, 1);
        qd_id[at] = id;
        qd_last[at] = tid;
      }
    }
    __syncthreads();
    const int nd = qd_n;
    for (int base = wave; base < nk; base += kWaves * kBatch) {
      if (base != wave) load_batch(base);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int kb = base + u * kWaves;
        if (kb >= nk) break;  // (wave-uniform)
        const int64_t k0 = (int64_t)kb * kBlock;
        const int64_t k1 = min<int64_t>(kv_len, k0 + kBlock) - 1;
        uint8_t c = kSkip;
        if (q1 + q_off >= k0) {  // else every key comes after every query position
          const int32_t first = __shfl(d0[u], 0);  // key k0
          const bool uni = __all(d0[u] == first && d1[u] == first);
          if (q_uniform && uni) {
            c = (first == q_id) ? classify_interval(q0 + q_off, q1 + q_off, k0, k1, INT64_MAX / 4,
                                                    q_whole && (k1 - k0 + 1) == kBlock)
                                : kSkip;
          } else {
            // any in-range pair (i, j) with j <= i and equal ids, through the
            // distinct query ids (positions stay below 2^31: p < 2^22 + 2^30)
            const int32_t j0 = (int32_t)k0 + lane, j1 = (int32_t)k0 + lane + 64;
            const bool v0 = j0 <= k1, v1 = j1 <= k1;
            const int32_t base_p = (int32_t)q0 + q_off;
            bool any = false;
            for (int x = 0; x < nd; ++x) {
              const int32_t id = qd_id[x], last = base_p + qd_last[x];
              any |= (v0 & (d0[u] == id) & (j0 <= last)) | (v1 & (d1[u] == id) & (j1 <= last));
            }
            c = __any(any) ? kPartial : kSkip;
          }
        }
        if (lane == 0) cls[kb] = c;
      }
    }
  } else if (kind == ATTN_MASK_CUSTOM) {
    // One wave per kv block: lane l holds rows q0 + l and q0 + l + 64 (when
    // in range) and reads each one's four words of the block.
    const int64_t W = 4 * (int64_t)nk;
    const int n_rows = (int)(q1 - q0 + 1);
    const int wave = tid >> 6, lane = tid & 63;
    for (int kb = wave; kb < nk; kb += kWaves) {
      const int nvalid = (int)min<int64_t>(kBlock, kv_len - (int64_t)kb * kBlock);
      uint32_t vm[4];  // in-range keys of each word
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = nvalid - 32 * t;
        vm[t] = n >= 32 ? ~0u : (n <= 0 ? 0u : ((1u << n) - 1u));
      }
      bool any = false, all = nvalid == kBlock;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = lane + 64 * h;
        if (r < n_rows) {
          const uint4 w = *reinterpret_cast<const uint4*>(bits + (q0 + r) * W + 4 * kb);
          any |= ((w.x & vm[0]) | (w.y & vm[1]) | (w.z & vm[2]) | (w.w & vm[3])) != 0u;
          all &= (w.x & w.y & w.z & w.w) == ~0u;
        } else {
          all = false;  // the block is not whole
        }
      }
      any = __any(any);
      all = __all(all);
      if (lane == 0) cls[kb] = !any ? kSkip : (all ? kFull : kPartial);
    }
  } else {
    const int64_t w = (kind == ATTN_MASK_SLIDING_WINDOW) ? (int64_t)window : INT64_MAX / 4;
    for (int kb = tid; kb < nk; kb += kThreads) {
      const int64_t k0 = (int64_t)kb * kBlock;
      const int64_t k1 = min<int64_t>(kv_len, k0 + kBlock) - 1;
      const bool whole = q_whole && (k1 - k0 + 1) == kBlock;
      uint8_t c;
      if (kind == ATTN_MASK_NONE)
        c = whole ? kFull : kPartial;
      else
        c = classify_interval(q0 + q_off, q1 + q_off, k0, k1, w, whole);
      cls[kb] = c;
    }
  }
  __syncthreads();

  // Stable compaction in ascending kb order.
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t base_p = 0, base_f = 0;
  int32_t* prow = kv_idx + (int64_t)qb * nk;
  int32_t* frow = full_idx + (int64_t)qb * nk;
  for (int c0 = 0; c0 < nk; c0 += kThreads) {
    const int kb = c0 + tid;
    const uint8_t c = (kb < nk) ? cls[kb] : kSkip;
    const uint64_t bp = __ballot(c == kPartial);
    const uint64_t bf = __ballot(c == kFull);
    if (lane == 0) {
      wave_counts[0][wave] = __popcll(bp);
      wave_counts[1][wave] = __popcll(bf);
    }
    __syncthreads();
    int32_t off_p = base_p, off_f = base_f, tot_p = 0, tot_f = 0;
    for (int w = 0; w < kWaves; ++w) {
      if (w < wave) {
        off_p += wave_counts[0][w];
        off_f += wave_counts[1][w];
      }
      tot_p += wave_counts[0][w];
      tot_f += wave_counts[1][w];
    }
    if (c == kPartial) prow[off_p + __popcll(bp & lower)] = kb;
    if (c == kFull) frow[off_f + __popcll(bf & lower)] = kb;
    base_p += tot_p;
    base_f += tot_f;
    __syncthreads();  // wave_counts reused next chunk
  }
  for (int t = tid; t < nk; t += kThreads) {
    if (t >= base_p) prow[t] = 0;
    if (t >= base_f) frow[t] = 0;
  }
  if (tid == 0) {
    kv_num[qb] = base_p;
    full_num[qb] = base_f;
  }
}

// Kernel 1 of every rule: one workgroup per query block.
__global__ __launch_bounds__(kThreads) void classify_compact_kernel(
    int32_t kind, int32_t q_off, int32_t window, const int32_t* __restrict__ doc,
    const uint32_t* __restrict__ bits, int32_t q_len, int32_t kv_len,
    int32_t nk, int32_t* __restrict__ kv_num, int32_t* __restrict__ kv_idx,
    int32_t* __restrict__ full_num, int32_t* __restrict__ full_idx) {
  extern __shared__ __attribute__((aligned(16))) uint8_t cls[];  // [nk]
  classify_block(blockIdx.x, kind, q_off, window, doc, bits, q_len, kv_len, nk, cls, kv_num, kv_idx, full_num,
                 full_idx);
}

// Work plan. With max_n the largest number of live kv blocks of any query
// block, the split length is C = max(kMinSplit, ceil(max_n / 2)); a query
// block with n > C blocks becomes two work items, its first C visited blocks
// and the remaining n - C, and other query blocks are one item. Items are
// ranked by decreasing cost (blocks visited), ties by t = 2 qb + chunk. Cutting
// a fixed first chunk (rather than halves) leaves short remainders that fill
// in beside short unsplit rows when the items are run longest first, so a
// causal launch is no longer set by its longest rows (three-way splits were
// measured slower: each extra item pays its own prologue latency and a
// larger merge).
// Each item is stored as a 16-byte descriptor, so the forward fetches all it
// needs to start an item with one scalar load:
//   plan[0] = number of items, plan[1] = C; plan[4 + 4 rank(t) + {0..3}] =
//   {qb | chunk << 20 | (k - 1) << 22, full blocks of qb, partial blocks of
//   qb, index of the item's first visited kv block}; unused entries hold -1.
// Every workgroup recomputes max_n, so the kernel needs no second pass.
constexpr int kMinSplit = kPlanMinSplit;

__device__ inline int32_t split_count(int32_t n, int32_t split_len) { return n <= split_len ? 1 : 2; }

// Blocks visited by chunk `chunk` of a query block with n blocks: [first, end).
__device__ inline int32_t chunk_first(int32_t chunk, int32_t split_len) { return chunk ? split_len : 0; }
__device__ inline int32_t chunk_end(int32_t chunk, int32_t k, int32_t n, int32_t split_len) {
  return (k > 1 && chunk == 0) ? split_len : n;
}

__device__ inline int32_t item_cost(int32_t t, const int32_t* kv_num, const int32_t* full_num,
                                    int32_t split_len) {
  const int32_t qb = t / kMaxChunks, chunk = t % kMaxChunks;
  const int32_t n = kv_num[qb] + full_num[qb];
  const int32_t k = split_count(n, split_len);
  if (chunk >= k) return -1;  // no such item
  return chunk_end(chunk, k, n, split_len) - chunk_first(chunk, split_len);
}

__global__ __launch_bounds__(kThreads) void plan_kernel(int32_t nq, int32_t nk,
                                                        const int32_t* __restrict__ kv_num,
                                                        const int32_t* __restrict__ kv_idx,
                                                        const int32_t* __restrict__ full_num,
                                                        const int32_t* __restrict__ full_idx,
                                                        int32_t* __restrict__ plan) {
  __shared__ int32_t cost_tile[kThreads];
  __shared__ int32_t red[kThreads / 64];
  const int tid = threadIdx.x;
  // max_n over all query blocks
  int32_t mx = 0;
  for (int q = tid; q < nq; q += kThreads) mx = max(mx, kv_num[q] + full_num[q]);
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = red[0];
  for (int w = 1; w < kThreads / 64; ++w) mx = max(mx, red[w]);
  const int32_t split_len = max(kMinSplit, (mx + 1) / 2);

  const int32_t n_items_total = kMaxChunks * nq;
  const int t = blockIdx.x * kThreads + tid;
  const int32_t mine = (t < n_items_total) ? item_cost(t, kv_num, full_num, split_len) : -1;
  int32_t rank = 0, count = 0;
  for (int t0 = 0; t0 < n_items_total; t0 += kThreads) {
    __syncthreads();
    const int u = t0 + tid;
    cost_tile[tid] = (u < n_items_total) ? item_cost(u, kv_num, full_num, split_len) : -1;
    __syncthreads();
    const int lim = min(kThreads, n_items_total - t0);
    for (int v = 0; v < lim; ++v) {
      const int32_t c = cost_tile[v];
      rank += (c > mine) | ((c == mine) & (t0 + v < t));
      count += c >= 0;
    }
  }
  if (t < n_items_total && mine >= 0) {
    const int32_t qb = t / kMaxChunks, chunk = t % kMaxChunks;
    const int32_t nf = full_num[qb], np = kv_num[qb];
    const int32_t k = split_count(nf + np, split_len);
    const int32_t first = chunk_first(chunk, split_len);  // first visited block of the item
    int4 d;
    d.x = qb | (chunk << 20) | ((k - 1) << 22);
    d.y = nf;
    d.z = np;
    d.w = (first < nf) ? full_idx[(int64_t)qb * nk + first]
                       : (first - nf < np ? kv_idx[(int64_t)qb * nk + first - nf] : 0);
    reinterpret_cast<int4*>(plan + 4)[rank] = d;
  }
  if (t < n_items_total && t >= count) reinterpret_cast<int4*>(plan + 4)[t] = make_int4(-1, -1, -1, -1);
  if (t == 0) {
    plan[0] = count;
    plan[1] = split_len;
    plan[2] = plan[3] = 0;
  }
}

// The same plan, ranked in parallel: every workgroup loads all rows' block
// counts into LDS (up to kPlanLdsRows rows) and computes every item's cost
// there; it then ranks 64 items, lane l taking item 64 b + l and each of the
// 4 waves comparing it against a quarter of all costs (broadcast LDS reads,
// four costs per read), and the quarters' counts are summed. Same output as
// plan_kernel.
constexpr int kPlanLdsRows = 4096;
// The one-launch path for the interval rules: up to this many query blocks
// and kv blocks (its plan arrays and classes stay within 64 KiB of LDS).
constexpr int kIntervalMaxRows = 1024;
constexpr int kIntervalMaxKvBlocks = 32768;

__device__ inline int32_t lds_item_cost(int32_t t, const int32_t* nf, const int32_t* np, int32_t split_len) {
  const int32_t qb = t / kMaxChunks, chunk = t % kMaxChunks;
  const int32_t n = nf[qb] + np[qb];
  const int32_t k = split_count(n, split_len);
  if (chunk >= k) return -1;
  return chunk_end(chunk, k, n, split_len) - chunk_first(chunk, split_len);
}

// Ranks items 64 tile .. 64 tile + 63 of the plan from the block counts of
// all nq query blocks in LDS (nf_s, np_s; mx their largest sum) and writes
// their descriptors; first_block(qb, pos) is the kv block at position pos of
// qb's visit order (full blocks, then partial), 0 past its end. Workgroup 0
// also writes the header.
template <class FirstBlock>
__device__ __forceinline__ void rank_tile(int tile, int32_t nq, const int32_t* nf_s, const int32_t* np_s,
                                          int32_t* cost_s, int32_t mx, FirstBlock first_block,
                                          int32_t* __restrict__ plan) {
  __shared__ int32_t red[kWaves];
  __shared__ int32_t part[kWaves][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t split_len = max(kMinSplit, (mx + 1) / 2);
  const int32_t n_items = kMaxChunks * nq;
  const int32_t n_pad = (n_items + 4 * kWaves - 1) / (4 * kWaves) * (4 * kWaves);
  int32_t cnt = 0;
  for (int t = tid; t < n_pad; t += kThreads) {
    const int32_t c = t < n_items ? lds_item_cost(t, nf_s, np_s, split_len) : -1;
    cost_s[t] = c;
    cnt += c >= 0;
  }
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
  if (lane == 0) red[wave] = cnt;
  __syncthreads();
  int32_t count = 0;
  for (int w = 0; w < kWaves; ++w) count += red[w];

  const int32_t t = tile * 64 + lane;  // this lane's item
  const int32_t mine = t < n_items ? cost_s[t] : -1;
  const int32_t span = n_pad / kWaves, u0 = wave * span;
  int32_t rank = 0;
  for (int u = u0; u < u0 + span; u += 4) {
    const int4 c4 = *reinterpret_cast<const int4*>(&cost_s[u]);
    rank += (c4.x > mine) | ((c4.x == mine) & (u < t));
    rank += (c4.y > mine) | ((c4.y == mine) & (u + 1 < t));
    rank += (c4.z > mine) | ((c4.z == mine) & (u + 2 < t));
    rank += (c4.w > mine) | ((c4.w == mine) & (u + 3 < t));
  }
  part[wave][lane] = rank;
  __syncthreads();
  if (wave == 0 && t < n_items) {
    rank = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
    if (mine >= 0) {
      const int32_t qb = t / kMaxChunks, chunk = t % kMaxChunks;
      const int32_t nf = nf_s[qb], np = np_s[qb];
      int4 d;
      d.x = qb | (chunk << 20) | ((split_count(nf + np, split_len) - 1) << 22);
      d.y = nf;
      d.z = np;
      d.w = first_block(qb, chunk_first(chunk, split_len));
      reinterpret_cast<int4*>(plan + 4)[rank] = d;
    }
    if (t >= count) reinterpret_cast<int4*>(plan + 4)[t] = make_int4(-1, -1, -1, -1);
  }
  if (tile == 0 && tid == 0) {
    plan[0] = count;
    plan[1] = split_len;
    plan[2] = plan[3] = 0;
  }
}

// The largest of every workgroup thread's value.
__device__ inline int32_t block_max(int32_t v) {
  __shared__ int32_t red[kWaves];
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = red[0];
  for (int w = 1; w < kWaves; ++w) v = max(v, red[w]);
  return v;
}

__global__ __launch_bounds__(kThreads) void plan_tile_kernel(int32_t nq, int32_t nk,
                                                             const int32_t* __restrict__ kv_num,
                                                             const int32_t* __restrict__ kv_idx,
                                                             const int32_t* __restrict__ full_num,
                                                             const int32_t* __restrict__ full_idx,
                                                             int32_t* __restrict__ plan) {
  __shared__ int32_t nf_s[kPlanLdsRows], np_s[kPlanLdsRows];
  __shared__ __attribute__((aligned(16))) int32_t cost_s[kMaxChunks * kPlanLdsRows];
  int32_t mx = 0;
  for (int q = threadIdx.x; q < nq; q += kThreads) {
    const int32_t f = full_num[q], p = kv_num[q];
    nf_s[q] = f;
    np_s[q] = p;
    mx = max(mx, f + p);
  }
  mx = block_max(mx);  // (its barrier also publishes nf_s, np_s)
  rank_tile(blockIdx.x, nq, nf_s, np_s, cost_s, mx,
            [&](int32_t qb, int32_t pos) {
              const int32_t nf = nf_s[qb], np = np_s[qb];
              return (pos < nf) ? full_idx[(int64_t)qb * nk + pos]
                                : (pos - nf < np ? kv_idx[(int64_t)qb * nk + pos - nf] : 0);
            },
            plan);
}

// Interval rules (none, causal, sliding window, with the query offset of the
// bottom-right kinds): a query block's live kv blocks are one run [lo, lo +
// n), and its full blocks one run [f, f + nf) inside it, because each class
// condition of classify_interval is monotone in kb (k0 and k1 grow with kb,
// so both pair offsets q - k1 and q - k0 shrink). Each bound is the first kb
// where a condition turns true: k0 = 128 kb is linear, and k1 = 128 kb + 127
// except for a last block cut by kv_len, which is checked on its own.
struct Runs {
  int32_t lo, n, f, nf;
};
__device__ inline Runs interval_runs(int32_t kind, int32_t q_off, int32_t window, int32_t q_len, int32_t kv_len,
                                     int32_t nk, int32_t qb) {
  const int64_t q0 = (int64_t)qb * kBlock;
  const int64_t q1 = min<int64_t>(q_len, q0 + kBlock) - 1;
  const bool q_whole = (q1 - q0 + 1) == kBlock;
  const int32_t n_whole = q_whole ? kv_len / kBlock : 0;  // kv blocks with all 128 keys in range
  Runs r;
  if (kind == ATTN_MASK_NONE) {
    r.lo = 0, r.n = nk, r.f = 0, r.nf = n_whole;
    return r;
  }
  const int64_t p0 = q0 + q_off, p1 = q1 + q_off;
  const int64_t w = (kind == ATTN_MASK_SLIDING_WINDOW) ? (int64_t)window : INT64_MAX / 4;
  // first kb with k0 > x, with k0 >= x, and with k1 >= x
  auto k0_gt = [&](int64_t x) { return x < 0 ? 0 : (int32_t)min<int64_t>(nk, x / kBlock + 1); };
  auto k0_ge = [&](int64_t x) { return x <= 0 ? 0 : (int32_t)min<int64_t>(nk, (x + kBlock - 1) / kBlock); };
  auto k1_ge = [&](int64_t x) {
    const int64_t a = x - (kBlock - 1);
    int32_t c = a <= 0 ? 0 : (int32_t)min<int64_t>(nk, (a + kBlock - 1) / kBlock);
    if (c == nk - 1 && (int64_t)kv_len - 1 < x) c = nk;  // the last block, cut by kv_len
    return c;
  };
  r.lo = k1_ge(p0 - w + 1);                 // not skipped: p0 - k1 <= W - 1
  r.n = max(0, k0_gt(p1) - r.lo);           // skipped from the first kb with p1 - k0 < 0
  r.f = k0_ge(p1 - w + 1);                  // full needs p1 - k0 <= W - 1 ...
  const int32_t f_end = min(n_whole, k1_ge(p0 + 1));  // ... and p0 - k1 >= 0, whole blocks
  r.nf = (r.n > 0) ? max(0, f_end - r.f) : 0;
  return r;
}
__device__ inline int32_t interval_block_at(const Runs& r, int32_t pos) {
  if (pos < r.nf) return r.f + pos;
  const int32_t i = pos - r.nf;  // partial index
  if (i >= r.n - r.nf) return 0;
  if (r.nf == 0) return r.lo + i;
  const int32_t before = r.f - r.lo;  // partial blocks before the full run
  return i < before ? r.lo + i : r.f + r.nf + (i - before);
}

// Kernel 1 and the plan in one launch for the interval rules: workgroup qb <
// nq classifies query block qb, and the (2 nq + 63) / 64 workgroups after
// them rank 64 plan items each from the counts of every query block in
// closed form, so no workgroup waits for another. Same output as the two
// kernels.
__global__ __launch_bounds__(kThreads) void interval_mask_kernel(
    int32_t kind, int32_t q_off, int32_t window, int32_t q_len, int32_t kv_len, int32_t nq, int32_t nk,
    int32_t* __restrict__ kv_num, int32_t* __restrict__ kv_idx, int32_t* __restrict__ full_num,
    int32_t* __restrict__ full_idx, int32_t* __restrict__ plan) {
  extern __shared__ __attribute__((aligned(16))) uint8_t cls[];  // [nk]
  __shared__ int32_t nf_s[kIntervalMaxRows], np_s[kIntervalMaxRows];
  __shared__ int32_t lo_s[kIntervalMaxRows], f_s[kIntervalMaxRows];
  __shared__ __attribute__((aligned(16))) int32_t cost_s[kMaxChunks * kIntervalMaxRows];
  if ((int)blockIdx.x < nq) {
    classify_block(blockIdx.x, kind, q_off, window, nullptr, nullptr, q_len, kv_len, nk, cls, kv_num, kv_idx,
                   full_num, full_idx);
    return;
  }
  const int tile = blockIdx.x - nq;
  int32_t mx = 0;
  for (int q = threadIdx.x; q < nq; q += kThreads) {
    const Runs r = interval_runs(kind, q_off, window, q_len, kv_len, nk, q);
    nf_s[q] = r.nf;
    np_s[q] = r.n - r.nf;
    lo_s[q] = r.lo;
    f_s[q] = r.f;
    mx = max(mx, r.n);
  }
  mx = block_max(mx);
  rank_tile(tile, nq, nf_s, np_s, cost_s, mx,
            [&](int32_t qb, int32_t pos) {
              const Runs r{lo_s[qb], nf_s[qb] + np_s[qb], f_s[qb], nf_s[qb]};
              return interval_block_at(r, pos);
            },
            plan);
}

// Dense byte mask -> CUSTOM bits. One wave per (row, 512-key chunk): lane l
// reads byte 64 u + l of the chunk for u = 0..7 (64 consecutive bytes per
// load instruction), and ballot u is words 16 c + 2 u and 16 c + 2 u + 1 of
// the row (bit l of the ballot = key 64 u + l of the chunk).
__global__ __launch_bounds__(kThreads) void pack_mask_kernel(const uint8_t* __restrict__ dense,
                                                             int64_t row_stride, int32_t q_len,
                                                             int32_t kv_len, int32_t W,
                                                             uint32_t* __restrict__ bits) {
  const int lane = threadIdx.x & 63;
  const int64_t chunks = (W + 15) / 16;
  const int64_t tasks = (int64_t)q_len * chunks;
  for (int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); t < tasks;
       t += (int64_t)gridDim.x * kWaves) {
    const int64_t i = t / chunks, c = t % chunks;
    const uint8_t* row = dense + i * row_stride;
    uint8_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t j = c * 512 + 64 * u + lane;
      v[u] = j < kv_len ? row[j] : 0;
    }
    uint64_t mine = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint64_t m = __ballot(v[u] != 0);
      if (lane == u) mine = m;
    }
    const int64_t w0 = c * 16 + 2 * lane;
    if (lane < 8 && w0 < W)
      *reinterpret_cast<uint2*>(bits + i * W + w0) = make_uint2((uint32_t)mine, (uint32_t)(mine >> 32));
  }
}

}  // namespace

hipError_t launch_pack_mask(const uint8_t* dense, int64_t row_stride, int32_t q_len, int32_t kv_len,
                            uint32_t* bits, hipStream_t stream) {
  const int32_t W = 4 * (int32_t)(((int64_t)kv_len + kBlock - 1) / kBlock);
  if (q_len == 0 || W == 0) return hipSuccess;
  const int64_t tasks = (int64_t)q_len * ((W + 15) / 16);
  const int64_t blocks = std::min<int64_t>((tasks + kWaves - 1) / kWaves, 16384);
  hipLaunchKernelGGL(pack_mask_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, dense, row_stride,
                     q_len, kv_len, W, bits);
  return hipGetLastError();
}

hipError_t launch_plan(int32_t nrows, int32_t ncols, const int32_t* part_num, const int32_t* part_idx,
                       const int32_t* full_num, const int32_t* full_idx, int32_t* plan, hipStream_t stream) {
  if (nrows == 0) return hipSuccess;
  if (nrows <= kPlanLdsRows)
    hipLaunchKernelGGL(plan_tile_kernel, dim3((kMaxChunks * nrows + 63) / 64), dim3(kThreads), 0, stream, nrows,
                       ncols, part_num, part_idx, full_num, full_idx, plan);
  else
    hipLaunchKernelGGL(plan_kernel, dim3((kMaxChunks * nrows + kThreads - 1) / kThreads), dim3(kThreads), 0,
                       stream, nrows, ncols, part_num, part_idx, full_num, full_idx, plan);
  return hipGetLastError();
}

hipError_t launch_block_mask(int32_t kind, int32_t q_off, int32_t window, const int32_t* doc,
                             const uint32_t* bits, int32_t q_len, int32_t kv_len, int32_t nq,
                             int32_t nk, int32_t* kv_num, int32_t* kv_idx, int32_t* full_num,
                             int32_t* full_idx, int32_t* schedule, hipStream_t stream) {
  if (nq == 0) return hipSuccess;
  // classes [nk] (bytes)
  const size_t lds = (size_t)((nk + 15) & ~15);
  if ((kind == ATTN_MASK_NONE || kind == ATTN_MASK_CAUSAL || kind == ATTN_MASK_SLIDING_WINDOW) &&
      nq <= kIntervalMaxRows && nk <= kIntervalMaxKvBlocks) {
    hipLaunchKernelGGL(interval_mask_kernel, dim3(nq + (kMaxChunks * nq + 63) / 64), dim3(kThreads), lds, stream,
                       kind, q_off, window, q_len, kv_len, nq, nk, kv_num, kv_idx, full_num, full_idx, schedule);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(classify_compact_kernel, dim3(nq), dim3(kThreads), lds, stream, kind, q_off,
                     window, doc, bits, q_len, kv_len, nk, kv_num, kv_idx, full_num, full_idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_plan(nq, nk, kv_num, kv_idx, full_num, full_idx, schedule, stream);
}

}  // namespace bsattn
