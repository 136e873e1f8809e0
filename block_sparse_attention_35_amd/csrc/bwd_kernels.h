// Block-sparse attention backward for gfx950: dQ, dK, dV of sum(dO * O)
// with the attention matrix recomputed from the saved logsumexp instead of
// stored ("Flash Attention 2 and the IO bottleneck" (tcdigital), section on
// recomputation in backpropagation). With P = exp(s' - lse) for the masked,
// scaled (and soft-capped) scores s' of the forward:
//   dV_j = sum_i P_ij dO_i,  dP_ij = dO_i . v_j,  D_i = dO_i . O_i,
//   dS_ij = P_ij (dP_ij - D_i) mod'_ij,  dQ_i = scale sum_j dS_ij k_j,
//   dK_j = scale sum_i dS_ij q_i,
// mod' = 1 - (s'/c)^2 with the soft-cap (1 without). D uses the forward's
// output O (sum_j P_ij dP_ij = dO_i . O_i).
//
// Two kernels, no floating-point atomics (deterministic; one integer ticket
// per split item): dK/dV per (batch, K/V head, kv
// block), looping over the query heads that share the K/V head and over the
// query blocks that see the kv block (the BlockMask transposed); dQ per
// (batch, query head, query block), over the kv blocks the forward visits.
// Both skip dead blocks, run full blocks without a per-pair test and test
// every pair of a partial block. Products on v_mfma_f32_32x32x16 from the
// input type, P and dS rounded to the input type for their products, fp32
// accumulation.
//
// Layouts (each wave owns 32 rows of the item's fixed block, as in the
// forward; the permuted-contraction trick is the forward's):
//  * dK/dV: S = Q K^T and dP = dO V^T with queries along M (Q and dO rows
//    read from LDS) and the wave's 32 keys along N (K and V rows held in
//    registers), so each lane holds one key. P and dS in that accumulator
//    layout are the B operands of dV^T += dO^T P and dK^T += Q^T dS, whose A
//    operands are transposed LDS reads of the dO and Q tiles.
//  * dQ: S^T = K Q^T and dP^T = V dO^T with the wave's 32 queries along N
//    (Q and dO rows in registers), so each lane holds one query; dS^T is the
//    B operand of dQ^T += K^T dS^T, whose A operand is a transposed LDS read
//    of the K tile.
#pragma once

#include "fwd_kernels.h"

namespace bsattn {

namespace {

// A-operand rows of a K-swizzled tile (slot c ^ (r & 7)): row lq, head dims
// 16c + 8hf .. +7 (16-byte chunk 2c + hf); rows 32t + lq add t * 4096.
__device__ inline lds_u8 plain_k(lds_u8 tile, int lane, int c) {
  const int lq = lane & 31, hf = lane >> 5;
  return tile + lq * 128 + (((2 * c + hf) ^ (lq & 7)) << 4);
}

// Tiles read both plain and transposed use one swizzle: 16-byte chunk c of
// row r sits in slot c ^ u(r), u(r) = 4 ((r >> 1) & 1) | ((r >> 2) & 3). With
// 64 banks of 4 bytes, a 16-byte slot of row r lands in bank group
// (8 r + slot) mod 16, so (a) the plain reads of 16 consecutive rows (one
// chunk each) hit 16 distinct groups: u takes 8 distinct values over the even
// rows and over the odd rows; (b) a transposed read of 4 aligned rows x up to
// 4 consecutive chunks does too: rows r and r + 2 differ in bit 2 of u, so
// their chunk sets are disjoint, and odd rows use the other half of the
// groups. u depends on row bits 1..3 only, so 32-row tiles and 16-row groups
// keep the pattern.
__device__ inline int uswz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
__device__ inline lds_u8 plain_u(lds_u8 tile, int lane, int c) {
  const int lq = lane & 31, hf = lane >> 5;
  return tile + lq * 128 + (((2 * c + hf) ^ uswz(lq)) << 4);
}
// Transposed-read addresses (the forward's V-operand layout, see LanePtrs)
// of the first (rows r1) and
// second (rows r1 + 8) read of head-dim tile te in a u-swizzled tile.
__device__ inline lds_u8 tr_u(lds_u8 tile, int lane, int te, int second) {
  const int hf = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
  const int r1 = hf * 4 + (i16 >> 2) + 8 * second;
  const int e = te * 32 + (g16 & 1) * 16 + (i16 & 3) * 4;
  const int c16 = e >> 3, half = (e >> 2) & 1;
  return tile + r1 * 128 + ((c16 ^ uswz(r1)) << 4) + half * 8;
}
// Per-lane byte offsets of the u-swizzled tile copies: lane l fills slot
// l & 7 of row l / 8 of an 8-row copy; copies 0 and 2 (rows with bit 3
// clear) and 1 and 3 (bit 3 set) need different chunks.
__device__ inline uint32_t u_off(int64_t sl_bytes, int lane, int odd) {
  const int r = (lane >> 3) + 8 * odd;
  return (uint32_t)((lane >> 3) * sl_bytes) + (uint32_t)(((lane & 7) ^ uswz(r)) * 16);
}
// One wave's share (rows 32 wave .. +31) of a u-swizzled 128-row tile copy
// from rows row0 .. of g (rows past n clamp to n - 1).
template <typename T>
__device__ inline void issue_rows_u(const T* g, int64_t sl, uint32_t off_even, uint32_t off_odd, int row0, int n,
                                    uint8_t* tile, int wave, int lane) {
  const int r0 = row0 + wave * 32;
  const uint32_t lds0 = lds_offset(tile) + (uint32_t)wave * 4096u;
  if (row0 + kBlock <= n) {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(g + (int64_t)r0 * sl);
    const int64_t step = sl * (int64_t)(8 * sizeof(T));
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_copy16_base(base + i * step, (i & 1) ? off_odd : off_even, lds0 + 1024u * i);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rt = wave * 32 + 8 * i + (lane >> 3);  // row in the tile
      const int row = min(r0 + 8 * i + (lane >> 3), n - 1);
      lds_copy16(g + (int64_t)row * sl + ((lane & 7) ^ uswz(rt)) * 8, lds0 + 1024u * i);
    }
  }
}
template <typename T>
__device__ inline typename Vec<T>::x8 read_tr2(lds_u8 lo_p, lds_u8 hi_p) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lo_p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)hi_p);
  const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(typename Vec<T>::x8, both);
}

template <typename T>
__device__ inline typename Vec<T>::x8 read16(lds_u8 p) {
  typedef __attribute__((address_space(3))) const typename Vec<T>::x8 lds_x8;
  return *reinterpret_cast<const lds_x8*>(p);
}

// Liveness of pair (query i, key j) in a partial block: the forward's rule,
// the kept key range [klo, khi) and, for CUSTOM, the pair's bit.
template <int KIND>
__device__ inline bool bwd_live(const FwdArgs& a, int i, int j, int klo, int khi, int32_t di, int32_t dj,
                                uint32_t word, int bit) {
  bool ok = (i < a.L) & (j >= klo) & pair_live<KIND>(i + a.m.q_off, j, khi, a.m.window, di, dj);
  if (KIND == ATTN_MASK_CUSTOM) ok &= (word >> bit) & 1u;
  return ok;
}

// P and the factor of dS from a raw score x = q.k: returns P, sets mod' (the
// soft-cap derivative, 1 without it).
template <bool SOFTCAP>
__device__ inline float bwd_prob(float x, float lse2, const FwdArgs& a, float& dmod) {
  if (SOFTCAP) {
    const float cap2 = a.softcap * kLog2e;
    const float y2 = softcap_log2(x, 2.0f * kLog2e * a.scale / a.softcap, cap2);  // s' log2 e
    const float t = y2 / cap2;                                                   // tanh
    dmod = 1.0f - t * t;
    return fast_exp2(y2 - lse2);
  }
  dmod = 1.0f;
  return fast_exp2(fmaf(x, a.scale * kLog2e, -lse2));
}

// ---------------------------------------------------------------------------
// D = dO . O and the logsumexp in log2 units, one row per 8 threads.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void bwd_prep(const BwdArgs& a, int block) {
  const int64_t rows = (int64_t)a.f.B * a.f.H * a.f.L;
  const int64_t row = (int64_t)block * (kThreads / 8) + threadIdx.x / 8;
  const int part = threadIdx.x % 8;
  float acc = 0.0f;
  if (row < rows) {
    if constexpr (std::is_same_v<T, float>) {
      const float4* o = static_cast<const float4*>(a.f.o) + row * 16 + part * 2;
      const float4* d = static_cast<const float4*>(a.dout) + row * 16 + part * 2;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float4 ov = o[u], dv = d[u];
        acc = fmaf(ov.x, dv.x, acc);
        acc = fmaf(ov.y, dv.y, acc);
        acc = fmaf(ov.z, dv.z, acc);
        acc = fmaf(ov.w, dv.w, acc);
      }
    } else {
      const auto* o = static_cast<const typename Vec<T>::x8*>(a.f.o) + row * 8 + part;
      const auto* d = static_cast<const typename Vec<T>::x8*>(a.dout) + row * 8 + part;
      const typename Vec<T>::x8 ov = *o, dv = *d;
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = fmaf((float)ov[u], (float)dv[u], acc);
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < rows && part == 0) {
    a.D[row] = acc;
    const float l = a.f.lse[row];
    a.lse2[row] = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// The BlockMask transposed: for kv block kb, its partial and full query
// blocks in ascending order (one workgroup per kv block; binary search in
// each query block's ascending lists, then a ballot compaction).
// ---------------------------------------------------------------------------
__device__ inline bool sorted_has(const int32_t* row, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (row[mid] < x)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo < n && row[lo] == x;
}

__device__ __forceinline__ void bwd_transpose(const BwdArgs& a, int kb) {
  __shared__ int32_t wave_counts[2][kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nq = a.f.m.nq, nk = a.f.m.nk;
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t base_p = 0, base_f = 0;
  for (int c0 = 0; c0 < nq; c0 += kThreads) {
    const int qb = c0 + tid;
    bool part = false, full = false;
    if (qb < nq) {
      full = sorted_has(a.f.m.full_idx + (int64_t)qb * nk, a.f.m.full_num[qb], kb);
      part = !full && sorted_has(a.f.m.kv_idx + (int64_t)qb * nk, a.f.m.kv_num[qb], kb);
    }
    const uint64_t bp = __ballot(part), bf = __ballot(full);
    if (lane == 0) {
      wave_counts[0][wave] = __popcll(bp);
      wave_counts[1][wave] = __popcll(bf);
    }
    __syncthreads();
    int32_t off_p = base_p, off_f = base_f, tot_p = 0, tot_f = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      if (w < wave) {
        off_p += wave_counts[0][w];
        off_f += wave_counts[1][w];
      }
      tot_p += wave_counts[0][w];
      tot_f += wave_counts[1][w];
    }
    if (part) a.tq_idx[(int64_t)kb * nq + off_p + __popcll(bp & lower)] = qb;
    if (full) a.tf_idx[(int64_t)kb * nq + off_f + __popcll(bf & lower)] = qb;
    base_p += tot_p;
    base_f += tot_f;
    __syncthreads();
  }
  if (tid == 0) {
    a.tq_num[kb] = base_p;
    a.tf_num[kb] = base_f;
  }
}

// Both in one launch (they are independent): workgroups 0 .. nk - 1
// transpose, the rest compute D and lse2.
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_prep_transpose_kernel(BwdArgs a) {
  if ((int)blockIdx.x < a.f.m.nk)
    bwd_transpose(a, blockIdx.x);
  else
    bwd_prep<T>(a, blockIdx.x - a.f.m.nk);
}

// Two-way split items: each chunk takes a ticket when it finishes; the first
// leaves its fp32 accumulators (N tiles of 16 registers, register order
// [wave][tile*16 + r][lane]) in its slot with device-scope stores and, once
// they have completed, marks the slot written; the second waits for the mark,
// adds the other chunk's partial (two terms: the sum does not depend on which
// finished first) and resets the counter for the next call. Counter: tickets
// 0 -> 1 -> 2 (or 3 -> 4), the mark adds 2: 4 = both finished and the partial
// written. The second chunk waits only on a chunk that has taken its ticket
// and writes without waiting on anything. Returns false in the chunk that
// exits.
template <int N>
__device__ inline bool merge_two(f32x16_t (&acc)[N], float* mine, float* other, int32_t* counter, int wave,
                                 int lane) {
  auto put = [](float* p, float x) { __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  auto get = [](float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  __shared__ int ticket;
  if (threadIdx.x == 0) ticket = atomicAdd(counter, 1);
  __syncthreads();
  if (ticket == 0) {
#pragma unroll
    for (int t = 0; t < N; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) put(mine + ((wave * N + t) * 16 + r) * 64 + lane, acc[t][r]);
    wait_vm_zero();
    __syncthreads();
    if (threadIdx.x == 0) atomicAdd(counter, 2);
    return false;
  }
  if (threadIdx.x == 0) {
    // A ticket of 3 already includes the mark. Otherwise wait for it
    // (bounded: the first chunk marks its partial within microseconds).
    if (ticket != 3)
      for (int spin = 0; spin < (1 << 24); ++spin) {
        if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 4) break;
        __builtin_amdgcn_s_sleep(1);
      }
    __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < N; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] += get(other + ((wave * N + t) * 16 + r) * 64 + lane);
  return true;
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
// One stage of the query side: Q and dO tiles (V-swizzled), the rows' lse2
// and D, their document ids and, for CUSTOM, word 4 kb + w of each row for
// wave w.
struct alignas(16) BwdQStage {
  uint8_t q[kBlock * 128];
  uint8_t dout[kBlock * 128];
  float lse2[kBlock];
  float D[kBlock];
  int32_t doc[kBlock];
  uint32_t bits[4][kBlock];
};

template <typename T, int KIND, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv_kernel(BwdArgs a) {
  using V = Vec<T>;
  using x8 = typename V::x8;
  using x4 = typename V::x4;
  __shared__ BwdQStage st[2];
  const FwdArgs& f = a.f;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, hf = lane >> 5;
  const int G = f.kv_group, Hk = f.H / G, BHk = f.B * Hk;
  // Item from the dK/dV plan (the forward plan's format over kv blocks):
  // kv block kb, chunk `chunk` of k; up to two items per kv block.
  const i32x4_t desc = ((const_i32x4_ptr)(a.tplan + 4))[blockIdx.x / BHk];
  if (desc[0] < 0) return;
  const int kb = desc[0] & 0xFFFFF, chunk = (desc[0] >> 20) & 3;
  const bool split = a.split_kv && ((desc[0] >> 22) & 3) > 0;
  if (chunk > 0 && !split) return;
  const int bk = blockIdx.x % BHk;
  const int b = bk / Hk, hk = bk % Hk;
  const int kv0 = kb * kBlock;
  const int key = kv0 + wave * 32 + lq;  // this lane's key
  int klo = 0, khi = f.S;
  if (f.key_start != nullptr) klo = min(max(((const_i32_ptr)f.key_start)[b], 0), f.S);
  if (f.key_end != nullptr) khi = max(min(((const_i32_ptr)f.key_end)[b], f.S), klo);

  // This lane's K and V rows as B operands (head dims 16c + 8hf .. +7).
  const T* kg = static_cast<const T*>(f.k) + b * f.k_sb + hk * f.k_sh;
  const T* vg = static_cast<const T*>(f.v) + b * f.v_sb + hk * f.v_sh;
  x8 kreg[4], vreg[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    kreg[c] = key < f.S ? *reinterpret_cast<const x8*>(kg + (int64_t)key * f.k_sl + c * 16 + hf * 8) : x8{};
    vreg[c] = key < f.S ? *reinterpret_cast<const x8*>(vg + (int64_t)key * f.v_sl + c * 16 + hf * 8) : x8{};
  }
  const int32_t dj = (KIND == ATTN_MASK_DOCUMENT && key < f.S) ? f.m.doc[key] : -1;

  const int nfull = desc[1], npart = desc[2];
  const int nblk = nfull + npart;
  // chunk 0 visits the first C blocks (C from the plan), chunk 1 the rest
  const int split_len = ((const_i32_ptr)a.tplan)[1];
  const int m_begin = (split && chunk == 1) ? split_len : 0;
  const int m_end = (split && chunk == 0) ? split_len : nblk;
  const int span = m_end - m_begin;
  const const_i32_ptr flist = (const_i32_ptr)(a.tf_idx + (int64_t)kb * f.m.nq);
  const const_i32_ptr plist = (const_i32_ptr)(a.tq_idx + (int64_t)kb * f.m.nq);
  // No kept key in the block: nothing to do (the gradients are zero).
  const bool keys_dead = kv0 >= khi || kv0 + kBlock <= klo;
  const bool keys_cut = kv0 < klo || kv0 + kBlock > khi;  // padding cuts the block
  const int total = keys_dead ? 0 : G * span;              // (query head, query block) pairs
  auto qblock = [&](int n) { const int m = m_begin + n % span; return m < nfull ? flist[m] : plist[m - nfull]; };

  const uint32_t off_e = u_off(f.q_sl * (int64_t)sizeof(T), lane, 0);
  const uint32_t off_o = u_off(f.q_sl * (int64_t)sizeof(T), lane, 1);
  auto issue = [&](int n, BwdQStage& s) __attribute__((always_inline)) {
    const int g = n / span, qb = qblock(n);
    const int h = hk * G + g;
    const int q0 = qb * kBlock;
    const T* qg = static_cast<const T*>(f.q) + b * f.q_sb + h * f.q_sh;
    const T* dg = static_cast<const T*>(a.dout) + b * f.q_sb + h * f.q_sh;
    issue_rows_u<T>(qg, f.q_sl, off_e, off_o, q0, f.L, s.q, wave, lane);
    issue_rows_u<T>(dg, f.q_sl, off_e, off_o, q0, f.L, s.dout, wave, lane);
    const int64_t rb = ((int64_t)b * f.H + h) * f.L;
    const int r = min(q0 + wave * 32 + lq, f.L - 1);
    if (lane < 32) {
      lds_copy4(a.lse2 + rb + r, lds_offset(s.lse2) + (uint32_t)wave * 128u);
      lds_copy4(a.D + rb + r, lds_offset(s.D) + (uint32_t)wave * 128u);
      if (KIND == ATTN_MASK_DOCUMENT) lds_copy4(f.m.doc + r, lds_offset(s.doc) + (uint32_t)wave * 128u);
    }
    if (KIND == ATTN_MASK_CUSTOM) {
      // word 4 kb + wave (this wave's keys) of rows q0 .. q0 + 127
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int rr = min(q0 + hh * 64 + lane, f.L - 1);
        lds_copy4(f.m.bits + (int64_t)rr * f.m.bits_w + 4 * kb + wave,
                  lds_offset(s.bits[wave]) + (uint32_t)hh * 256u);
      }
    }
  };

  f32x16_t dkacc[2], dvacc[2];
#pragma unroll
  for (int te = 0; te < 2; ++te)
#pragma unroll
    for (int r = 0; r < 16; ++r) dkacc[te][r] = dvacc[te][r] = 0.0f;

  if (total > 0) issue(0, st[0]);
  wait_vm_zero();  // K/V rows and the first stage (no compiler-tracked load stays in flight)
  for (int n = 0; n < total; ++n) {
    BwdQStage& s = st[n & 1];
    const int m = m_begin + n % span;
    const int qb = qblock(n);
    const int q0 = qb * kBlock;
    wait_vm_zero();
    wait_lgkm_zero();
    barrier_only();
    if (n + 1 < total) issue(n + 1, st[(n + 1) & 1]);
    const bool partial = m >= nfull || keys_cut;
    const lds_u8 qt_base = (lds_u8)s.q, dt_base = (lds_u8)s.dout;
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      // Sliding windows: a query tile of a partial block whose rule
      // positions all lie before this wave's keys, or all a window or more
      // past them, has no live pair; its MFMAs and vector work are skipped
      // (wave-uniform; its P and dS would be 0).
      if (KIND == ATTN_MASK_SLIDING_WINDOW && partial) {
        const int p0 = q0 + 32 * qt + f.m.q_off, j0 = kv0 + 32 * wave;
        if (p0 + 31 < j0 || p0 - (j0 + 31) >= f.m.window) continue;
      }
      f32x16_t sacc = {}, dpacc = {};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sacc = V::mma(read16<T>(plain_u(qt_base, lane, c) + qt * 4096), kreg[c], sacc);
        dpacc = V::mma(read16<T>(plain_u(dt_base, lane, c) + qt * 4096), vreg[c], dpacc);
      }
      x8 pk[2], dsk[2];
      // P and dS of the tile, with the pair test a compile-time choice (one
      // uniform branch per tile: a runtime test per element cut the code
      // into many small branched blocks), at raised wave priority: the
      // vector phase between the tile's MFMAs, issued first when the other
      // wave on the SIMD is in its MFMAs.
      auto elem = [&](auto partial_c) __attribute__((always_inline)) {
        constexpr bool PARTIAL = decltype(partial_c)::value;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int rl = qt * 32 + 8 * q4 + 4 * hf;  // block row of registers 4 q4 .. 4 q4 + 3
          typedef __attribute__((address_space(3))) const f32x4_t lds_f4;
          const f32x4_t l4 = *reinterpret_cast<lds_f4*>((lds_u8)s.lse2 + rl * 4);
          const f32x4_t d4 = *reinterpret_cast<lds_f4*>((lds_u8)s.D + rl * 4);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = 4 * q4 + u;
            float dmod;
            float p = bwd_prob<SOFTCAP>(sacc[r], l4[u], f, dmod);
            if (PARTIAL) {
              const int32_t di = (KIND == ATTN_MASK_DOCUMENT) ? s.doc[rl + u] : 0;
              const uint32_t word = (KIND == ATTN_MASK_CUSTOM) ? s.bits[wave][rl + u] : 0u;
              if (!bwd_live<KIND>(f, q0 + rl + u, key, klo, khi, di, dj, word, lq)) p = 0.0f;
            }
            const float ds = p * (dpacc[r] - d4[u]) * dmod;
            pk[r >> 3][r & 7] = (T)p;
            dsk[r >> 3][r & 7] = (T)ds;
          }
        }
      };
      __builtin_amdgcn_s_setprio(1);
      if (partial)
        elem(std::true_type{});
      else
        elem(std::false_type{});
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int te = 0; te < 2; ++te) {
          const int g16 = qt * 2 + gi;
          dvacc[te] = V::mma(read_tr2<T>(tr_u(dt_base, lane, te, 0) + g16 * 2048, tr_u(dt_base, lane, te, 1) + g16 * 2048),
                             pk[gi], dvacc[te]);
          dkacc[te] = V::mma(read_tr2<T>(tr_u(qt_base, lane, te, 0) + g16 * 2048, tr_u(qt_base, lane, te, 1) + g16 * 2048),
                             dsk[gi], dkacc[te]);
        }
    }
  }

  if (split) {
    f32x16_t acc[4] = {dkacc[0], dkacc[1], dvacc[0], dvacc[1]};
    float* base = a.part_kv + ((int64_t)kb * 2 * BHk + bk) * kBwdKvSlot;
    if (!merge_two<4>(acc, base + (int64_t)chunk * BHk * kBwdKvSlot, base + (int64_t)(1 - chunk) * BHk * kBwdKvSlot,
                      a.counters_kv + (int64_t)kb * BHk + bk, wave, lane))
      return;
    dkacc[0] = acc[0], dkacc[1] = acc[1], dvacc[0] = acc[2], dvacc[1] = acc[3];
  }

  // dK = scale * dK^T, dV = dV^T: lane = key, registers 4 q4 .. +3 of tile te
  // = head dims te 32 + 8 q4 + 4 hf .. +3.
  if (key < f.S) {
    T* dkg = static_cast<T*>(a.dk) + b * f.k_sb + hk * f.k_sh + (int64_t)key * f.k_sl;
    T* dvg = static_cast<T*>(a.dv) + b * f.v_sb + hk * f.v_sh + (int64_t)key * f.v_sl;
#pragma unroll
    for (int te = 0; te < 2; ++te)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int e0 = te * 32 + q4 * 8 + hf * 4;
        x4 kv, vv;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kv[u] = (T)(dkacc[te][q4 * 4 + u] * f.scale);
          vv[u] = (T)dvacc[te][q4 * 4 + u];
        }
        *reinterpret_cast<x4*>(dkg + e0) = kv;
        *reinterpret_cast<x4*>(dvg + e0) = vv;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
// One stage of the key side: K (V-swizzled, read plain and transposed), V
// (K-swizzled, read plain), the keys' document ids and, for CUSTOM, the
// wave's 32 rows' words of the block.
struct alignas(16) BwdKStage {
  uint8_t k[kBlock * 128];
  uint8_t v[kBlock * 128];
  int32_t doc[kBlock];
  uint32_t bits[kBlock * 4];
};

template <typename T, int KIND, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs a) {
  using V = Vec<T>;
  using x8 = typename V::x8;
  using x4 = typename V::x4;
  __shared__ BwdKStage st[2];
  const FwdArgs& f = a.f;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, hf = lane >> 5;
  const int BH = f.B * f.H;
  // Item from the forward's plan: query block qb, chunk of k (f.split
  // enables the two-way split).
  const WorkItem wi = work_item(f, blockIdx.x / BH);
  if (wi.skip) return;
  const int qb = wi.qb;
  const int bh = xcd_head_order(blockIdx.x % BH, BH, f.kv_group);
  const int b = bh / f.H, h = bh % f.H, hk = h / f.kv_group;
  const int q0 = qb * kBlock;
  const int qi = q0 + wave * 32 + lq;  // this lane's query
  int klo = 0, khi = f.S;
  if (f.key_start != nullptr) klo = min(max(((const_i32_ptr)f.key_start)[b], 0), f.S);
  if (f.key_end != nullptr) khi = max(min(((const_i32_ptr)f.key_end)[b], f.S), klo);

  const T* qg = static_cast<const T*>(f.q) + b * f.q_sb + h * f.q_sh;
  const T* dg = static_cast<const T*>(a.dout) + b * f.q_sb + h * f.q_sh;
  const T* kg = static_cast<const T*>(f.k) + b * f.k_sb + hk * f.k_sh;
  const T* vg = static_cast<const T*>(f.v) + b * f.v_sb + hk * f.v_sh;
  x8 qop[4], doop[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qop[c] = qi < f.L ? *reinterpret_cast<const x8*>(qg + (int64_t)qi * f.q_sl + c * 16 + hf * 8) : x8{};
    doop[c] = qi < f.L ? *reinterpret_cast<const x8*>(dg + (int64_t)qi * f.q_sl + c * 16 + hf * 8) : x8{};
  }
  const int64_t row = (int64_t)bh * f.L + min(qi, f.L - 1);
  const float lse2 = a.lse2[row], Dq = a.D[row];
  const int32_t di = (KIND == ATTN_MASK_DOCUMENT && qi < f.L) ? f.m.doc[qi] : -1;

  const int nfull = ((const_i32_ptr)f.m.full_num)[qb], npart = ((const_i32_ptr)f.m.kv_num)[qb];
  const int nblk = nfull + npart;
  const const_i32_ptr flist = (const_i32_ptr)(f.m.full_idx + (int64_t)qb * f.m.nk);
  const const_i32_ptr plist = (const_i32_ptr)(f.m.kv_idx + (int64_t)qb * f.m.nk);
  auto kvblock = [&](int m) { return m < nfull ? flist[m] : plist[m - nfull]; };
  const int split_len = f.m.schedule[1];
  const int m_begin = (wi.split && wi.chunk == 1) ? split_len : 0;
  const int m_end = (wi.split && wi.chunk == 0) ? split_len : nblk;
  // K is u-swizzled (read plain and transposed), V K-swizzled (plain).
  const uint32_t k_off_e = u_off(f.k_sl * (int64_t)sizeof(T), lane, 0);
  const uint32_t k_off_o = u_off(f.k_sl * (int64_t)sizeof(T), lane, 1);
  const uint32_t v_off =
      (uint32_t)((lane >> 3) * f.v_sl * (int64_t)sizeof(T)) + (uint32_t)(((lane & 7) ^ (lane >> 3)) * 16);
  auto issue = [&](int m, BwdKStage& s) __attribute__((always_inline)) {
    const int kb = kvblock(m), kv0 = kb * kBlock;
    issue_rows_u<T>(kg, f.k_sl, k_off_e, k_off_o, kv0, f.S, s.k, wave, lane);
    issue_rows<T, false>(vg, f.v_sl, v_off, kv0, f.S, s.v, wave, lane);
    if (KIND == ATTN_MASK_DOCUMENT && lane < 32)
      lds_copy4(f.m.doc + min(kv0 + wave * 32 + lane, f.S - 1), lds_offset(s.doc) + (uint32_t)wave * 128u);
    if (KIND == ATTN_MASK_CUSTOM) issue_bits(f.m.bits, f.m.bits_w, q0 + wave * 32, f.L, kb, s.bits, wave, lane);
  };

  f32x16_t dqacc[2];
#pragma unroll
  for (int te = 0; te < 2; ++te)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[te][r] = 0.0f;

  if (m_end > m_begin) issue(m_begin, st[0]);
  wait_vm_zero();
  for (int m = m_begin; m < m_end; ++m) {
    BwdKStage& s = st[(m - m_begin) & 1];
    const int kv0 = kvblock(m) * kBlock;
    wait_vm_zero();
    wait_lgkm_zero();
    barrier_only();
    if (m + 1 < m_end) issue(m + 1, st[(m + 1 - m_begin) & 1]);
    if (kv0 >= khi || kv0 + kBlock <= klo) continue;  // no kept key
    const bool partial = m >= nfull || kv0 < klo || kv0 + kBlock > khi;
    // Full and partial blocks get a body of their own (the pair test a
    // compile-time choice), so each is straight-line code the scheduler can
    // interleave.
    auto body = [&](auto partial_c) __attribute__((always_inline)) {
    constexpr bool PARTIAL = decltype(partial_c)::value;
    uint32_t mw[4] = {0u, 0u, 0u, 0u};
    if (KIND == ATTN_MASK_CUSTOM && PARTIAL) {
      typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4;
      const u32x4_t w4 = *reinterpret_cast<lds_u32x4*>((lds_u8)s.bits + (wave * 32 + lq) * 16);
      mw[0] = w4[0], mw[1] = w4[1], mw[2] = w4[2], mw[3] = w4[3];
    }
    const lds_u8 kt_base = (lds_u8)s.k, vt_base = (lds_u8)s.v;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // Sliding windows: a key tile that every row of this wave sees as
      // after its position, or a window or more behind it, is skipped
      // (wave-uniform; its dS would be 0).
      if (KIND == ATTN_MASK_SLIDING_WINDOW && PARTIAL) {
        const int p0 = q0 + 32 * wave + f.m.q_off, j0 = kv0 + 32 * t;
        if (p0 + 31 < j0 || p0 - (j0 + 31) >= f.m.window) continue;
      }
      f32x16_t sacc = {}, dpacc = {};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sacc = V::mma(read16<T>(plain_u(kt_base, lane, c) + t * 4096), qop[c], sacc);
        dpacc = V::mma(read16<T>(plain_k(vt_base, lane, c) + t * 4096), doop[c], dpacc);
      }
      x8 dsk[2];
      __builtin_amdgcn_s_setprio(1);  // the vector phase (as in dK/dV)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jl = t * 32 + acc_row(r, hf);
        float dmod;
        float p = bwd_prob<SOFTCAP>(sacc[r], lse2, f, dmod);
        if (PARTIAL) {
          const int32_t dj = (KIND == ATTN_MASK_DOCUMENT) ? s.doc[jl] : 0;
          if (!bwd_live<KIND>(f, qi, kv0 + jl, klo, khi, di, dj, mw[t], acc_row(r, hf))) p = 0.0f;
        }
        dsk[r >> 3][r & 7] = (T)(p * (dpacc[r] - Dq) * dmod);
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int te = 0; te < 2; ++te)
          dqacc[te] = V::mma(read_tr2<T>(tr_u(kt_base, lane, te, 0) + (t * 2 + gi) * 2048,
                                         tr_u(kt_base, lane, te, 1) + (t * 2 + gi) * 2048),
                             dsk[gi], dqacc[te]);
    }
    };
    if (partial)
      body(std::true_type{});
    else
      body(std::false_type{});
  }

  if (wi.split) {
    float* base = a.part_q + ((int64_t)qb * 2 * BH + bh) * kBwdQSlot;
    if (!merge_two<2>(dqacc, base + (int64_t)wi.chunk * BH * kBwdQSlot, base + (int64_t)(1 - wi.chunk) * BH * kBwdQSlot,
                      a.counters_q + (int64_t)qb * BH + bh, wave, lane))
      return;
  }

  if (qi < f.L) {
    T* dqg = static_cast<T*>(a.dq) + b * f.q_sb + h * f.q_sh + (int64_t)qi * f.q_sl;
#pragma unroll
    for (int te = 0; te < 2; ++te)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        x4 outv;
#pragma unroll
        for (int u = 0; u < 4; ++u) outv[u] = (T)(dqacc[te][q4 * 4 + u] * f.scale);
        *reinterpret_cast<x4*>(dqg + te * 32 + q4 * 8 + hf * 4) = outv;
      }
  }
}

// ---------------------------------------------------------------------------
// fp32: the same items, plans and split merges as the 16-bit kernels, with
// v_mfma_f32_32x32x2_f32 (one contraction element per lane and step; lane
// half hf takes head dim 32 hf + j at step j) on padded row-major LDS tiles
// filled through registers, one stage per workgroup.
// ---------------------------------------------------------------------------
constexpr int kB32Stride = 68;  // floats per LDS row (64 + 4 padding)

// Rows row0 .. row0 + 127 of a [rows][64] fp32 matrix (row stride sl; rows
// at or past n read as zero) into a padded LDS tile; 8 float4 per thread.
__device__ inline void load_tile32(const float* g, int64_t sl, int row0, int n, float* tile) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = threadIdx.x + u * kThreads, row = c >> 4, ch = c & 15;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row0 + row < n) x = *reinterpret_cast<const float4*>(g + (int64_t)(row0 + row) * sl + ch * 4);
    *reinterpret_cast<float4*>(tile + row * kB32Stride + ch * 4) = x;
  }
}

// One row of 64 floats into the 32 per-lane contraction elements.
__device__ inline void load_row32(const float* row, bool valid, int hf, float (&x)[32]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) v = *reinterpret_cast<const float4*>(row + hf * 32 + c * 4);
    x[4 * c + 0] = v.x, x[4 * c + 1] = v.y, x[4 * c + 2] = v.z, x[4 * c + 3] = v.w;
  }
}

__device__ inline f32x16_t mma32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

struct alignas(16) Bwd32QStage {
  float q[kBlock * kB32Stride];
  float dout[kBlock * kB32Stride];
  float lse2[kBlock];
  float D[kBlock];
  int32_t doc[kBlock];
  uint32_t bits[4][kBlock];
};

// dK, dV of one kv block (one plan item) in fp32. Lanes are keys: S = Q K^T
// and dP = dO V^T put query rows acc_row(r, hf) of tile qt beside this
// lane's key, which is the B-operand layout of dV^T += dO^T P and
// dK^T += Q^T dS (contraction over the queries in register order).
// One workgroup per CU: the K and V rows (64 registers), four accumulator
// tiles and a tile's scores, probabilities and dS stay in registers, more
// than the 256 of two waves per SIMD.
template <int KIND, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 1) void bwd32_dkdv_kernel(BwdArgs a) {
  __shared__ Bwd32QStage s;
  const FwdArgs& f = a.f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 31, hf = lane >> 5;
  const int G = f.kv_group, Hk = f.H / G, BHk = f.B * Hk;
  const i32x4_t desc = ((const_i32x4_ptr)(a.tplan + 4))[blockIdx.x / BHk];
  if (desc[0] < 0) return;
  const int kb = desc[0] & 0xFFFFF, chunk = (desc[0] >> 20) & 3;
  const bool split = a.split_kv && ((desc[0] >> 22) & 3) > 0;
  if (chunk > 0 && !split) return;
  const int bk = blockIdx.x % BHk;
  const int b = bk / Hk, hk = bk % Hk;
  const int kv0 = kb * kBlock;
  const int key = kv0 + wave * 32 + lq;  // this lane's key
  int klo = 0, khi = f.S;
  if (f.key_start != nullptr) klo = min(max(((const_i32_ptr)f.key_start)[b], 0), f.S);
  if (f.key_end != nullptr) khi = max(min(((const_i32_ptr)f.key_end)[b], f.S), klo);

  const float* kg = static_cast<const float*>(f.k) + b * f.k_sb + hk * f.k_sh;
  const float* vg = static_cast<const float*>(f.v) + b * f.v_sb + hk * f.v_sh;
  float kr[32], vr[32];
  load_row32(kg + (int64_t)key * f.k_sl, key < f.S, hf, kr);
  load_row32(vg + (int64_t)key * f.v_sl, key < f.S, hf, vr);
  const int32_t dj = (KIND == ATTN_MASK_DOCUMENT && key < f.S) ? f.m.doc[key] : -1;

  const int nfull = desc[1], npart = desc[2];
  const int nblk = nfull + npart;
  const int split_len = ((const_i32_ptr)a.tplan)[1];
  const int m_begin = (split && chunk == 1) ? split_len : 0;
  const int m_end = (split && chunk == 0) ? split_len : nblk;
  const int span = m_end - m_begin;
  const const_i32_ptr flist = (const_i32_ptr)(a.tf_idx + (int64_t)kb * f.m.nq);
  const const_i32_ptr plist = (const_i32_ptr)(a.tq_idx + (int64_t)kb * f.m.nq);
  const bool keys_dead = kv0 >= khi || kv0 + kBlock <= klo;
  const bool keys_cut = kv0 < klo || kv0 + kBlock > khi;
  const int total = keys_dead ? 0 : G * span;  // (query head, query block) pairs

  f32x16_t dkacc[2], dvacc[2];
#pragma unroll
  for (int te = 0; te < 2; ++te)
#pragma unroll
    for (int r = 0; r < 16; ++r) dkacc[te][r] = dvacc[te][r] = 0.0f;

  for (int n = 0; n < total; ++n) {
    const int g = n / span, m = m_begin + n % span;
    const int qb = m < nfull ? flist[m] : plist[m - nfull];
    const int h = hk * G + g, q0 = qb * kBlock;
    const float* qg = static_cast<const float*>(f.q) + b * f.q_sb + h * f.q_sh;
    const float* dg = static_cast<const float*>(a.dout) + b * f.q_sb + h * f.q_sh;
    __syncthreads();
    load_tile32(qg, f.q_sl, q0, f.L, s.q);
    load_tile32(dg, f.q_sl, q0, f.L, s.dout);
    if (tid < kBlock) {
      const int64_t rb = ((int64_t)b * f.H + h) * f.L;
      const int r = min(q0 + tid, f.L - 1);
      s.lse2[tid] = a.lse2[rb + r];
      s.D[tid] = a.D[rb + r];
      if (KIND == ATTN_MASK_DOCUMENT) s.doc[tid] = f.m.doc[r];
    }
    if (KIND == ATTN_MASK_CUSTOM) {
      // word 4 kb + w (wave w's keys) of rows q0 .. q0 + 127
      for (int u = tid; u < 4 * kBlock; u += kThreads) {
        const int w = u >> 7, row = u & (kBlock - 1);
        s.bits[w][row] = f.m.bits[(int64_t)min(q0 + row, f.L - 1) * f.m.bits_w + 4 * kb + w];
      }
    }
    __syncthreads();
    const bool partial = m >= nfull || keys_cut;
#pragma unroll 1
    for (int qt = 0; qt < 4; ++qt) {
      f32x16_t sacc = {}, dpacc = {};
      const float* qrow = s.q + (qt * 32 + lq) * kB32Stride + hf * 32;
      const float* drow = s.dout + (qt * 32 + lq) * kB32Stride + hf * 32;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        sacc = mma32(qrow[j], kr[j], sacc);
        dpacc = mma32(drow[j], vr[j], dpacc);
      }
      float p[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = qt * 32 + acc_row(r, hf);
        float dmod;
        float pr = bwd_prob<SOFTCAP>(sacc[r], s.lse2[rl], f, dmod);
        if (partial) {
          const int32_t di = (KIND == ATTN_MASK_DOCUMENT) ? s.doc[rl] : 0;
          const uint32_t word = (KIND == ATTN_MASK_CUSTOM) ? s.bits[wave][rl] : 0u;
          if (!bwd_live<KIND>(f, q0 + rl, key, klo, khi, di, dj, word, lq)) pr = 0.0f;
        }
        p[r] = pr;
        ds[r] = pr * (dpacc[r] - s.D[rl]) * dmod;
      }
#pragma unroll
      for (int te = 0; te < 2; ++te)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = qt * 32 + acc_row(r, hf);
          dvacc[te] = mma32(s.dout[rl * kB32Stride + te * 32 + lq], p[r], dvacc[te]);
          dkacc[te] = mma32(s.q[rl * kB32Stride + te * 32 + lq], ds[r], dkacc[te]);
        }
    }
  }

  if (split) {
    f32x16_t acc[4] = {dkacc[0], dkacc[1], dvacc[0], dvacc[1]};
    float* base = a.part_kv + ((int64_t)kb * 2 * BHk + bk) * kBwdKvSlot;
    if (!merge_two<4>(acc, base + (int64_t)chunk * BHk * kBwdKvSlot, base + (int64_t)(1 - chunk) * BHk * kBwdKvSlot,
                      a.counters_kv + (int64_t)kb * BHk + bk, wave, lane))
      return;
    dkacc[0] = acc[0], dkacc[1] = acc[1], dvacc[0] = acc[2], dvacc[1] = acc[3];
  }

  // lane = key; registers 4 q4 .. +3 of tile te = head dims te 32 + 8 q4 + 4 hf .. +3
  if (key < f.S) {
    float* dkg = static_cast<float*>(a.dk) + b * f.k_sb + hk * f.k_sh + (int64_t)key * f.k_sl;
    float* dvg = static_cast<float*>(a.dv) + b * f.v_sb + hk * f.v_sh + (int64_t)key * f.v_sl;
#pragma unroll
    for (int te = 0; te < 2; ++te)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int e0 = te * 32 + q4 * 8 + hf * 4;
        const f32x16_t& dk4 = dkacc[te];
        const f32x16_t& dv4 = dvacc[te];
        *reinterpret_cast<float4*>(dkg + e0) = make_float4(dk4[q4 * 4] * f.scale, dk4[q4 * 4 + 1] * f.scale,
                                                           dk4[q4 * 4 + 2] * f.scale, dk4[q4 * 4 + 3] * f.scale);
        *reinterpret_cast<float4*>(dvg + e0) = make_float4(dv4[q4 * 4], dv4[q4 * 4 + 1], dv4[q4 * 4 + 2], dv4[q4 * 4 + 3]);
      }
  }
}

struct alignas(16) Bwd32KStage {
  float k[kBlock * kB32Stride];
  float v[kBlock * kB32Stride];
  int32_t doc[kBlock];
};

// dQ of one query block (one item of the forward's plan) in fp32. Lanes are
// queries, as in the forward: S^T = K Q^T and dP^T = V dO^T, then
// dQ^T += K^T dS^T with the keys of the accumulator rows as contraction.
template <int KIND, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 2) void bwd32_dq_kernel(BwdArgs a) {
  __shared__ Bwd32KStage s;
  const FwdArgs& f = a.f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 31, hf = lane >> 5;
  const int BH = f.B * f.H;
  const WorkItem wi = work_item(f, blockIdx.x / BH);
  if (wi.skip) return;
  const int qb = wi.qb;
  const int bh = xcd_head_order(blockIdx.x % BH, BH, f.kv_group);
  const int b = bh / f.H, h = bh % f.H, hk = h / f.kv_group;
  const int q0 = qb * kBlock;
  const int qi = q0 + wave * 32 + lq;  // this lane's query
  int klo = 0, khi = f.S;
  if (f.key_start != nullptr) klo = min(max(((const_i32_ptr)f.key_start)[b], 0), f.S);
  if (f.key_end != nullptr) khi = max(min(((const_i32_ptr)f.key_end)[b], f.S), klo);

  const float* qg = static_cast<const float*>(f.q) + b * f.q_sb + h * f.q_sh;
  const float* dg = static_cast<const float*>(a.dout) + b * f.q_sb + h * f.q_sh;
  const float* kg = static_cast<const float*>(f.k) + b * f.k_sb + hk * f.k_sh;
  const float* vg = static_cast<const float*>(f.v) + b * f.v_sb + hk * f.v_sh;
  float qv[32], dov[32];
  load_row32(qg + (int64_t)qi * f.q_sl, qi < f.L, hf, qv);
  load_row32(dg + (int64_t)qi * f.q_sl, qi < f.L, hf, dov);
  const int64_t row = (int64_t)bh * f.L + min(qi, f.L - 1);
  const float lse2 = a.lse2[row], Dq = a.D[row];
  const int32_t di = (KIND == ATTN_MASK_DOCUMENT && qi < f.L) ? f.m.doc[qi] : -1;

  const int nfull = f.m.full_num[qb], npart = f.m.kv_num[qb];
  const int nblk = nfull + npart;
  const int32_t* flist = f.m.full_idx + (int64_t)qb * f.m.nk;
  const int32_t* plist = f.m.kv_idx + (int64_t)qb * f.m.nk;
  const int split_len = f.m.schedule[1];
  const int m_begin = (wi.split && wi.chunk == 1) ? split_len : 0;
  const int m_end = (wi.split && wi.chunk == 0) ? split_len : nblk;

  f32x16_t dqacc[2];
#pragma unroll
  for (int te = 0; te < 2; ++te)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[te][r] = 0.0f;

  for (int m = m_begin; m < m_end; ++m) {
    const int kb = m < nfull ? flist[m] : plist[m - nfull];
    const int kv0 = kb * kBlock;
    if (kv0 >= khi || kv0 + kBlock <= klo) continue;  // no kept key (uniform over the workgroup)
    const bool partial = m >= nfull || kv0 < klo || kv0 + kBlock > khi;
    __syncthreads();
    load_tile32(kg, f.k_sl, kv0, f.S, s.k);
    load_tile32(vg, f.v_sl, kv0, f.S, s.v);
    if (KIND == ATTN_MASK_DOCUMENT && tid < kBlock) s.doc[tid] = f.m.doc[min(kv0 + tid, f.S - 1)];
    uint4 mw = make_uint4(0u, 0u, 0u, 0u);
    if (KIND == ATTN_MASK_CUSTOM && partial)
      mw = *reinterpret_cast<const uint4*>(f.m.bits + (int64_t)min(qi, f.L - 1) * f.m.bits_w + 4 * kb);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x16_t sacc = {}, dpacc = {};
      const float* krow = s.k + (t * 32 + lq) * kB32Stride + hf * 32;
      const float* vrow = s.v + (t * 32 + lq) * kB32Stride + hf * 32;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        sacc = mma32(krow[j], qv[j], sacc);
        dpacc = mma32(vrow[j], dov[j], dpacc);
      }
      const uint32_t word = t == 0 ? mw.x : t == 1 ? mw.y : t == 2 ? mw.z : mw.w;
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jl = t * 32 + acc_row(r, hf);
        float dmod;
        float p = bwd_prob<SOFTCAP>(sacc[r], lse2, f, dmod);
        if (partial) {
          const int32_t dj = (KIND == ATTN_MASK_DOCUMENT) ? s.doc[jl] : 0;
          if (!bwd_live<KIND>(f, qi, kv0 + jl, klo, khi, di, dj, word, acc_row(r, hf))) p = 0.0f;
        }
        ds[r] = p * (dpacc[r] - Dq) * dmod;
      }
#pragma unroll
      for (int te = 0; te < 2; ++te)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jl = t * 32 + acc_row(r, hf);
          dqacc[te] = mma32(s.k[jl * kB32Stride + te * 32 + lq], ds[r], dqacc[te]);
        }
    }
  }

  if (wi.split) {
    float* base = a.part_q + ((int64_t)qb * 2 * BH + bh) * kBwdQSlot;
    if (!merge_two<2>(dqacc, base + (int64_t)wi.chunk * BH * kBwdQSlot, base + (int64_t)(1 - wi.chunk) * BH * kBwdQSlot,
                      a.counters_q + (int64_t)qb * BH + bh, wave, lane))
      return;
  }

  if (qi < f.L) {
    float* dqg = static_cast<float*>(a.dq) + b * f.q_sb + h * f.q_sh + (int64_t)qi * f.q_sl;
#pragma unroll
    for (int te = 0; te < 2; ++te)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16_t& d4 = dqacc[te];
        *reinterpret_cast<float4*>(dqg + te * 32 + q4 * 8 + hf * 4) =
            make_float4(d4[q4 * 4] * f.scale, d4[q4 * 4 + 1] * f.scale, d4[q4 * 4 + 2] * f.scale,
                        d4[q4 * 4 + 3] * f.scale);
      }
  }
}

template <int KIND, bool SOFTCAP>
hipError_t launch_bwd_kernels(int32_t dtype, const BwdArgs& a, hipStream_t stream) {
  const int64_t Hk = a.f.H / a.f.kv_group;
  const dim3 block(kThreads);
  // up to two items per kv block / query block (items past a plan's end exit)
  const dim3 g_dkdv((unsigned)((int64_t)a.f.B * Hk * a.f.m.nk * kMaxChunks));
  const dim3 g_dq((unsigned)((int64_t)a.f.B * a.f.H * a.f.m.nq * kMaxChunks));
  switch (dtype) {
    case ATTN_BF16:
      if (a.f.m.nk > 0) hipLaunchKernelGGL((bwd_dkdv_kernel<__bf16, KIND, SOFTCAP>), g_dkdv, block, 0, stream, a);
      if (a.f.m.nq > 0) hipLaunchKernelGGL((bwd_dq_kernel<__bf16, KIND, SOFTCAP>), g_dq, block, 0, stream, a);
      break;
    case ATTN_F16:
      if (a.f.m.nk > 0) hipLaunchKernelGGL((bwd_dkdv_kernel<_Float16, KIND, SOFTCAP>), g_dkdv, block, 0, stream, a);
      if (a.f.m.nq > 0) hipLaunchKernelGGL((bwd_dq_kernel<_Float16, KIND, SOFTCAP>), g_dq, block, 0, stream, a);
      break;
    case ATTN_F32:
      if (a.f.m.nk > 0) hipLaunchKernelGGL((bwd32_dkdv_kernel<KIND, SOFTCAP>), g_dkdv, block, 0, stream, a);
      if (a.f.m.nq > 0) hipLaunchKernelGGL((bwd32_dq_kernel<KIND, SOFTCAP>), g_dq, block, 0, stream, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// The dK/dV and dQ kernels of one mask family (defined in bwd_<family>.hip).
template <int KIND>
hipError_t launch_backward_family(int32_t dtype, const BwdArgs& a, hipStream_t stream) {
  return a.f.softcap > 0.0f ? launch_bwd_kernels<KIND, true>(dtype, a, stream)
                            : launch_bwd_kernels<KIND, false>(dtype, a, stream);
}

}  // namespace bsattn
