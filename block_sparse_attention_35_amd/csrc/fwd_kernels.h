// Fused block-sparse attention forward for gfx950: the kernels, and the
// launch templates instantiated by one translation unit per mask family
// (fwd_*.hip), so the instantiations compile in parallel.
//
// O = softmax(Q K^T * scale + mask bias [+ soft-cap score_mod]) V and the
// per-row logsumexp, without writing the L x S score table anywhere: a
// workgroup owns one work item (128 query rows of one batch*head, all of
// their live kv blocks or one chunk of them), walks the item's full kv
// blocks and then its partial kv blocks from the BlockMask, and keeps a
// running row max and row sum (online softmax) while accumulating P V.
// Definition: "SDPA replaces hand-written attention", section 1 (Attention
// equation and its four steps); running max / running sum instead of the
// score table: same page, section 2, and "FlashAttention" (service-dock),
// tiled softmax is exact; tiles kept in on-chip memory with only the result
// written back: "Flash Attention 2 and the IO bottleneck" (tcdigital),
// section on tiling. Skipped / partial / full blocks: "FlexAttention on Apple
// Silicon: block masks", closing section; soft-cap: same page, "Bonus".
// User-supplied masks (kind CUSTOM) arrive bit-packed, four words per (query
// row, kv block); each block's words are staged with its K tile and read by
// the pair test of partial blocks only.
//
// Work layout (4 waves of 64 lanes, each wave owns 32 query rows):
//  * S^T = K_j Q^T is computed with 32x32 MFMA tiles, kv along M and queries
//    along N, so each lane holds one query (lane % 32) and 16 kv values per
//    32x32 tile. Row max / row sum are then in-lane reductions plus one swap
//    between the two 32-lane halves.
//  * The S^T accumulator layout (lane = query, registers = kv) is exactly the
//    B operand layout of O^T = V^T P^T once probabilities are packed to
//    16 bits, because the contraction index may be permuted freely as long as
//    both operands use the same permutation; the matching V^T operand comes
//    from transposed LDS reads (ds_read_b64_tr_b16) of the row-major V tile.
//  * K and V tiles go from global memory straight to LDS (double buffered,
//    16-byte chunks XOR-swizzled); each block is two phases of MFMA chunks
//    with the vector work of the softmax placed between the MFMAs.
//  * Long query blocks are split into two work items whose partial results
//    the later one merges (see the work plan of the block-mask builder).
//
// bf16/fp16 use v_mfma_f32_32x32x16_{bf16,f16}; fp32 uses v_mfma_f32_32x32x2_f32
// and keeps probabilities in fp32.
#pragma once

#include <cmath>
#include <type_traits>

#include "bsattn.h"
#include "internal.h"

namespace bsattn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
struct Vec;
template <>
struct Vec<__bf16> {
  using x8 = bf16x8_t;
  using x4 = bf16x4_t;
  using x2 = bf16x2_t;
  static __device__ inline f32x16_t mma(x8 a, x8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // acc + a.x + a.y in fp32 (v_dot2c_f32_bf16 against (1, 1)). Written as
  // volatile asm so it stays in the chunk that produces `a` (a plain builtin
  // is only ordered by its data and gets sunk to the end of the phase, where
  // the sum is used).
  static __device__ inline float add_pair(x2 a, float acc) {
    asm volatile("v_dot2c_f32_bf16 %0, 0x3f803f80, %1" : "+v"(acc) : "v"(a));
    return acc;
  }
};
template <>
struct Vec<_Float16> {
  using x8 = f16x8_t;
  using x4 = f16x4_t;
  using x2 = f16x2_t;
  static __device__ inline f32x16_t mma(x8 a, x8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  // acc + a.x + a.y in fp32 (v_dot2c_f32_f16 against (1, 1)), volatile asm
  // for the same reason as the bf16 form.
  static __device__ inline float add_pair(x2 a, float acc) {
    asm volatile("v_dot2c_f32_f16 %0, 0x3c003c00, %1" : "+v"(acc) : "v"(a));
    return acc;
  }
};

// A v_dot2c result may be read by another VALU instruction only three wait
// states after it is written. The compiler keeps that distance for the
// instructions it knows, not for the asm dot above, so the two row sums pass
// through this (tied to both, so it sits after the last dot and before the
// first other reader) before anything else reads them.
__device__ inline void dot_results_settle(float& a, float& b) {
  asm volatile("s_nop 2" : "+v"(a), "+v"(b));
}

// Other half's value combined with ours: v_permlane32_swap exchanges lanes
// l and l^32 between its two operands; with both operands equal, the two
// results of each lane are {x_l, x_(l^32)} in some order.
__device__ inline float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half_min(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// c * tanh(y), y = s * scale / c, in base-2 units of the result, from
// c tanh(y) = c - 2c / (e^(2y) + 1): one multiply, exp, add, reciprocal and
// FMA. It saturates to +-c for large |y| (e = inf or 0); near y = 0 the
// cancellation costs at most an absolute 2^-23 c, far below the rounding of
// the probabilities.
__device__ inline float softcap_log2(float s, float two_log2e_scale_over_cap, float cap_log2e) {
  const float e = fast_exp2(s * two_log2e_scale_over_cap);
  return fmaf(-2.0f * cap_log2e, __builtin_amdgcn_rcpf(1.0f + e), cap_log2e);
}

// The soft-cap's reciprocal term r = 1 / (e^(2y) + 1) of a raw score s (y =
// s * scale / c): the capped score in base-2 units is cL - 2 cL r with cL =
// c log2(e), so a block keeps r (the largest capped score is that of the
// smallest r) and a probability is exp2(fma(r, -2 cL, cL - m)): one FMA
// fewer per score than forming the capped score first. A masked pair has
// r = +inf, hence probability 0.
__device__ inline float softcap_recip(float s, float two_log2e_scale_over_cap) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(s * two_log2e_scale_over_cap));
}

// A query at rule position p (its row i plus the mask's query offset) may see
// key j, with j < S checked; di, dj are the document ids of row i and key j.
// (CUSTOM checks j < S here; its bit is tested by the caller.)
template <int KIND>
__device__ inline bool pair_live(int p, int j, int S, int W, int32_t di, int32_t dj) {
  bool ok = j < S;
  if (KIND == ATTN_MASK_CAUSAL) ok &= j <= p;
  if (KIND == ATTN_MASK_SLIDING_WINDOW) ok &= (j <= p) & (p - j < W);
  if (KIND == ATTN_MASK_DOCUMENT) ok &= (j <= p) & (di == dj);
  return ok;
}

// Row of the 32x32 MFMA accumulator held in register r by lane half hf.
__device__ inline int acc_row(int r, int hf) { return ((r >> 2) << 3) + (hf << 2) + (r & 3); }

// Per-lane online-softmax state for one query row (half of its kv values).
struct RowState {
  float m;  // running max in log2 units (-inf before the first live key)
  float l;  // running sum of this lane half's probabilities
};

// Turn four S^T tiles (raw q.k) into probabilities in place and update the
// running statistics. Returns alpha, the factor that rescales the previous
// accumulator. kv0: absolute index of the block's first key.
template <int KIND, bool PARTIAL, bool SOFTCAP>
__device__ inline float softmax_tiles(f32x16_t (&s)[4], RowState& st, int qi, int kv0, int hf,
                                      const FwdArgs& a, int32_t dq, const int32_t* doc_k, int klo,
                                      int khi, uint4 mw) {
  const float c1 = a.scale * kLog2e;
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = s[t][r];
      if (SOFTCAP) x = softcap_log2(x, 2.0f * kLog2e * a.scale / a.softcap, a.softcap * kLog2e);
      if (PARTIAL) {
        const int jl = t * 32 + acc_row(r, hf);
        const int32_t dj = (KIND == ATTN_MASK_DOCUMENT) ? doc_k[jl] : 0;
        // kept keys [klo, khi): the mask's own j < S, and key padding
        bool ok = pair_live<KIND>(qi + a.m.q_off, kv0 + jl, khi, a.m.window, dq, dj) && kv0 + jl >= klo;
        if (KIND == ATTN_MASK_CUSTOM) {
          const uint32_t w = t == 0 ? mw.x : t == 1 ? mw.y : t == 2 ? mw.z : mw.w;
          ok &= (w >> acc_row(r, hf)) & 1u;
        }
        if (!ok) x = -INFINITY;
      }
      s[t][r] = x;
      mx = fmaxf(mx, x);
    }
  }
  mx = half_max(mx);
  // Without the soft-cap the max is over raw scores; scale > 0 keeps order.
  const float m_blk = SOFTCAP ? mx : mx * c1;
  const float m_new = fmaxf(st.m, m_blk);
  const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
  const float alpha = fast_exp2(st.m - m_use);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = s[t][r];
      s[t][r] = SOFTCAP ? fast_exp2(x - m_use) : fast_exp2(fmaf(x, c1, -m_use));
    }
  }
  st.m = m_new;
  return alpha;
}

// ---------------------------------------------------------------------------
// bf16 / fp16 kernel
// ---------------------------------------------------------------------------
// LDS holds two K tiles and two V tiles (128 rows x 128 bytes each, row-major)
// plus the document ids of each K tile. Rows are split in eight 16-byte
// chunks stored XOR-swizzled: K chunk c of row r sits in slot c ^ (r & 7)
// (conflict-free 16-byte reads of 8 consecutive rows); V chunk c sits in slot
// c ^ 2(r & 3) (conflict-free transposed reads of 4 rows x 32 bytes by each
// 16-lane group).
struct alignas(16) KStage {
  uint8_t k[kBlock * 128];
  int32_t doc[kBlock];
};
struct alignas(16) VStage {
  uint8_t v[kBlock * 128];
};

// The running max only moves when a block's max exceeds it by more than this
// many powers of two, so probabilities stay <= 2^8 and the accumulator rescale
// is skipped for most blocks. The result is algebraically the same: numerator
// and normaliser share the reference.
constexpr float kRescaleLog2 = 8.0f;

// Workgroup barrier without memory fences: the caller waits for exactly the
// memory operations it needs first (the fences of __syncthreads would also
// wait for the next tile's in-flight copies). The signal fences only keep the
// compiler from moving memory accesses across the barrier.
__device__ inline void barrier_only() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8]
// | vmcnt[5:4] << 14), leaving the other counters unconstrained.
__device__ inline void wait_vm_zero() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ inline void wait_lgkm_zero() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Wait until at most N vector memory operations of this wave are in flight.
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt has six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Block index lists are read through the constant address space so the loads
// are scalar (they never change during a launch).
typedef __attribute__((address_space(4))) const int32_t* const_i32_ptr;

// Global -> LDS copies (global_load_lds_dword{x4}): lane l writes bytes
// [size*l, size*(l+1)) after the wave-uniform base in M0. They are issued as
// inline asm so that the compiler's own wait insertion, which cannot tell
// these LDS writes from the tiles being read, adds no wait for the copies in
// flight before every LDS read; every wait on them is explicit (wait_vm_zero,
// then a barrier). The instructions have no result registers and their
// address registers are read at issue. The compiler spaces its own memory
// instructions from the writes they depend on, but not inside asm: an LDS
// DMA reads M0 one wait state after the write at the earliest (the s_nop 0
// between the two), and a vector memory instruction reads an SGPR that a VALU
// instruction wrote (a v_readfirstlane of the base) five wait states after
// the write at the earliest (the s_nop 4 of the second form). The first form
// takes a 64-bit address per lane; the second a wave-uniform base in SGPRs
// plus a 32-bit byte offset per lane, which keeps the per-tile address
// arithmetic scalar.
__device__ inline uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
__device__ inline void lds_copy16(const void* src, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_wave_base))
               : "memory", "m0");
}
__device__ inline void lds_copy16_base(const void* sbase, uint32_t lane_off, uint32_t lds_wave_base) {
  // readfirstlane returns int: widen through uint32_t so the low word is
  // zero-extended (a sign extension would set the high word's bits).
  const uint64_t p = (uint64_t)(uintptr_t)sbase;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(lane_off), "s"((const void*)(uintptr_t)(lo | (hi << 32))),
                 "s"(__builtin_amdgcn_readfirstlane(lds_wave_base))
               : "memory", "m0");
}
__device__ inline void lds_copy4(const void* src, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_wave_base))
               : "memory", "m0");
}

// One wave's share of a tile copy: tile rows 32w .. 32w+31 (4 KiB), four
// copies of 8 rows. Lane l of copy i fills slot l & 7 of tile row
// 32w + 8i + l/8 and fetches the global chunk that the swizzle puts there;
// that chunk depends only on the lane, so the per-lane byte offset (relative
// to the copy's first row) is fixed for the whole launch. Rows past the end
// are clamped to the last key (their scores are masked); that only happens on
// a ragged last tile.
template <typename T, bool IS_V>
__device__ inline void issue_rows(const T* g, int64_t sl, uint32_t lane_off, int kv0, int S,
                                  uint8_t* tile, int wave, int lane) {
  const int row0 = kv0 + wave * 32;  // first key of this wave's rows
  const uint32_t lds0 = lds_offset(tile) + (uint32_t)wave * 4096u;
  if (kv0 + kBlock <= S) {
    // One 64-bit multiply per tile; copy i starts 8 i rows further on.
    const uint8_t* base = reinterpret_cast<const uint8_t*>(g + (int64_t)row0 * sl);
    const int64_t step = sl * (int64_t)(8 * sizeof(T));
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_copy16_base(base + i * step, lane_off, lds0 + 1024u * i);
  } else {
    const int chunk = IS_V ? ((lane & 7) ^ (((lane >> 3) & 3) << 1)) : ((lane & 7) ^ (lane >> 3));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(row0 + 8 * i + (lane >> 3), S - 1);
      lds_copy16(g + (int64_t)key * sl + chunk * 8, lds0 + 1024u * i);
    }
  }
}

template <typename T, int KIND>
__device__ inline void issue_k(const T* kg, int64_t k_sl, uint32_t k_off, const int32_t* doc, int kv0,
                               int S, KStage& st, int wave, int lane) {
  issue_rows<T, false>(kg, k_sl, k_off, kv0, S, st.k, wave, lane);
  if (KIND == ATTN_MASK_DOCUMENT) {
    // ids of keys 32*wave .. 32*wave+31 of the tile, 4 bytes per lane
    if (lane < 32) {
      const int64_t j = min(kv0 + wave * 32 + lane, S - 1);
      lds_copy4(doc + j, lds_offset(st.doc) + (uint32_t)wave * 128u);
    }
  }
}

typedef __attribute__((address_space(3))) const uint8_t* lds_u8;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// All LDS of a workgroup: two K stages and two V stages.
struct alignas(16) Lds {
  KStage k[2];
  VStage v[2];
};
// The chained sliding-window kernel: K stages without document ids (the
// rule needs none), two V stages, and the next item's Q rows, copied by LDS
// DMA during an item's last block: 80 KiB, two workgroups per CU.
struct alignas(16) KStageRows {
  uint8_t k[kBlock * 128];
};
struct alignas(16) LdsChain {
  KStageRows k[2];
  VStage v[2];
  uint8_t q[kBlock * 128];
};
// For CUSTOM masks, also each stage's mask words: [query row][4].
struct alignas(16) LdsBits {
  KStage k[2];
  VStage v[2];
  uint32_t bits[2][kBlock * 4];
};

// Mask words of this wave's 32 query rows (row0 .. row0 + 31; rows past L
// repeat row L - 1) for kv block kb: 16 bytes per row, lanes 0..31.
__device__ inline void issue_bits(const uint32_t* bits, int W, int row0, int L, int kb, uint32_t* stage,
                                  int wave, int lane) {
  if (lane < 32) {
    const int r = min(row0 + lane, L - 1);
    lds_copy16(bits + (int64_t)r * W + 4 * kb, lds_offset(stage) + (uint32_t)wave * 512u);
  }
}

// Per-lane LDS read addresses into stage 0; stage 1 is a constant away, and
// every read of a step is one of these plus a constant that fits the
// instruction's offset field.
//  * k[c]: K operand of contraction step c (head dims 16c + 8hf .. +7) of
//    key lq of the tile's first 32-key tile: row lq, chunk 2c + hf, stored
//    in slot (2c + hf) ^ (lq & 7). Tile t adds 4096 bytes.
//  * v[te]: V^T operand of head-dim tile te. For 16-key group g, lane half
//    hf holds keys 16g + 4hf + {0..3} and 16g + 8 + 4hf + {0..3} of P^T; the
//    matching V^T operand comes from two transposed LDS reads: in each
//    16-lane group, lane i16 supplies the address of row (key)
//    r0 + i16/4, head dims eb + 4(i16%4) .. +3 (16-byte chunk eb/8 + ...,
//    swizzled by 2(row & 3)), and receives head dim eb + i16 of rows
//    r0 .. r0+3. Group g adds 2048 bytes; the second read adds 1024.
struct LanePtrs {
  lds_u8 k[4];
  lds_u8 v[2];
};

template <class LdsT>
__device__ inline LanePtrs make_lane_ptrs(const LdsT& lds, int lane) {
  LanePtrs p;
  const int lq = lane & 31, hf = lane >> 5;
  const lds_u8 kb = (lds_u8)lds.k[0].k;
  const lds_u8 vb = (lds_u8)lds.v[0].v;
#pragma unroll
  for (int c = 0; c < 4; ++c) p.k[c] = kb + lq * 128 + (((2 * c + hf) ^ (lq & 7)) << 4);
  const int g16 = lane >> 4, i16 = lane & 15;
  const int r1 = hf * 4 + (i16 >> 2);  // row of group 0
#pragma unroll
  for (int te = 0; te < 2; ++te) {
    const int e = te * 32 + (g16 & 1) * 16 + (i16 & 3) * 4;
    const int c16 = e >> 3, half = (e >> 2) & 1;
    p.v[te] = vb + r1 * 128 + ((c16 ^ ((r1 & 3) << 1)) << 4) + half * 8;
  }
  return p;
}

// Classes of a 32 x 32 score tile in a partial block.
enum { kTileLive = 0, kTileMixed = 1, kTileDead = 2 };

// Keeps the compiler's schedulers from moving any instruction across this
// point, so the source order of the chunks below is the issue order.
__device__ inline void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// One KV block for this wave's 32 query rows, in two phases of 16 chunks,
// each chunk one MFMA plus a slice of vector work that does not depend on
// it, so LDS latency is covered and the matrix and vector units overlap:
//  Q. S^T = K Q^T (MFMA j: 32-key tile j / 4, contraction step j % 4; K
//     fragments read four MFMAs ahead), with the score_mod, mask and max of
//     the tile finished before.
//  P. O^T += V^T P^T (MFMA i: 16-key group i / 2, head-dim tile i % 2; V
//     fragments read four MFMAs ahead), with the probabilities of the next
//     group.
template <typename T, int KIND, bool SOFTCAP, bool PARTIAL, bool PADDED, class KSt>
__device__ __forceinline__ void fwd_block(const KSt& kst, const lds_u8 (&kp)[4], const lds_u8 (&vp)[2],
                                          const typename Vec<T>::x8 (&qop)[4], f32x16_t (&oacc)[2],
                                          float& m_ref, float& l, int qi, int row0, int kv0, int lane, const FwdArgs& a,
                                          int32_t dq, int klo, int khi, const uint32_t* mbits) {
  using V = Vec<T>;
  using x8 = typename V::x8;
  typedef __attribute__((address_space(3))) const x8 lds_x8;
  const int hf = lane >> 5;
  const float c1 = a.scale * kLog2e;

  // K operand of QK MFMA j: head dims 16c + 8hf .. +7 of key 32t + lq.
  auto k_frag = [&](int j) -> x8 {
    const int t = j >> 2, c = j & 3;
    return *reinterpret_cast<const lds_x8*>(kp[c] + t * 4096);
  };
  // V^T operand of PV MFMA i: two transposed reads, 8 rows apart (see
  // LanePtrs).
  auto v_frag = [&](int i) -> x8 {
    const int g = i >> 1, te = i & 1;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp[te] + g * 2048));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp[te] + g * 2048 + 1024));
    const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(x8, both);
  };
  // In a partial block, each 32 x 32 tile of this wave (its rows row0 ..
  // row0 + 31 x keys kv0 + 32t .. +31) is classified in closed form, with
  // scalar arithmetic only, from the rule's offset interval and the kept key
  // range [klo, khi) (the whole [0, S) without padding), as whole blocks are:
  // all pairs live, none live, or mixed. Only mixed tiles test pairs, and
  // only live tiles skip the test; for document masks the interval decides
  // only "none live".
  int tile_cls[4] = {kTileLive, kTileLive, kTileLive, kTileLive};
  // Sliding windows: a dead tile's QK and PV MFMAs and its exponentials are
  // skipped too (wave-uniform branches; its probabilities would be 0). Each of
  // a window's two partial blocks holds 0..3 dead tiles per wave. For the
  // other rules the branches cost more than they save.
  constexpr bool SKIP_DEAD = PARTIAL && KIND == ATTN_MASK_SLIDING_WINDOW;
  // CUSTOM: this lane's row's mask words of the block (word t = tile t).
  uint32_t mw[4] = {0u, 0u, 0u, 0u};
  if (PARTIAL && KIND == ATTN_MASK_CUSTOM) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4;
    const u32x4_t w4 = *reinterpret_cast<lds_u32x4*>((lds_u8)mbits + ((row0 % kBlock) + (lane & 31)) * 16);
    mw[0] = w4[0], mw[1] = w4[1], mw[2] = w4[2], mw[3] = w4[3];
  }
  if (PARTIAL) {
    const int i0 = row0 + a.m.q_off, i1 = i0 + 31;  // the rows' rule positions
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j0 = kv0 + 32 * t, j1 = min(j0 + 31, khi - 1);
      const bool outside = j0 > khi - 1 || (PADDED && j0 + 31 < klo);
      const bool edge = j0 + 31 > khi - 1 || (PADDED && j0 < klo);  // range ends inside
      int c;
      if (outside) {
        c = kTileDead;
      } else if (KIND == ATTN_MASK_CUSTOM) {
        // from the words of the wave's 32 rows: none set, all set, or mixed
        if (__ballot(mw[t] != 0u) == 0)
          c = kTileDead;
        else if (!edge && __ballot(mw[t] != ~0u) == 0)
          c = kTileLive;
        else
          c = kTileMixed;
      } else if (KIND == ATTN_MASK_NONE) {
        c = edge ? kTileMixed : kTileLive;
      } else {
        const int dmin = i0 - j1, dmax = i1 - j0;  // offsets p - j of the tile
        const int w = (KIND == ATTN_MASK_SLIDING_WINDOW) ? a.m.window : 0x7fffffff;
        if (dmax < 0 || dmin > w - 1)
          c = kTileDead;
        else if (KIND != ATTN_MASK_DOCUMENT && dmin >= 0 && dmax <= w - 1 && !edge)
          c = kTileLive;
        else
          c = kTileMixed;
      }
      tile_cls[t] = c;
    }
  }
  // Pair test of a mixed tile as an interval of the key's offset inside the
  // tile: this lane's key of register r is kv0 + 32t + 4hf + c(r), with
  // c(r) = 8(r / 4) + r % 4; it is live when lo - 32t <= c(r) <= hi - 32t.
  // hi bounds by j <= p and j < khi, lo by p - j < W (sliding windows) and
  // j >= klo (padding), p = qi + q_off the row's rule position.
  const int rel = qi + a.m.q_off - kv0 - 4 * hf;
  const int hi = (KIND == ATTN_MASK_NONE || KIND == ATTN_MASK_CUSTOM) ? khi - 1 - kv0 - 4 * hf
                                                                      : min(rel, khi - 1 - kv0 - 4 * hf);
  // (A window wider than 2^30 never bites: S is far smaller.)
  int lo = (KIND == ATTN_MASK_SLIDING_WINDOW) ? rel - min(a.m.window - 1, 1 << 30) : -(1 << 30);
  if (PADDED) lo = max(lo, klo - kv0 - 4 * hf);

  // Score_mod, mask and running max of scores 4k .. 4k+3 (tile k / 4), in
  // the tile's mode.
  float mx = SOFTCAP ? INFINITY : -INFINITY;
  f32x16_t s[4];
  auto mask_chunk = [&](auto mode_c, int k) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_c)::value;
    const int t = k >> 2;
#pragma unroll
    for (int e = 4 * k; e < 4 * k + 4; ++e) {
      const int r = e & 15;
      if (MODE == kTileDead) {
        // Written here, in the dead tile's own path (a constant would be
        // materialised before the branch, on every path): -inf, or with the
        // soft-cap +inf in the reciprocal form.
        float dead;
        if (SOFTCAP)
          asm volatile("v_mov_b32 %0, 0x7f800000" : "=v"(dead));
        else
          asm volatile("v_mov_b32 %0, 0xff800000" : "=v"(dead));
        s[t][r] = dead;
        continue;
      }
      float x = s[t][r];
      if (SOFTCAP) x = softcap_recip(x, 2.0f * kLog2e * a.scale / a.softcap);
      if (MODE == kTileMixed) {
        const int c = ((r >> 2) << 3) + (r & 3);
        bool live = c <= hi - 32 * t;
        if (KIND == ATTN_MASK_SLIDING_WINDOW || PADDED) live &= c >= lo - 32 * t;
        // (Read unconditionally: the four ids of a register group are one
        // 16-byte LDS read.)
        if constexpr (KIND == ATTN_MASK_DOCUMENT) live &= kst.doc[t * 32 + acc_row(r, hf)] == dq;
        if (KIND == ATTN_MASK_CUSTOM) live &= (mw[t] >> (c + 4 * hf)) & 1u;
        x = live ? x : (SOFTCAP ? INFINITY : -INFINITY);
      }
      s[t][r] = x;
      mx = SOFTCAP ? fminf(mx, x) : fmaxf(mx, x);
    }
  };
  // Runs f with the mode of tile t as a compile-time constant (one scalar
  // branch per tile).
  auto with_mode = [&](int t, auto&& f) __attribute__((always_inline)) {
    if (!PARTIAL || tile_cls[t] == kTileLive)
      f(std::integral_constant<int, kTileLive>{});
    else if (tile_cls[t] == kTileDead)
      f(std::integral_constant<int, kTileDead>{});
    else
      f(std::integral_constant<int, kTileMixed>{});
  };

  // Phase Q. Tile t is complete after chunk 4t + 3; its scores are
  // processed in chunks 4t + 4 .. 4t + 7 (tile 3 after the phase).
  x8 kf[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) kf[j] = k_frag(j);
  sched_fence();
  auto q_chunk = [&](int j) __attribute__((always_inline)) {
    if (j + 4 < 16) kf[j + 4] = k_frag(j + 4);
    const int t = j >> 2, c = j & 3;
    if (!SKIP_DEAD || tile_cls[t] != kTileDead) s[t] = V::mma(kf[j], qop[c], c == 0 ? f32x16_t{} : s[t]);
  };
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    q_chunk(j);
    sched_fence();
  }
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    with_mode(t, [&](auto mode_c) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 4 * t + 4; j < 4 * t + 8; ++j) {
        q_chunk(j);
        mask_chunk(mode_c, j - 4);
        sched_fence();
      }
    });
  }
  x8 vf[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) vf[i] = v_frag(i);
  with_mode(3, [&](auto mode_c) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 12; k < 16; ++k) mask_chunk(mode_c, k);
  });
  // Without the soft-cap the max is over raw scores (scale > 0 keeps order);
  // with it, the smallest reciprocal term gives the largest capped score.
  const float cap2 = a.softcap * kLog2e;
  const float m_blk = SOFTCAP ? fmaf(-2.0f * cap2, half_min(mx), cap2) : half_max(mx) * c1;

  // Lazy rescale (wave-uniform branch).
  const bool grow = m_blk > m_ref + kRescaleLog2;
  // (Before a row's first live key, m_ref = -inf and the accumulators are
  // zero: nothing to rescale, as at every item's first block.)
  if (__ballot(grow && m_ref != -INFINITY) != 0) {
    const float alpha = grow ? fast_exp2(m_ref - m_blk) : 1.0f;
    l *= alpha;
#pragma unroll
    for (int te = 0; te < 2; ++te)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[te][r] *= alpha;
  }
  if (grow) m_ref = m_blk;
  const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;

  // Probabilities of scores 4k .. 4k+3 (group k / 2, entries 4(k % 2) ..),
  // rounded to T (nearest even) for P V; the normaliser sums the rounded
  // values.
  x8 pk[8];
  float psum[2] = {0.0f, 0.0f};
  auto prob_chunk = [&](int k) {
    const int g = k >> 1;
    if (SKIP_DEAD && tile_cls[g >> 1] == kTileDead) return;
#pragma unroll
    for (int u = (k & 1) * 4; u < (k & 1) * 4 + 4; u += 2) {
      const float x0 = s[g >> 1][(g & 1) * 8 + u], x1 = s[g >> 1][(g & 1) * 8 + u + 1];
      const float p0 = SOFTCAP ? fast_exp2(fmaf(x0, -2.0f * cap2, cap2 - m_use)) : fast_exp2(fmaf(x0, c1, -m_use));
      const float p1 = SOFTCAP ? fast_exp2(fmaf(x1, -2.0f * cap2, cap2 - m_use)) : fast_exp2(fmaf(x1, c1, -m_use));
      const typename V::x2 pr = {(T)p0, (T)p1};
      psum[(u >> 1) & 1] = V::add_pair(pr, psum[(u >> 1) & 1]);
      pk[g][u] = pr[0];
      pk[g][u + 1] = pr[1];
    }
  };

  // Phase P. Group g's probabilities are made in chunks 2g - 2 and 2g - 1
  // (group 0 before the phase) and used by MFMAs 2g and 2g + 1. The phase
  // runs at raised wave priority: it is bound by the vector unit, and when
  // the other wave on the SIMD is in its MFMA-bound phase Q, issuing this
  // wave's vector work first keeps both units busy.
  __builtin_amdgcn_s_setprio(1);
  prob_chunk(0);
  prob_chunk(1);
  sched_fence();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i + 4 < 16) vf[i + 4] = v_frag(i + 4);
    if (!SKIP_DEAD || tile_cls[i >> 2] != kTileDead) oacc[i & 1] = V::mma(vf[i], pk[i >> 1], oacc[i & 1]);
    if (i + 2 < 16) prob_chunk(i + 2);
    sched_fence();
  }
  dot_results_settle(psum[0], psum[1]);
  l += psum[0] + psum[1];
  __builtin_amdgcn_s_setprio(0);
}

// Workgroups are dispatched to the 8 XCDs in turn (workgroup i to XCD
// i mod 8), each XCD with its own L2. With grouped heads (query heads
// h G .. h G + G - 1 share K/V head h), batch*head index p of a launch
// whose B*H is a multiple of 8 is taken as (p mod 8) (B*H / 8) + p / 8, so
// the consecutive indices of one K/V head's query heads land on one XCD and
// read its K/V through one L2 (GQA causal 8192, 32 query / 8 K/V heads:
// -1.6%; S=16384: -4%). Without grouping the order stays as it is.
__device__ inline int xcd_head_order(int p, int BH, int G) {
  return (G > 1 && (BH & 7) == 0) ? (p & 7) * (BH >> 3) + (p >> 3) : p;
}

// One work item of the plan written by the mask builder (a 16-byte
// descriptor, one scalar load): query block qb, which of its k chunks of kv
// blocks the item visits, the block counts of qb and the item's first block.
struct WorkItem {
  int qb, chunk, k;
  int nfull, npart;  // full and partial kv blocks of qb
  int first_kb;      // kv block index of the item's first visited block
  bool split;        // the item is one of k > 1 chunks whose results are merged
  bool skip;         // no work (past the end of the plan, or a later chunk when
                     // splitting is off: then the first item visits every block)
};

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const i32x4_t* const_i32x4_ptr;

__device__ inline WorkItem work_item(const FwdArgs& a, int e) {
  const i32x4_t d = ((const_i32x4_ptr)(a.m.schedule + 4))[e];
  WorkItem w;
  w.skip = d[0] < 0;
  w.qb = d[0] & 0xFFFFF;
  w.chunk = (d[0] >> 20) & 3;
  w.k = ((d[0] >> 22) & 3) + 1;
  w.nfull = d[1];
  w.npart = d[2];
  w.first_kb = d[3];
  w.split = a.split && w.k > 1;
  w.skip = w.skip || (w.chunk > 0 && !w.split);
  if (w.skip) w.qb = w.chunk = w.nfull = w.npart = w.first_kb = 0;
  return w;
}

template <typename T, int KIND, bool SOFTCAP, bool PADDED, bool KVSPLIT>
__global__ __launch_bounds__(kThreads, 2) void fwd16_kernel(FwdArgs a) {
  using V = Vec<T>;
  using x8 = typename V::x8;
  using x4 = typename V::x4;
  constexpr bool BITS = KIND == ATTN_MASK_CUSTOM;
  __shared__ std::conditional_t<BITS, LdsBits, Lds> lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, hf = lane >> 5;
  const int BH = a.B * a.H;
  const int item = blockIdx.x;
  WorkItem wi;
  int b, h;
  if (KVSPLIT) {
    // Split-KV item (query block qb, chunk c of kv_split, batch b, K/V head
    // hk, query head h = hk * G + g). The batch*K/V-head index varies
    // fastest, so (with B*H_kv a multiple of 8) every item that reads one
    // K/V head lands on one XCD and shares its L2.
    const int G = a.kv_group, BHk = a.B * (a.H / G), k = a.kv_split;
    const int bk = item % BHk, rest = item / BHk;
    const int c = rest % k, rest2 = rest / k;
    const int g = rest2 % G;
    b = bk / (a.H / G);
    h = (bk % (a.H / G)) * G + g;
    wi.qb = rest2 / G;
    wi.chunk = c;
    wi.k = k;
    wi.nfull = ((const_i32_ptr)a.m.full_num)[wi.qb];
    wi.npart = ((const_i32_ptr)a.m.kv_num)[wi.qb];
    wi.split = true;
    wi.skip = false;
    wi.first_kb = 0;  // set below, once the item's range is known
  } else {
    wi = work_item(a, item / BH);
    if (wi.skip) return;
    const int pbh = xcd_head_order(item % BH, BH, a.kv_group);
    b = pbh / a.H;
    h = pbh % a.H;
  }
  const int qb = wi.qb;
  const int bh = b * a.H + h;

  const T* qg = static_cast<const T*>(a.q) + b * a.q_sb + h * a.q_sh;
  const int hk = h / a.kv_group;  // K/V head of query head h
  const T* kg = static_cast<const T*>(a.k) + b * a.k_sb + hk * a.k_sh;
  const T* vg = static_cast<const T*>(a.v) + b * a.v_sb + hk * a.v_sh;
  T* og = static_cast<T*>(a.o) + b * a.o_sb + h * a.o_sh;
  // Kept keys [klo, khi) of this batch entry (all of [0, S) without padding).
  int klo = 0, khi = a.S;
  if (PADDED) {
    if (a.key_start != nullptr) klo = min(max(((const_i32_ptr)a.key_start)[b], 0), a.S);
    if (a.key_end != nullptr) khi = max(min(((const_i32_ptr)a.key_end)[b], a.S), klo);
  }

  const int nfull = wi.nfull;
  const int npart = wi.npart;
  const int nblk = nfull + npart;
  const const_i32_ptr full_list = (const_i32_ptr)(a.m.full_idx + (int64_t)qb * a.m.nk);
  const const_i32_ptr part_list = (const_i32_ptr)(a.m.kv_idx + (int64_t)qb * a.m.nk);
  // First key of the n-th visited block: full blocks first, then partial.
  auto kv_start = [&](int n) { return (n < nfull ? full_list[n] : part_list[n - nfull]) * kBlock; };
  // This item visits blocks [m_begin, m_end) of that order: a split query
  // block's first chunk is its first C blocks (C from the plan), the second
  // the rest; split-KV chunk c of k takes blocks [c n / k, (c + 1) n / k).
  int m_begin, m_end;
  if (KVSPLIT) {
    m_begin = (int)((int64_t)wi.chunk * nblk / wi.k);
    m_end = (int)((int64_t)(wi.chunk + 1) * nblk / wi.k);
    if (m_end > m_begin) wi.first_kb = kv_start(m_begin) / kBlock;
  } else {
    const int split_len = a.m.schedule[1];
    m_begin = (wi.split && wi.chunk == 1) ? split_len : 0;
    m_end = (wi.split && wi.chunk == 0) ? split_len : nblk;
  }
  // Per-lane byte offsets of the tile copies (see issue_rows).
  const uint32_t k_off =
      (uint32_t)((lane >> 3) * a.k_sl * (int64_t)sizeof(T)) + (uint32_t)(((lane & 7) ^ (lane >> 3)) * 16);
  const uint32_t v_off = (uint32_t)((lane >> 3) * a.v_sl * (int64_t)sizeof(T)) +
                         (uint32_t)(((lane & 7) ^ (((lane >> 3) & 3) << 1)) * 16);

  // Block m's K and V tiles live in stage (m - m_begin) % 2. The index of
  // the block after the next one is loaded a block ahead, so no block waits
  // on a scalar load before issuing its copies.
  int kv_next = 0;   // first key of the next block to copy
  int kv_after = 0;  // first key of the block after it
  if (m_end > m_begin) {
    kv_next = wi.first_kb * kBlock;
    if (m_begin + 1 < m_end) kv_after = kv_start(m_begin + 1);
    issue_k<T, KIND>(kg, a.k_sl, k_off, a.m.doc, kv_next, a.S, lds.k[0], wave, lane);
    issue_rows<T, true>(vg, a.v_sl, v_off, kv_next, a.S, lds.v[0].v, wave, lane);
    if constexpr (BITS)
      issue_bits(a.m.bits, a.m.bits_w, qb * kBlock + wave * 32, a.L, kv_next / kBlock, lds.bits[0], wave, lane);
  }

  const int row0 = qb * kBlock + wave * 32;  // this wave's first query row
  const int qi = row0 + lq;                   // this lane's query row
  x8 qop[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (qi < a.L)
      qop[c] = *reinterpret_cast<const x8*>(qg + (int64_t)qi * a.q_sl + c * 16 + hf * 8);
    else
      qop[c] = x8{};
  }
  const int32_t dq = (KIND == ATTN_MASK_DOCUMENT && qi < a.L) ? a.m.doc[qi] : -1;
  // Q, dq and tile 0 have landed: no load the compiler tracks is still in
  // flight inside the loop, so it adds no wait there (such a wait would also
  // drain the next tile's copies, which share the in-order counter).
  wait_vm_zero();

  // Per-lane LDS read addresses of each stage.
  const LanePtrs lp = make_lane_ptrs(lds, lane);

  f32x16_t oacc[2];
#pragma unroll
  for (int te = 0; te < 2; ++te)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[te][r] = 0.0f;
  float m_ref = -INFINITY, l = 0.0f;

  // Two stages and one barrier per block: once every wave's copies of block
  // m have landed and every wave has finished block m-1, the copies of block
  // m+1 go into the stage block m-1 used, and block m is computed. Full and
  // partial blocks run in separate loops, so each loop body has a single
  // definition of the accumulators and they stay in place.
  auto block = [&](auto partial_c, int m) __attribute__((always_inline)) {
    constexpr bool PARTIAL = decltype(partial_c)::value;
    const int par = (m - m_begin) & 1;
    lds_u8 kp[4], vp[2];
    // Computed once per block; the empty asm keeps the compiler from
    // recomputing each address before every read instead of holding it.
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kp[c] = lp.k[c] + par * (int)sizeof(KStage);
      asm volatile("" : "+v"(kp[c]));
    }
#pragma unroll
    for (int te = 0; te < 2; ++te) {
      vp[te] = lp.v[te] + par * (int)sizeof(VStage);
      asm volatile("" : "+v"(vp[te]));
    }
    const int kv0 = kv_next;
    wait_vm_zero();    // this wave's copies of block m
    wait_lgkm_zero();  // this wave's reads of block m-1
    barrier_only();
    if (m + 1 < m_end) {
      kv_next = kv_after;
      issue_k<T, KIND>(kg, a.k_sl, k_off, a.m.doc, kv_next, a.S, lds.k[1 - par], wave, lane);
      issue_rows<T, true>(vg, a.v_sl, v_off, kv_next, a.S, lds.v[1 - par].v, wave, lane);
      if constexpr (BITS)
        issue_bits(a.m.bits, a.m.bits_w, qb * kBlock + wave * 32, a.L, kv_next / kBlock, lds.bits[1 - par],
                   wave, lane);
      if (m + 2 < m_end) kv_after = kv_start(m + 2);
    }
    const uint32_t* mb = nullptr;
    if constexpr (BITS) mb = lds.bits[par];
    if (PADDED) {
      // A block with no kept key is skipped; a full block that a padding
      // boundary cuts runs the per-tile pair tests of a partial block.
      if (kv0 + kBlock <= klo || kv0 >= khi) return;
      if (!PARTIAL && (kv0 < klo || kv0 + kBlock > khi)) {
        fwd_block<T, KIND, SOFTCAP, true, true>(lds.k[par], kp, vp, qop, oacc, m_ref, l, qi, row0, kv0,
                                                lane, a, dq, klo, khi, mb);
        return;
      }
    }
    fwd_block<T, KIND, SOFTCAP, PARTIAL, PADDED>(lds.k[par], kp, vp, qop, oacc, m_ref, l, qi, row0, kv0,
                                                 lane, a, dq, klo, khi, mb);
  };
  int m = m_begin;
  for (; m < min(m_end, nfull); ++m) block(std::false_type{}, m);
  for (; m < m_end; ++m) block(std::true_type{}, m);

  float lt = half_sum(l);  // the row's sum of (rounded) probabilities

  if (KVSPLIT) {
    // Split-KV: leave this chunk's unnormalised O (row-major [row][64]), its
    // reference max and its sum for the query rows in range; the merge kernel,
    // launched next on the stream, combines the chunks.
    if (qi < a.L) {
      float* slot = a.partials + (((int64_t)qb * a.kv_split + wi.chunk) * BH + bh) * kSlotFloats;
      float* orow = slot + (wave * 32 + lq) * 64;
#pragma unroll
      for (int te = 0; te < 2; ++te)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          float4 o4;
          o4.x = oacc[te][r4 * 4 + 0];
          o4.y = oacc[te][r4 * 4 + 1];
          o4.z = oacc[te][r4 * 4 + 2];
          o4.w = oacc[te][r4 * 4 + 3];
          *reinterpret_cast<float4*>(orow + te * 32 + r4 * 8 + hf * 4) = o4;
        }
      if (hf == 0) {
        slot[4 * 32 * 64 + wave * 32 + lq] = m_ref;
        slot[4 * 32 * 64 + kBlock + wave * 32 + lq] = lt;
      }
    }
    return;
  }

  if (wi.split) {
    // The two chunks of a split query block each take a ticket when they
    // finish. The first to finish leaves its partial result (O^T, m, l) in
    // the query block's slot and then marks it written; the second waits for
    // that mark and merges both, in chunk order, so the result does not
    // depend on which finished first and only one partial is ever written.
    // Counter: first ticket 0 -> 1, second ticket -> 2 (or 3 -> 4), the
    // first's mark adds 2: both finished and the partial written = 4. The
    // partial is written and read with device-scope (sc1) accesses, and its
    // writes have completed before the mark is added, so the chunks may run
    // on different XCDs without device-scope fences (which would write back
    // and invalidate the XCD's whole L2, K/V tiles of other workgroups
    // included). The second chunk waits only on a chunk that has already
    // taken its ticket, that is, one that is running and writes without
    // waiting on anything.
    const int64_t bhn = (int64_t)a.B * a.H;
    float* slot = a.partials + ((int64_t)qb * bhn + bh) * kSlotFloats;
    auto put = [](float* p, float x) { __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    auto get = [](float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    __shared__ int ticket;
    int32_t* counter = a.counters + (int64_t)qb * bhn + bh;
    if (tid == 0) ticket = atomicAdd(counter, 1);
    __syncthreads();
    if (ticket == 0) {
#pragma unroll
      for (int te = 0; te < 2; ++te)
#pragma unroll
        for (int r = 0; r < 16; ++r) put(slot + (wave * 32 + te * 16 + r) * 64 + lane, oacc[te][r]);
      if (hf == 0) {
        put(slot + 4 * 32 * 64 + wave * 32 + lq, m_ref);
        put(slot + 4 * 32 * 64 + kBlock + wave * 32 + lq, lt);
      }
      wait_vm_zero();  // this wave's partial writes have completed
      __syncthreads();
      if (tid == 0) atomicAdd(counter, 2);
      return;
    }
    if (tid == 0) {
      // A ticket of 3 is the first chunk's ticket plus its mark: the partial
      // is already there. Otherwise wait for the mark (bounded: the first
      // chunk marks its partial within microseconds).
      if (ticket != 3)
        for (int spin = 0; spin < (1 << 24); ++spin) {
          if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 4) break;
          __builtin_amdgcn_s_sleep(1);
        }
      __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
    }
    __syncthreads();
    // Merge in chunk order: weights w_c = 2^(m_c - max m), O = w_0 O_0 +
    // w_1 O_1, l = w_0 l_0 + w_1 l_1.
    const float m_o = get(slot + 4 * 32 * 64 + wave * 32 + lq);
    const float l_o = get(slot + 4 * 32 * 64 + kBlock + wave * 32 + lq);
    const float m0 = wi.chunk == 0 ? m_ref : m_o, m1 = wi.chunk == 0 ? m_o : m_ref;
    const float l0 = wi.chunk == 0 ? lt : l_o, l1 = wi.chunk == 0 ? l_o : lt;
    const float m_new = fmaxf(m0, m1);
    const float w0 = (m0 == -INFINITY) ? 0.0f : fast_exp2(m0 - m_new);
    const float w1 = (m1 == -INFINITY) ? 0.0f : fast_exp2(m1 - m_new);
#pragma unroll
    for (int te = 0; te < 2; ++te)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float ov = get(slot + (wave * 32 + te * 16 + r) * 64 + lane);
        const float o0 = wi.chunk == 0 ? oacc[te][r] : ov, o1 = wi.chunk == 0 ? ov : oacc[te][r];
        oacc[te][r] = fmaf(w1, o1, w0 * o0);
      }
    lt = fmaf(w1, l1, w0 * l0);
    m_ref = m_new;
  }

  // Epilogue: O = O^T / l (0 for a row without live keys), lse = ln(sum exp).
  const float inv = (lt > 0.0f) ? 1.0f / lt : 0.0f;
  if (qi < a.L) {
#pragma unroll
    for (int te = 0; te < 2; ++te) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int e0 = te * 32 + r4 * 8 + hf * 4;
        x4 outv;
#pragma unroll
        for (int u = 0; u < 4; ++u) outv[u] = (T)(oacc[te][r4 * 4 + u] * inv);
        *reinterpret_cast<x4*>(og + (int64_t)qi * a.o_sl + e0) = outv;
      }
    }
    if (a.lse != nullptr && hf == 0)
      a.lse[(int64_t)bh * a.L + qi] = (lt > 0.0f) ? (m_ref + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Chained work items (sliding windows): the items of a window are short (a
// few kv blocks each) and many, so a workgroup that owned one item would pay
// the item's start-up latency (descriptor, Q rows, first K/V tiles) and its
// output stores with nothing to overlap them. Here each resident workgroup
// owns one batch*head and walks the plan entries r0, r0 + R, r0 + 2R, ... of
// it (R = grid size / (B*H), so the R workgroups of a head run R consecutive
// query blocks at a time and share their K/V tiles in L2; with B*H a multiple
// of 8 all of a head's workgroups sit on one XCD). The two-stage block
// pipeline runs across item boundaries: during an item's last block the next
// item's first K/V tiles and its Q rows are copied into LDS, and an item's
// output is stored only after the next item's first barrier, so neither the
// loads nor the stores of one item wait behind the other.
// ---------------------------------------------------------------------------
template <typename T, int KIND, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 2) void fwd16_chain_kernel(FwdArgs a) {
  using V = Vec<T>;
  using x8 = typename V::x8;
  using x4 = typename V::x4;
  __shared__ LdsChain lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, hf = lane >> 5;
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int b = bh / a.H, h = bh % a.H;
  const int rstep = gridDim.x / BH;
  const int nitems = ((const_i32_ptr)a.m.schedule)[0];

  const T* qg = static_cast<const T*>(a.q) + b * a.q_sb + h * a.q_sh;
  const int hk = h / a.kv_group;
  const T* kg = static_cast<const T*>(a.k) + b * a.k_sb + hk * a.k_sh;
  const T* vg = static_cast<const T*>(a.v) + b * a.v_sb + hk * a.v_sh;
  T* og = static_cast<T*>(a.o) + b * a.o_sb + h * a.o_sh;
  const uint32_t k_off =
      (uint32_t)((lane >> 3) * a.k_sl * (int64_t)sizeof(T)) + (uint32_t)(((lane & 7) ^ (lane >> 3)) * 16);
  const uint32_t v_off = (uint32_t)((lane >> 3) * a.v_sl * (int64_t)sizeof(T)) +
                         (uint32_t)(((lane & 7) ^ (((lane >> 3) & 3) << 1)) * 16);
  const LanePtrs lp = make_lane_ptrs(lds, lane);

  // The next plan entry with work (a later chunk of a split query block has
  // none: splitting is off here, so a first chunk visits every block).
  auto next_item = [&](int& r, WorkItem& w) {
    for (; r < nitems; r += rstep) {
      w = work_item(a, r);
      if (!w.skip) break;
    }
  };
  int r = blockIdx.x / BH;
  WorkItem wi;
  next_item(r, wi);
  if (r >= nitems) return;

  // Q rows of query block qb: each wave copies its 32 rows (4 KiB, rows past
  // L clamped to the last row) into the Q stage by LDS DMA, like the K/V
  // tiles, and reads its operands from there once the copies have landed
  // (zero past L). Loads into registers here would be tracked by the
  // compiler's wait insertion, which does not see the asm copies: a wait it
  // adds for such a load also waits for every copy issued after it.
  auto issue_q = [&](int qb) {
    const uint32_t lds0 = lds_offset(lds.q) + (uint32_t)wave * 4096u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = min(qb * kBlock + wave * 32 + 8 * i + (lane >> 3), a.L - 1);
      lds_copy16(qg + (int64_t)row * a.q_sl + (lane & 7) * 8, lds0 + 1024u * i);
    }
  };
  auto read_q = [&](int qb, x8 (&dst)[4]) {
    typedef __attribute__((address_space(3))) const x8 lds_x8;
    const int qi = qb * kBlock + wave * 32 + lq;
    const lds_u8 rowp = (lds_u8)lds.q + (wave * 32 + lq) * 128;
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[c] = (qi < a.L) ? *reinterpret_cast<const lds_x8*>(rowp + c * 32 + hf * 16) : x8{};
  };
  auto issue_block = [&](int kv0, int stage) {
    issue_rows<T, false>(kg, a.k_sl, k_off, kv0, a.S, lds.k[stage].k, wave, lane);
    issue_rows<T, true>(vg, a.v_sl, v_off, kv0, a.S, lds.v[stage].v, wave, lane);
  };
  // First key of visited block n of item w (full blocks first, then partial).
  auto kv_start = [&](const WorkItem& w, int n) {
    const const_i32_ptr fl = (const_i32_ptr)(a.m.full_idx + (int64_t)w.qb * a.m.nk);
    const const_i32_ptr pl = (const_i32_ptr)(a.m.kv_idx + (int64_t)w.qb * a.m.nk);
    return (n < w.nfull ? fl[n] : pl[n - w.nfull]) * kBlock;
  };

  x8 qop[4];
  issue_q(wi.qb);
  int kv_next = wi.first_kb * kBlock;
  issue_block(kv_next, 0);
  wait_vm_zero();

  // The previous item's output, held until the next item's first barrier.
  x4 ohold[2][4];
  float lse_hold = 0.0f;
  int prev_qi = -1;  // this lane's row of the held output (-1: none)
  auto flush_held = [&]() {
    if (prev_qi >= 0 && prev_qi < a.L) {
#pragma unroll
      for (int te = 0; te < 2; ++te)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<x4*>(og + (int64_t)prev_qi * a.o_sl + te * 32 + r4 * 8 + hf * 4) = ohold[te][r4];
      if (a.lse != nullptr && hf == 0) a.lse[(int64_t)bh * a.L + prev_qi] = lse_hold;
    }
    prev_qi = -1;
  };

  int par = 0;  // stage of the current block
  while (true) {
    const int qb = wi.qb;
    const int nfull = wi.nfull, nblk = wi.nfull + wi.npart;
    const int row0 = qb * kBlock + wave * 32;
    const int qi = row0 + lq;
    // The entry after this one, looked up now so its descriptor has landed
    // by this item's last block.
    int r_n = r + rstep;
    WorkItem wn = wi;
    next_item(r_n, wn);
    const bool has_next = r_n < nitems;
    // First key of the block after the next one (a block ahead, as in the
    // one-item kernel, so no copy waits on a scalar load).
    int kv_after = nblk > 1 ? kv_start(wi, 1) : (has_next ? wn.first_kb * kBlock : 0);
    const int32_t dq = (KIND == ATTN_MASK_DOCUMENT && qi < a.L) ? a.m.doc[qi] : -1;

    f32x16_t oacc[2];
#pragma unroll
    for (int te = 0; te < 2; ++te)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) oacc[te][rr] = 0.0f;
    float m_ref = -INFINITY, l = 0.0f;

    auto block = [&](auto partial_c, int m) __attribute__((always_inline)) {
      constexpr bool PARTIAL = decltype(partial_c)::value;
      lds_u8 kp[4], vp[2];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        kp[c] = lp.k[c] + par * (int)sizeof(lds.k[0]);
        asm volatile("" : "+v"(kp[c]));
      }
#pragma unroll
      for (int te = 0; te < 2; ++te) {
        vp[te] = lp.v[te] + par * (int)sizeof(lds.v[0]);
        asm volatile("" : "+v"(vp[te]));
      }
      const int kv0 = kv_next;
      wait_vm_zero();    // this wave's copies of block m (and Q rows, older stores)
      wait_lgkm_zero();  // this wave's reads of the previous block
      barrier_only();
      if (m == 0) {
        // The previous item's output: its stores are issued now and finish
        // during this block. This item's Q rows (this wave's own copies).
        flush_held();
        read_q(qb, qop);
      }
      if (m + 1 < nblk) {
        kv_next = kv_after;
        issue_block(kv_next, 1 - par);
        if (m + 2 < nblk)
          kv_after = kv_start(wi, m + 2);
        else if (has_next)
          kv_after = wn.first_kb * kBlock;
      } else if (has_next) {
        // Last block: the next item's first tiles and Q rows (the Q stage is
        // rewritten once this wave's reads of it have completed).
        kv_next = kv_after;
        issue_block(kv_next, 1 - par);
        if (m == 0) wait_lgkm_zero();
        issue_q(wn.qb);
      }
      fwd_block<T, KIND, SOFTCAP, PARTIAL, false>(lds.k[par], kp, vp, qop, oacc, m_ref, l, qi, row0, kv0, lane,
                                                  a, dq, 0, a.S, nullptr);
      par ^= 1;
    };
    int m = 0;
    for (; m < nfull; ++m) block(std::false_type{}, m);
    for (; m < nblk; ++m) block(std::true_type{}, m);
    if (nblk == 0) {
      // No live block (rows without keys): the tiles copied for this item
      // go unused; the next item's first tiles replace them in the same
      // stage once this wave's own copies have landed (each wave writes only
      // its quarter of a stage).
      flush_held();
      wait_vm_zero();
      if (has_next) {
        kv_next = wn.first_kb * kBlock;
        issue_block(kv_next, par);
        issue_q(wn.qb);
      }
    }

    // Epilogue: O = O^T / l (0 for a row without live keys), held in
    // registers until the next item's first barrier (or stored now).
    const float lt = half_sum(l);
    const float inv = (lt > 0.0f) ? 1.0f / lt : 0.0f;
#pragma unroll
    for (int te = 0; te < 2; ++te)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
        for (int u = 0; u < 4; ++u) ohold[te][r4][u] = (T)(oacc[te][r4 * 4 + u] * inv);
    lse_hold = (lt > 0.0f) ? (m_ref + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    prev_qi = qi;
    if (!has_next) break;
    r = r_n;
    wi = wn;
  }
  flush_held();
}

// ---------------------------------------------------------------------------
// fp32 kernel: same structure with v_mfma_f32_32x32x2_f32 (one element of the
// contraction per lane and step), probabilities kept in fp32.
// ---------------------------------------------------------------------------
constexpr int kF32RowStride = 68;  // floats per LDS row (64 + 4 padding)

template <int KIND, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 2) void fwd32_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) float k_lds[kBlock * kF32RowStride];
  __shared__ __attribute__((aligned(16))) float v_lds[kBlock * kF32RowStride];
  __shared__ int32_t doc_k[kBlock];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 31, hf = lane >> 5;
  const int BH = a.B * a.H;
  const int item = blockIdx.x;
  // fp32 never splits (no workspace): a first item visits every block.
  const WorkItem wi = work_item(a, item / BH);
  if (wi.skip) return;
  const int qb = wi.qb;
  const int bh = item % BH;
  const int b = bh / a.H, h = bh % a.H;

  const float* qg = static_cast<const float*>(a.q) + b * a.q_sb + h * a.q_sh;
  const int hk = h / a.kv_group;  // K/V head of query head h
  const float* kg = static_cast<const float*>(a.k) + b * a.k_sb + hk * a.k_sh;
  const float* vg = static_cast<const float*>(a.v) + b * a.v_sb + hk * a.v_sh;
  float* og = static_cast<float*>(a.o) + b * a.o_sb + h * a.o_sh;
  // Kept keys [klo, khi) of this batch entry (all of [0, S) without padding).
  int klo = 0, khi = a.S;
  if (a.key_start != nullptr) klo = min(max(a.key_start[b], 0), a.S);
  if (a.key_end != nullptr) khi = max(min(a.key_end[b], a.S), klo);

  const int qi = qb * kBlock + wave * 32 + lq;
  // Contraction step j of lane half hf covers head dim e = 32*hf + j.
  float qv[32];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (qi < a.L) x = *reinterpret_cast<const float4*>(qg + (int64_t)qi * a.q_sl + hf * 32 + c * 4);
    qv[4 * c + 0] = x.x;
    qv[4 * c + 1] = x.y;
    qv[4 * c + 2] = x.z;
    qv[4 * c + 3] = x.w;
  }
  const int32_t dq = (KIND == ATTN_MASK_DOCUMENT && qi < a.L) ? a.m.doc[qi] : -1;

  f32x16_t oacc[2];
#pragma unroll
  for (int te = 0; te < 2; ++te)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[te][r] = 0.0f;
  RowState st{-INFINITY, 0.0f};

  const int nfull = a.m.full_num[qb];
  const int npart = a.m.kv_num[qb];
  const int32_t* full_list = a.m.full_idx + (int64_t)qb * a.m.nk;
  const int32_t* part_list = a.m.kv_idx + (int64_t)qb * a.m.nk;

  for (int n = 0; n < nfull + npart; ++n) {
    const int kb = n >= nfull ? part_list[n - nfull] : full_list[n];
    const int kv0 = kb * kBlock;
    // Skip blocks with no kept key; a padding boundary inside a full block
    // makes it partial.
    if (kv0 + kBlock <= klo || kv0 >= khi) continue;
    const bool partial = n >= nfull || kv0 < klo || kv0 + kBlock > khi;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int cidx = tid + u * kThreads;  // 2048 float4 chunks per tile
      const int row = cidx >> 4, ch = cidx & 15;
      float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
      if (kv0 + row < a.S) {
        kx = *reinterpret_cast<const float4*>(kg + (int64_t)(kv0 + row) * a.k_sl + ch * 4);
        vx = *reinterpret_cast<const float4*>(vg + (int64_t)(kv0 + row) * a.v_sl + ch * 4);
      }
      *reinterpret_cast<float4*>(k_lds + row * kF32RowStride + ch * 4) = kx;
      *reinterpret_cast<float4*>(v_lds + row * kF32RowStride + ch * 4) = vx;
    }
    if (KIND == ATTN_MASK_DOCUMENT && partial && tid < kBlock)
      doc_k[tid] = (kv0 + tid < a.S) ? a.m.doc[kv0 + tid] : -1;
    // CUSTOM: this lane's row's mask words of the block
    uint4 mw = make_uint4(0u, 0u, 0u, 0u);
    if (KIND == ATTN_MASK_CUSTOM && partial)
      mw = *reinterpret_cast<const uint4*>(a.m.bits + (int64_t)min(qi, a.L - 1) * a.m.bits_w + 4 * kb);
    __syncthreads();

    f32x16_t s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = 0.0f;
      const float* krow = k_lds + (t * 32 + lq) * kF32RowStride + hf * 32;
#pragma unroll
      for (int j = 0; j < 32; ++j) s[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[j], qv[j], s[t], 0, 0, 0);
    }

    float alpha;
    if (partial)
      alpha = softmax_tiles<KIND, true, SOFTCAP>(s, st, qi, kv0, hf, a, dq, doc_k, klo, khi, mw);
    else
      alpha = softmax_tiles<KIND, false, SOFTCAP>(s, st, qi, kv0, hf, a, dq, doc_k, klo, khi, mw);

    float psum = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) psum += s[t][r];
    st.l = st.l * alpha + psum;
#pragma unroll
    for (int te = 0; te < 2; ++te)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[te][r] *= alpha;

    // O^T += V^T P^T: step (t, r) pairs lane half 0's key acc_row(r,0) with
    // lane half 1's key acc_row(r,1) of tile t; A = V[key][e], B = p.
#pragma unroll
    for (int te = 0; te < 2; ++te) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float va = v_lds[(t * 32 + acc_row(r, hf)) * kF32RowStride + te * 32 + lq];
          oacc[te] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, s[t][r], oacc[te], 0, 0, 0);
        }
      }
    }
  }

  const float l = half_sum(st.l);
  const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
  if (qi < a.L) {
#pragma unroll
    for (int te = 0; te < 2; ++te) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int e0 = te * 32 + r4 * 8 + hf * 4;
        float4 outv = make_float4(oacc[te][r4 * 4 + 0] * inv, oacc[te][r4 * 4 + 1] * inv,
                                  oacc[te][r4 * 4 + 2] * inv, oacc[te][r4 * 4 + 3] * inv);
        *reinterpret_cast<float4*>(og + (int64_t)qi * a.o_sl + e0) = outv;
      }
    }
    if (a.lse != nullptr && hf == 0)
      a.lse[(int64_t)bh * a.L + qi] = (l > 0.0f) ? (st.m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
  }
}

// Merges of one output row over the k <= kKvSplitMax chunks of a split visit
// list. Chunk c's partial result sits at slot0 + c * cstride: the row's
// unnormalised O (64 floats) at o_off, its max (log2 units) at m_off and its
// sum at l_off. With w_c = 2^(m_c - max m) (0 for a chunk without live keys),
// O = sum w_c O_c / sum w_c l_c (0 when the sum is 0) and lse = (max m + log2
// sum w_c l_c) ln 2, the sums taken in chunk order, each product rounded
// before it is added. Both forms below give the same bits.
static_assert(kKvSplitMax <= 64, "four chunks per lane in merge_row");
constexpr int kMergeRows = kThreads / 16;  // output rows per merge_row workgroup (16 lanes each)

// Sixteen lanes per row, four rows per wave (the split-KV merge: many rows, a
// few chunks each): lane e of a row's group holds head dims 4e .. 4e + 3 and
// reads them with one 16-byte load per chunk; lane c reads the m and l of
// chunks c, c + 16, c + 32 and c + 48 in the same round as the O values of the
// first 16 chunks (later ones 16 at a time). The weights reach the group's
// lanes by shuffles; no fused multiply-adds are formed.
template <typename T>
__device__ inline void merge_row(const float* slot0, int64_t cstride, int o_off, int m_off, int l_off, int k,
                                 int lane, T* out, float* lse) {
#pragma clang fp contract(off)
  const int e = lane & 15, base = lane & ~15;
  float4 o[16];
  auto load_o = [&](int c0) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      o[j] = (c0 + j < k) ? *reinterpret_cast<const float4*>(slot0 + (int64_t)(c0 + j) * cstride + o_off + 4 * e)
                          : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  };
  load_o(0);
  float mc[4], lc[4];
  float mmax = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int c = e + 16 * t;
    mc[t] = c < k ? slot0[(int64_t)c * cstride + m_off] : -INFINITY;
    lc[t] = c < k ? slot0[(int64_t)c * cstride + l_off] : 0.0f;
    mmax = fmaxf(mmax, mc[t]);
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, off));
  float wc[4], wlc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    wc[t] = (mc[t] == -INFINITY) ? 0.0f : fast_exp2(mc[t] - mmax);
    wlc[t] = wc[t] * lc[t];
  }
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float lsum = 0.0f;
  for (int c0 = 0; c0 < k; c0 += 16) {
    if (c0 > 0) load_o(c0);
    const int t = c0 >> 4;
    const float wt = t == 0 ? wc[0] : t == 1 ? wc[1] : t == 2 ? wc[2] : wc[3];
    const float wlt = t == 0 ? wlc[0] : t == 1 ? wlc[1] : t == 2 ? wlc[2] : wlc[3];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (c0 + j < k) {
        const float w = __shfl(wt, base + j);
        const float wl = __shfl(wlt, base + j);
        acc.x = acc.x + w * o[j].x;
        acc.y = acc.y + w * o[j].y;
        acc.z = acc.z + w * o[j].z;
        acc.w = acc.w + w * o[j].w;
        lsum = lsum + wl;
      }
    }
  }
  const float inv = (lsum > 0.0f) ? 1.0f / lsum : 0.0f;
  typename Vec<T>::x4 ov;
  ov[0] = (T)(acc.x * inv);
  ov[1] = (T)(acc.y * inv);
  ov[2] = (T)(acc.z * inv);
  ov[3] = (T)(acc.w * inv);
  *reinterpret_cast<typename Vec<T>::x4*>(out + 4 * e) = ov;
  if (lse != nullptr && e == 0) *lse = (lsum > 0.0f) ? (mmax + __builtin_amdgcn_logf(lsum)) * kLn2 : -INFINITY;
}

// One workgroup per row (the packed decode merge: few rows, more chunks):
// thread t takes chunk t / 4 and head dims 16 (t % 4) .. +15, so every load
// is in flight at once, and the products and sums go through LDS.
template <typename T>
__device__ inline void merge_row_block(const float* slot0, int64_t cstride, int o_off, int m_off, int l_off, int k,
                                 T* out, float* lse) {
  static_assert(kThreads == 4 * kKvSplitMax, "one thread per (chunk, quarter row)");
  __shared__ float s_m[kKvSplitMax], s_wl[kKvSplitMax];
  __shared__ float s_o[kKvSplitMax][kHeadDim + 4];
  const int t = threadIdx.x, c = t >> 2, e0 = (t & 3) * 16;
  float m = -INFINITY, lc = 0.0f;
  float4 o[4];
  if (c < k) {
    const float* sl = slot0 + c * cstride;
    m = sl[m_off];
    lc = sl[l_off];
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = *reinterpret_cast<const float4*>(sl + o_off + e0 + 4 * u);
    if ((t & 3) == 0) s_m[c] = m;
  }
  __syncthreads();
  float mmax = -INFINITY;
  for (int cc = 0; cc < k; ++cc) mmax = fmaxf(mmax, s_m[cc]);
  if (c < k) {
    const float w = (m == -INFINITY) ? 0.0f : fast_exp2(m - mmax);
    if ((t & 3) == 0) s_wl[c] = w * lc;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      s_o[c][e0 + 4 * u + 0] = w * o[u].x;
      s_o[c][e0 + 4 * u + 1] = w * o[u].y;
      s_o[c][e0 + 4 * u + 2] = w * o[u].z;
      s_o[c][e0 + 4 * u + 3] = w * o[u].w;
    }
  }
  __syncthreads();
  if (t < kHeadDim) {
    float acc = 0.0f, lsum = 0.0f;
    for (int cc = 0; cc < k; ++cc) {
      acc += s_o[cc][t];
      lsum += s_wl[cc];
    }
    const float inv = (lsum > 0.0f) ? 1.0f / lsum : 0.0f;
    out[t] = (T)(acc * inv);
    if (lse != nullptr && t == 0)
      *lse = (lsum > 0.0f) ? (mmax + __builtin_amdgcn_logf(lsum)) * kLn2 : -INFINITY;
  }
}

// Merge of split-KV chunks: sixteen lanes per output row, rows ordered query
// row first, then batch*head, so a workgroup reads neighbouring rows of the
// same slots; slots are [qb][chunk][B*H].
template <typename T>
__global__ __launch_bounds__(kThreads) void kv_merge_kernel(FwdArgs a) {
  const int64_t gr = (int64_t)blockIdx.x * kMergeRows + (threadIdx.x >> 4);
  const int lane = threadIdx.x & 63;
  const int BH = a.B * a.H;
  if (gr >= (int64_t)BH * a.L) return;
  const int bh = (int)(gr / a.L), qi = (int)(gr % a.L);
  const int qb = qi / kBlock, row = qi % kBlock;
  const int b = bh / a.H, h = bh % a.H;
  const int k = a.kv_split;
  const float* slot0 = a.partials + ((int64_t)qb * k * BH + bh) * kSlotFloats;
  merge_row<T>(slot0, (int64_t)BH * kSlotFloats, row * kHeadDim, 4 * 32 * 64 + row, 4 * 32 * 64 + kBlock + row, k,
               lane, static_cast<T*>(a.o) + b * a.o_sb + h * a.o_sh + (int64_t)qi * a.o_sl,
               a.lse == nullptr ? nullptr : a.lse + (int64_t)bh * a.L + qi);
}

// ---------------------------------------------------------------------------
// Packed-row kernel: few query rows per K/V head (decode, short queries)
// ---------------------------------------------------------------------------
// When the L queries of the G query heads that share one K/V head number at
// most 32 rows, they fill the N side of one 32 x 32 MFMA tile: packed row
// r = g L + l (query head hk G + g, query l). A work item is one (batch, K/V
// head, chunk of the visit list), so K and V are read once per K/V head and
// no MFMA column goes to rows past L, as it would in a 128-row query tile.
// Each wave takes its own 32 keys of every 128-key block (keys 32w .. 32w+31),
// copies exactly those K and V rows into its part of each LDS stage and keeps
// its own running max and sum: inside the loop the waves never wait on each
// other, and each keeps kPackStages - 1 blocks of copies in flight. At the
// end the four waves' (max, sum, O) combine through LDS: into the output when
// the item holds the whole visit list, else into the item's partial slot,
// which packed_merge_kernel combines over the chunks.
constexpr int kPackStages = 2;

template <int NS, bool BITS>
struct alignas(16) PackLds {
  KStage k[NS];
  VStage v[NS];
  uint8_t q[kPackRows * 128];  // the packed rows' Q, row-major
  int32_t doc_q[kPackRows];    // document id of each packed row's query
  // CUSTOM: per stage and wave, each packed row's mask word of the wave's keys
  uint32_t bits[BITS ? NS : 1][4][kPackRows];
};
// Row stride (floats) of each wave's O in the combine area: 4 floats of
// padding spread the rows over the LDS banks.
constexpr int kPackORow = kHeadDim + 4;
static_assert(sizeof(float) * 4 * kPackRows * (kPackORow + 2) <=
                  (sizeof(KStage) + sizeof(VStage)) * kPackStages,
              "the combine area fits in the stages");

template <typename T, int KIND, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 2) void packed_kernel(FwdArgs a) {
  using V = Vec<T>;
  using x8 = typename V::x8;
  typedef __attribute__((address_space(3))) const x8 lds_x8;
  constexpr int NS = kPackStages;
  constexpr bool BITS = KIND == ATTN_MASK_CUSTOM;
  // vector memory operations one wave issues per block: 4 K, 4 V copies (and
  // the keys' document ids, or the rows' mask words)
  constexpr int kPerBlock = (KIND == ATTN_MASK_DOCUMENT || BITS) ? 9 : 8;
  static_assert((NS - 1) * kPerBlock < 64, "copies in flight fit vmcnt");
  __shared__ PackLds<NS, BITS> lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, hf = lane >> 5;
  const int G = a.kv_group, Hk = a.H / G, k = a.pack_split;
  const int R = a.L * G;  // packed rows in use (<= 32)
  const int bk = blockIdx.x % (a.B * Hk), chunk = blockIdx.x / (a.B * Hk);
  const int b = bk / Hk, hk = bk % Hk;
  const float c1 = a.scale * kLog2e;

  const T* kg = static_cast<const T*>(a.k) + b * a.k_sb + hk * a.k_sh;
  const T* vg = static_cast<const T*>(a.v) + b * a.v_sb + hk * a.v_sh;
  // Kept keys [klo, khi) of this batch entry (all of [0, S) without padding).
  int klo = 0, khi = a.S;
  if (a.key_start != nullptr) klo = min(max(((const_i32_ptr)a.key_start)[b], 0), a.S);
  if (a.key_end != nullptr) khi = max(min(((const_i32_ptr)a.key_end)[b], a.S), klo);

  // The one query block's visit list (full blocks first), cut into k chunks.
  const int nfull = ((const_i32_ptr)a.m.full_num)[0];
  const int nblk = nfull + ((const_i32_ptr)a.m.kv_num)[0];
  const const_i32_ptr full_list = (const_i32_ptr)a.m.full_idx;
  const const_i32_ptr part_list = (const_i32_ptr)a.m.kv_idx;
  auto kv_start = [&](int n) { return (n < nfull ? full_list[n] : part_list[n - nfull]) * kBlock; };
  const int m_begin = (int)((int64_t)chunk * nblk / k);
  const int m_end = (int)((int64_t)(chunk + 1) * nblk / k);

  // Q of the packed rows, 8 rows per wave (rows past R repeat row 0; their
  // results are never stored), and the rows' document ids.
  {
    const int r = wave * 8 + (lane >> 3);
    const int rr = r < R ? r : 0;
    const T* src = static_cast<const T*>(a.q) + b * a.q_sb + (hk * G + rr / a.L) * a.q_sh +
                   (int64_t)(rr % a.L) * a.q_sl + (lane & 7) * 8;
    lds_copy16(src, lds_offset(lds.q) + (uint32_t)wave * 1024u);
    if (KIND == ATTN_MASK_DOCUMENT && wave == 0 && lane < 32)
      lds_copy4(a.m.doc + (lq < R ? lq % a.L : 0), lds_offset(lds.doc_q));
  }
  const uint32_t k_off =
      (uint32_t)((lane >> 3) * a.k_sl * (int64_t)sizeof(T)) + (uint32_t)(((lane & 7) ^ (lane >> 3)) * 16);
  const uint32_t v_off = (uint32_t)((lane >> 3) * a.v_sl * (int64_t)sizeof(T)) +
                         (uint32_t)(((lane & 7) ^ (((lane >> 3) & 3) << 1)) * 16);
  auto issue = [&](int kv0, int st) __attribute__((always_inline)) {
    issue_k<T, KIND>(kg, a.k_sl, k_off, a.m.doc, kv0, a.S, lds.k[st], wave, lane);
    issue_rows<T, true>(vg, a.v_sl, v_off, kv0, a.S, lds.v[st].v, wave, lane);
    if constexpr (BITS) {
      // word `wave` (this wave's 32 keys) of each packed row's query
      if (lane < 32)
        lds_copy4(a.m.bits + (int64_t)(lq % a.L) * a.m.bits_w + 4 * (kv0 / kBlock) + wave,
                  lds_offset(lds.bits[st][wave]));
    }
  };
  // Blocks m_begin .. m_begin + NS - 2 go out first; block m then refills the
  // stage of block m - 1 with block m + NS - 1. The first key of the block
  // to copy next is loaded one block ahead.
  const int nb = m_end - m_begin;
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (i < nb) issue(kv_start(m_begin + i), i);
  int kv_issue = (nb > NS - 1) ? kv_start(m_begin + NS - 1) : 0;
  // Wait for Q (issued before every block copy), then share it.
  const int pro = min(NS - 1, nb);
  switch (pro) {  // blocks issued after Q
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<kPerBlock>(); break;
    case 2: wait_vm<2 * kPerBlock>(); break;
    default: wait_vm<3 * kPerBlock>(); break;
  }
  barrier_only();
  x8 qop[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qop[c] = *reinterpret_cast<const lds_x8*>((lds_u8)lds.q + lq * 128 + (2 * c + hf) * 16);
  const int lrow = lq % a.L;                   // this lane's query
  const int p = lrow + a.m.q_off;              // its rule position
  const int32_t dq = (KIND == ATTN_MASK_DOCUMENT) ? lds.doc_q[lq] : 0;

  const LanePtrs lp = make_lane_ptrs(lds, lane);
  f32x16_t oacc[2];
#pragma unroll
  for (int te = 0; te < 2; ++te)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[te][r] = 0.0f;
  float m_ref = -INFINITY, l = 0.0f;

  int st = 0;  // stage of block m
  for (int m = m_begin; m < m_end; ++m) {
    const int kv0 = kv_start(m);
    wait_lgkm_zero();  // this wave's reads of block m - 1, and the list loads
    switch (min(NS - 2, m_end - 1 - m)) {  // blocks issued after block m
      case 0: wait_vm<0>(); break;
      case 1: wait_vm<kPerBlock>(); break;
      default: wait_vm<2 * kPerBlock>(); break;
    }
    if (m + NS - 1 < m_end) {
      issue(kv_issue, st == 0 ? NS - 1 : st - 1);
      if (m + NS < m_end) kv_issue = kv_start(m + NS);
    }
    const bool full = m < nfull && kv0 >= klo && kv0 + kBlock <= khi;
    if (kv0 + kBlock <= klo || kv0 >= khi) {  // no kept key
      st = (st + 1 == NS) ? 0 : st + 1;
      continue;
    }
    // S^T = K Q^T for this wave's 32 keys (tile `wave` of the block).
    f32x16_t s = {};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const x8 kf = *reinterpret_cast<const lds_x8*>(lp.k[c] + st * (int)sizeof(KStage) + wave * 4096);
      s = V::mma(kf, qop[c], s);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = s[r];
      if (SOFTCAP) x = softcap_log2(x, 2.0f * kLog2e * a.scale / a.softcap, a.softcap * kLog2e);
      if (!full) {
        const int jl = wave * 32 + acc_row(r, hf);
        const int32_t dj = (KIND == ATTN_MASK_DOCUMENT) ? lds.k[st].doc[jl] : 0;
        bool ok = pair_live<KIND>(p, kv0 + jl, khi, a.m.window, dq, dj) && kv0 + jl >= klo;
        if constexpr (BITS) ok &= (lds.bits[st][wave][lq] >> acc_row(r, hf)) & 1u;
        if (!ok) x = -INFINITY;
      }
      s[r] = x;
      mx = fmaxf(mx, x);
    }
    mx = half_max(mx);
    const float m_blk = SOFTCAP ? mx : mx * c1;
    const bool grow = m_blk > m_ref + kRescaleLog2;
    if (__ballot(grow && m_ref != -INFINITY) != 0) {
      const float alpha = grow ? fast_exp2(m_ref - m_blk) : 1.0f;
      l *= alpha;
#pragma unroll
      for (int te = 0; te < 2; ++te)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[te][r] *= alpha;
    }
    if (grow) m_ref = m_blk;
    const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;
    // Probabilities, rounded to T for P V; the sum takes the rounded values.
    x8 pk[2];
    float psum[2] = {0.0f, 0.0f};
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int u = 0; u < 8; u += 2) {
        const float x0 = s[gi * 8 + u], x1 = s[gi * 8 + u + 1];
        const float p0 = SOFTCAP ? fast_exp2(x0 - m_use) : fast_exp2(fmaf(x0, c1, -m_use));
        const float p1 = SOFTCAP ? fast_exp2(x1 - m_use) : fast_exp2(fmaf(x1, c1, -m_use));
        const typename V::x2 pr = {(T)p0, (T)p1};
        psum[(u >> 1) & 1] = V::add_pair(pr, psum[(u >> 1) & 1]);
        pk[gi][u] = pr[0];
        pk[gi][u + 1] = pr[1];
      }
    dot_results_settle(psum[0], psum[1]);
    l += psum[0] + psum[1];
    // O^T += V^T P^T over the wave's two 16-key groups (2 wave, 2 wave + 1).
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int te = 0; te < 2; ++te) {
        const lds_u8 vb = lp.v[te] + st * (int)sizeof(VStage) + (2 * wave + gi) * 2048;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vb);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 1024));
        const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[te] = V::mma(__builtin_bit_cast(x8, both), pk[gi], oacc[te]);
      }
    st = (st + 1 == NS) ? 0 : st + 1;
  }
  const float lt = half_sum(l);

  // Combine the four waves: every copy has landed (the last block waited for
  // all), so once every wave's reads are done the stages hold each wave's
  // max, sum and O (row r, head dims te 32 + 8q + 4hf .. +3 in registers
  // 4q .. 4q+3 of tile te).
  wait_lgkm_zero();
  barrier_only();
  float* cm = reinterpret_cast<float*>(&lds);       // [4][32] maxima
  float* cl = cm + 4 * kPackRows;                   // [4][32] sums
  float* co = cl + 4 * kPackRows;                   // [4][32][kPackORow] O
  if (hf == 0) {
    cm[wave * kPackRows + lq] = m_ref;
    cl[wave * kPackRows + lq] = lt;
  }
#pragma unroll
  for (int te = 0; te < 2; ++te)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 o4 = {oacc[te][4 * q4], oacc[te][4 * q4 + 1], oacc[te][4 * q4 + 2], oacc[te][4 * q4 + 3]};
      *reinterpret_cast<float4*>(co + (wave * kPackRows + lq) * kPackORow + te * 32 + 8 * q4 + 4 * hf) = o4;
    }
  wait_lgkm_zero();
  barrier_only();
  // Thread: packed row tid / 8, head dims 8 (tid % 8) .. +7; waves in order.
  const int row = tid >> 3, e0 = (tid & 7) * 8;
  if (row >= R) return;
  float mw[4], wt[4];
  float mmax = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mw[w] = cm[w * kPackRows + row];
    mmax = fmaxf(mmax, mw[w]);
  }
  float lsum = 0.0f;
  float o8[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wt[w] = (mw[w] == -INFINITY) ? 0.0f : fast_exp2(mw[w] - mmax);
    lsum = (w == 0) ? wt[0] * cl[row] : fmaf(wt[w], cl[w * kPackRows + row], lsum);
    const float* orow = co + (w * kPackRows + row) * kPackORow + e0;
#pragma unroll
    for (int u = 0; u < 8; ++u) o8[u] = (w == 0) ? wt[0] * orow[u] : fmaf(wt[w], orow[u], o8[u]);
  }
  if (k > 1) {
    float* slot = a.partials + ((int64_t)bk * k + chunk) * kPackSlotFloats;
#pragma unroll
    for (int u = 0; u < 8; u += 4)
      *reinterpret_cast<float4*>(slot + row * kHeadDim + e0 + u) = {o8[u], o8[u + 1], o8[u + 2], o8[u + 3]};
    if (e0 == 0) {
      slot[kPackRows * kHeadDim + row] = mmax;
      slot[kPackRows * kHeadDim + kPackRows + row] = lsum;
    }
    return;
  }
  const int h = hk * G + row / a.L, qi = row % a.L;
  const float inv = (lsum > 0.0f) ? 1.0f / lsum : 0.0f;
  x8 outv;
#pragma unroll
  for (int u = 0; u < 8; ++u) outv[u] = (T)(o8[u] * inv);
  *reinterpret_cast<x8*>(static_cast<T*>(a.o) + b * a.o_sb + h * a.o_sh + (int64_t)qi * a.o_sl + e0) = outv;
  if (a.lse != nullptr && e0 == 0)
    a.lse[((int64_t)b * a.H + h) * a.L + qi] =
        (lsum > 0.0f) ? (mmax + __builtin_amdgcn_logf(lsum)) * kLn2 : -INFINITY;
}

// Merge of the packed kernel's chunks: one workgroup per (batch, K/V head,
// packed row); slots are [batch * K/V head][chunk].
template <typename T>
__global__ __launch_bounds__(kThreads) void packed_merge_kernel(FwdArgs a) {
  const int G = a.kv_group, Hk = a.H / G, R = a.L * G;
  const int bk = blockIdx.x / R, row = blockIdx.x % R;
  const int b = bk / Hk, hk = bk % Hk;
  const int h = hk * G + row / a.L, qi = row % a.L;
  const float* slot0 = a.partials + (int64_t)bk * a.pack_split * kPackSlotFloats;
  merge_row_block<T>(slot0, kPackSlotFloats, row * kHeadDim, kPackRows * kHeadDim + row,
                     kPackRows * kHeadDim + kPackRows + row, a.pack_split,
                     static_cast<T*>(a.o) + b * a.o_sb + h * a.o_sh + (int64_t)qi * a.o_sl,
                     a.lse == nullptr ? nullptr : a.lse + ((int64_t)b * a.H + h) * a.L + qi);
}

template <int KIND, bool SOFTCAP>
hipError_t launch_packed(int32_t dtype, const FwdArgs& a, hipStream_t stream) {
  const int64_t bhk = (int64_t)a.B * (a.H / a.kv_group);
  const dim3 grid((unsigned)(bhk * a.pack_split)), merge_grid((unsigned)(bhk * a.L * a.kv_group)),
      block(kThreads);
  const bool merge = a.pack_split > 1;
  switch (dtype) {
    case ATTN_BF16:
      hipLaunchKernelGGL((packed_kernel<__bf16, KIND, SOFTCAP>), grid, block, 0, stream, a);
      if (merge) hipLaunchKernelGGL(packed_merge_kernel<__bf16>, merge_grid, block, 0, stream, a);
      break;
    case ATTN_F16:
      hipLaunchKernelGGL((packed_kernel<_Float16, KIND, SOFTCAP>), grid, block, 0, stream, a);
      if (merge) hipLaunchKernelGGL(packed_merge_kernel<_Float16>, merge_grid, block, 0, stream, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KIND, bool SOFTCAP, bool PADDED, bool KVSPLIT>
hipError_t launch_split(int32_t dtype, const FwdArgs& a, hipStream_t stream) {
  // Up to kMaxChunks work items per query block (items past the plan's end
  // return at once), or kv_split split-KV chunks followed by their merge.
  const int64_t chunks = a.kv_split > 0 ? a.kv_split : a.items_per_qb;
  const dim3 grid((unsigned)((int64_t)a.B * a.H * a.m.nq * chunks));
  const dim3 block(kThreads);
  const dim3 merge_grid((unsigned)(((int64_t)a.B * a.H * a.L + kMergeRows - 1) / kMergeRows));
  switch (dtype) {
    case ATTN_BF16:
      hipLaunchKernelGGL((fwd16_kernel<__bf16, KIND, SOFTCAP, PADDED, KVSPLIT>), grid, block, 0, stream, a);
      if (KVSPLIT) hipLaunchKernelGGL(kv_merge_kernel<__bf16>, merge_grid, block, 0, stream, a);
      break;
    case ATTN_F16:
      hipLaunchKernelGGL((fwd16_kernel<_Float16, KIND, SOFTCAP, PADDED, KVSPLIT>), grid, block, 0, stream, a);
      if (KVSPLIT) hipLaunchKernelGGL(kv_merge_kernel<_Float16>, merge_grid, block, 0, stream, a);
      break;
    case ATTN_F32:
      hipLaunchKernelGGL((fwd32_kernel<KIND, SOFTCAP>), grid, block, 0, stream, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KIND, bool SOFTCAP>
hipError_t launch_chain(int32_t dtype, const FwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.chain), block(kThreads);
  switch (dtype) {
    case ATTN_BF16:
      hipLaunchKernelGGL((fwd16_chain_kernel<__bf16, KIND, SOFTCAP>), grid, block, 0, stream, a);
      break;
    case ATTN_F16:
      hipLaunchKernelGGL((fwd16_chain_kernel<_Float16, KIND, SOFTCAP>), grid, block, 0, stream, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Split-KV items have kernels of their own, so the others keep their code.
template <int KIND, bool SOFTCAP, bool PADDED>
hipError_t launch_kind(int32_t dtype, const FwdArgs& a, hipStream_t stream) {
  if constexpr (KIND == ATTN_MASK_SLIDING_WINDOW && !PADDED)
    if (a.chain > 0) return launch_chain<KIND, SOFTCAP>(dtype, a, stream);
  if (a.pack_split > 0) return launch_packed<KIND, SOFTCAP>(dtype, a, stream);
  return (a.kv_split > 0 && dtype != ATTN_F32) ? launch_split<KIND, SOFTCAP, PADDED, true>(dtype, a, stream)
                                               : launch_split<KIND, SOFTCAP, PADDED, false>(dtype, a, stream);
}

template <int KIND, bool PADDED>
hipError_t launch_softcap(int32_t dtype, const FwdArgs& a, hipStream_t stream) {
  return a.softcap > 0.0f ? launch_kind<KIND, true, PADDED>(dtype, a, stream)
                          : launch_kind<KIND, false, PADDED>(dtype, a, stream);
}

// Key padding has kernels of its own, so the unpadded ones carry no range
// tests.
template <int KIND>
hipError_t launch_padded(int32_t dtype, const FwdArgs& a, hipStream_t stream) {
  return (a.key_start != nullptr || a.key_end != nullptr) ? launch_softcap<KIND, true>(dtype, a, stream)
                                                          : launch_softcap<KIND, false>(dtype, a, stream);
}

}  // namespace

// Launch of the forward for one mask family (defined in fwd_<family>.hip).
template <int KIND>
hipError_t launch_family(int32_t dtype, const FwdArgs& a, hipStream_t stream) {
  return launch_padded<KIND>(dtype, a, stream);
}

}  // namespace bsattn
