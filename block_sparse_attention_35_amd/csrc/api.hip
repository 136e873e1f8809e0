// C ABI entry points: host-side validation, then an asynchronous launch on
// the caller's stream. Nothing here allocates device memory or synchronises.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "bsattn.h"
#include "internal.h"

namespace {

thread_local char g_last_error[512] = "";

attn_status fail(attn_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

attn_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ATTN_OK;
  return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Arrays with no elements may be null (an empty tensor has no storage).
bool arrays_present(const attn_block_mask* bm, int32_t nq, int32_t nk) {
  const bool per_q = nq == 0 || (bm->kv_num_blocks && bm->full_kv_num_blocks && bm->schedule);
  const bool per_pair = (int64_t)nq * nk == 0 || (bm->kv_indices && bm->full_kv_indices);
  return per_q && per_pair;
}

constexpr int64_t kMaxSeqStride = int64_t(1) << 24;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Fill batch/head/sequence strides (elements) and check the head-dim stride
// and 16-byte row alignment.
// The stride of a dimension of size 1 is never used and may be anything.
attn_status strides_of(const char* name, const int64_t* st, int32_t B, int32_t H, int32_t len,
                       int32_t E, int esize, int64_t out[3]) {
  if (st == nullptr) {
    out[2] = E;
    out[1] = (int64_t)len * E;
    out[0] = (int64_t)H * len * E;
    return ATTN_OK;
  }
  if (len == 0) {  // no elements: strides are never used
    out[0] = out[1] = out[2] = 0;
    return ATTN_OK;
  }
  if (st[3] != 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: head-dim stride must be 1", name);
  const int32_t size[3] = {B, H, len};
  for (int d = 0; d < 3; ++d) {
    if (size[d] <= 1) {
      out[d] = 0;
      continue;
    }
    if (st[d] < 0) return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: negative stride", name);
    if ((st[d] * esize) % 16 != 0)
      return fail(ATTN_ERR_INVALID_ARGUMENT, "%s: stride %d (%lld elements) breaks 16-byte alignment",
                  name, d, (long long)st[d]);
    out[d] = st[d];
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

int32_t attn_num_blocks(int32_t len, int32_t block_size) {
  if (len < 0 || block_size != ATTN_BLOCK_SIZE) return -1;
  return (int32_t)(((int64_t)len + block_size - 1) / block_size);
}

int32_t attn_block_mask_schedule_len(int32_t q_len, int32_t kv_len, int32_t block_size) {
  const int32_t nq = attn_num_blocks(q_len, block_size);
  if (nq < 0 || attn_num_blocks(kv_len, block_size) < 0) return -1;
  return 4 + 8 * nq;
}

}  // extern "C"

namespace {

// Shared body of the two builders: validates, fills bm's fields and enqueues
// the classification and the work plan.
attn_status build_impl(int32_t kind, int32_t window, const int32_t* document_id,
                       const uint32_t* bits, int32_t q_len, int32_t kv_len, int32_t block_size,
                       attn_block_mask* bm, void* stream) {
  g_last_error[0] = '\0';
  if (bm == nullptr) return fail(ATTN_ERR_INVALID_ARGUMENT, "block mask struct is null");
  if (q_len < 0 || kv_len < 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "negative length (q_len=%d, kv_len=%d)", q_len, kv_len);
  if (block_size != ATTN_BLOCK_SIZE)
    return fail(ATTN_ERR_UNSUPPORTED, "block_size %d: only %d is supported", block_size,
                ATTN_BLOCK_SIZE);
  const bool windowed = kind == ATTN_MASK_SLIDING_WINDOW || kind == ATTN_MASK_SLIDING_WINDOW_LOWER_RIGHT;
  const bool documents = kind == ATTN_MASK_DOCUMENT || kind == ATTN_MASK_DOCUMENT_BIDIRECTIONAL;
  const bool custom = kind == ATTN_MASK_CUSTOM;
  if (windowed && window < 1)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "sliding window must be >= 1 (got %d)", window);
  if (documents && document_id == nullptr)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "document mask needs document_id");
  if (custom && bits == nullptr && (int64_t)q_len * kv_len > 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "custom mask needs its bits");
  if (custom && (reinterpret_cast<uintptr_t>(bits) & 15u) != 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "custom mask bits must be 16-byte aligned");
  const int32_t nq = attn_num_blocks(q_len, block_size);
  const int32_t nk = attn_num_blocks(kv_len, block_size);
  if (!arrays_present(bm, nq, nk))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "block mask array pointer is null");
  if (nk > ATTN_MAX_KV_BLOCKS)
    return fail(ATTN_ERR_UNSUPPORTED, "%d kv blocks exceed the supported %d", nk,
                ATTN_MAX_KV_BLOCKS);
  bm->q_len = q_len;
  bm->kv_len = kv_len;
  bm->block_size = block_size;
  bm->num_q_blocks = nq;
  bm->num_kv_blocks = nk;
  bm->kind = kind;
  bm->window = windowed ? window : 0;
  bm->document_id = documents ? document_id : nullptr;
  bm->mask_bits = custom ? bits : nullptr;
  const bsattn::MaskForm form = bsattn::mask_form(kind, q_len, kv_len);
  return hip_status(bsattn::launch_block_mask(form.kind, form.q_off, bm->window, bm->document_id,
                                              bm->mask_bits, q_len, kv_len, nq, nk,
                                              bm->kv_num_blocks, bm->kv_indices,
                                              bm->full_kv_num_blocks, bm->full_kv_indices,
                                              bm->schedule, static_cast<hipStream_t>(stream)),
                    "block mask launch");
}

}  // namespace

extern "C" {

attn_status attn_build_block_mask(int32_t kind, int32_t window, const int32_t* document_id,
                                  int32_t q_len, int32_t kv_len, int32_t block_size,
                                  attn_block_mask* bm, void* stream) {
  if (kind < ATTN_MASK_NONE || kind > ATTN_MASK_DOCUMENT_BIDIRECTIONAL) {
    g_last_error[0] = '\0';
    return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown mask kind %d%s", kind,
                kind == ATTN_MASK_CUSTOM ? " (custom masks: attn_build_block_mask_custom)" : "");
  }
  return build_impl(kind, window, document_id, nullptr, q_len, kv_len, block_size, bm, stream);
}

int32_t attn_mask_words(int32_t kv_len) {
  if (kv_len < 0) return -1;
  return 4 * attn_num_blocks(kv_len, ATTN_BLOCK_SIZE);
}

attn_status attn_pack_mask(const uint8_t* dense, int64_t row_stride, int32_t q_len, int32_t kv_len,
                           uint32_t* bits, void* stream) {
  g_last_error[0] = '\0';
  if (q_len < 0 || kv_len < 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "negative length (q_len=%d, kv_len=%d)", q_len, kv_len);
  if (row_stride < kv_len)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "row_stride %lld < kv_len %d", (long long)row_stride, kv_len);
  if ((int64_t)q_len * kv_len > 0 && (dense == nullptr || bits == nullptr))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "dense and bits must be non-null");
  if ((reinterpret_cast<uintptr_t>(bits) & 15u) != 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "bits must be 16-byte aligned");
  return hip_status(bsattn::launch_pack_mask(dense, row_stride, q_len, kv_len, bits,
                                             static_cast<hipStream_t>(stream)),
                    "mask pack launch");
}

attn_status attn_build_block_mask_custom(const uint32_t* bits, int32_t q_len, int32_t kv_len,
                                         int32_t block_size, attn_block_mask* bm, void* stream) {
  return build_impl(ATTN_MASK_CUSTOM, 0, nullptr, bits, q_len, kv_len, block_size, bm, stream);
}

}  // extern "C"

namespace {

// Zeroes n 32-bit words (a kernel rather than a memset node, so a captured
// call clears the counters on every replay too).
__global__ void zero_words_kernel(int32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// attn_forward with H_kv K/V heads (H_kv == H: no sharing).
attn_status forward_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                         int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t L, int32_t S,
                         int32_t E, const int64_t* q_strides, const int64_t* k_strides,
                         const int64_t* v_strides, const int64_t* o_strides,
                         const attn_block_mask* bm, int32_t score_mod, float softcap, float scale,
                         const int32_t* key_start, const int32_t* key_end, void* workspace,
                         size_t workspace_size, void* stream, bool clear_counters = false) {
  g_last_error[0] = '\0';
  if (bm == nullptr) return fail(ATTN_ERR_INVALID_ARGUMENT, "block mask is null");
  // A tensor with no elements may have a null pointer.
  if ((!q && L > 0) || (!o && L > 0) || (!k && S > 0) || (!v && S > 0))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "q, k, v and o must be non-null");
  int esize;
  switch (dtype) {
    case ATTN_F32: esize = 4; break;
    case ATTN_BF16: esize = 2; break;
    case ATTN_F16: esize = 2; break;
    default: return fail(ATTN_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  }
  if (B < 1 || H < 1 || L < 0 || S < 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "bad sizes B=%d H=%d L=%d S=%d", B, H, L, S);
  if (H_kv < 1 || H % H_kv != 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "H=%d query heads cannot share H_kv=%d K/V heads", H, H_kv);
  if (E != bsattn::kHeadDim)
    return fail(ATTN_ERR_UNSUPPORTED, "head dim %d: only %d is supported", E, bsattn::kHeadDim);
  if (bm->q_len != L || bm->kv_len != S || bm->block_size != ATTN_BLOCK_SIZE)
    return fail(ATTN_ERR_INVALID_ARGUMENT,
                "block mask was built for q_len=%d kv_len=%d block=%d, tensors have L=%d S=%d",
                bm->q_len, bm->kv_len, bm->block_size, L, S);
  if (bm->num_q_blocks != attn_num_blocks(L, ATTN_BLOCK_SIZE) ||
      bm->num_kv_blocks != attn_num_blocks(S, ATTN_BLOCK_SIZE) ||
      !arrays_present(bm, bm->num_q_blocks, bm->num_kv_blocks))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "block mask is not built");
  if (bm->kind < ATTN_MASK_NONE || bm->kind > ATTN_MASK_CUSTOM ||
      ((bm->kind == ATTN_MASK_SLIDING_WINDOW || bm->kind == ATTN_MASK_SLIDING_WINDOW_LOWER_RIGHT) &&
       bm->window < 1) ||
      ((bm->kind == ATTN_MASK_DOCUMENT || bm->kind == ATTN_MASK_DOCUMENT_BIDIRECTIONAL) &&
       bm->document_id == nullptr) ||
      (bm->kind == ATTN_MASK_CUSTOM &&
       ((bm->mask_bits == nullptr && (int64_t)L * S > 0) ||
        (reinterpret_cast<uintptr_t>(bm->mask_bits) & 15u) != 0)))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "block mask fields are inconsistent");
  if (score_mod != ATTN_SCORE_NONE && score_mod != ATTN_SCORE_SOFTCAP)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown score_mod %d", score_mod);
  if (score_mod == ATTN_SCORE_SOFTCAP && !(std::isfinite(softcap) && softcap > 0.0f))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "soft-cap must be finite and > 0");
  if (!(std::isfinite(scale) && scale > 0.0f))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "q, k, v and o must be 16-byte aligned");

  bsattn::FwdArgs a{};
  int64_t st[3];
  attn_status s;
  if ((s = strides_of("q", q_strides, B, H, L, E, esize, st)) != ATTN_OK) return s;
  a.q_sb = st[0], a.q_sh = st[1], a.q_sl = st[2];
  if ((s = strides_of("k", k_strides, B, H_kv, S, E, esize, st)) != ATTN_OK) return s;
  a.k_sb = st[0], a.k_sh = st[1], a.k_sl = st[2];
  if ((s = strides_of("v", v_strides, B, H_kv, S, E, esize, st)) != ATTN_OK) return s;
  a.v_sb = st[0], a.v_sh = st[1], a.v_sl = st[2];
  if ((s = strides_of("o", o_strides, B, H, L, E, esize, st)) != ATTN_OK) return s;
  a.o_sb = st[0], a.o_sh = st[1], a.o_sl = st[2];
  // Tile copies address 8 consecutive K/V rows with a 32-bit byte offset.
  if (a.k_sl > kMaxSeqStride || a.v_sl > kMaxSeqStride)
    return fail(ATTN_ERR_UNSUPPORTED, "k/v sequence stride above %lld elements",
                (long long)kMaxSeqStride);
  if ((int64_t)B * H * bm->num_q_blocks * 2 > 0x7fffffffLL)
    return fail(ATTN_ERR_UNSUPPORTED, "too many work items");
  const size_t need =
      bsattn::workspace_bytes(dtype, (int64_t)B * H, bm->num_q_blocks, bm->num_kv_blocks);
  if (need > 0) {
    if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
        workspace_size < need)
      return fail(ATTN_ERR_INVALID_ARGUMENT,
                  "workspace must be 256-byte aligned and hold %zu bytes (got %zu)", need,
                  workspace == nullptr ? (size_t)0 : workspace_size);
    a.kv_split = bsattn::kv_split_count(dtype, (int64_t)B * H, bm->num_q_blocks, bm->num_kv_blocks);
    a.split = a.kv_split > 0 ? 0 : 1;
    a.counters = static_cast<int32_t*>(workspace);
    a.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + bsattn::kCountersBytes);
  }
  if (bsattn::use_packed(dtype, L, H / H_kv)) {
    a.pack_split = bsattn::packed_split_count((int64_t)B * H_kv, bm->num_kv_blocks, need);
    a.kv_split = 0;
    a.split = 0;
  }

  a.q = q, a.k = k, a.v = v, a.o = o, a.lse = lse;
  a.B = B, a.H = H, a.L = L, a.S = S;
  a.kv_group = H / H_kv;
  a.key_start = key_start;
  a.key_end = key_end;
  a.m.kv_num = bm->kv_num_blocks;
  a.m.kv_idx = bm->kv_indices;
  a.m.full_num = bm->full_kv_num_blocks;
  a.m.full_idx = bm->full_kv_indices;
  a.m.schedule = bm->schedule;
  a.m.doc = bm->document_id;
  a.m.bits = bm->mask_bits;
  a.m.bits_w = 4 * bm->num_kv_blocks;
  a.m.nq = bm->num_q_blocks;
  a.m.nk = bm->num_kv_blocks;
  const bsattn::MaskForm form = bsattn::mask_form(bm->kind, L, S);
  a.m.kind = form.kind;
  a.m.q_off = form.q_off;
  a.m.window = bm->window;
  a.scale = scale;
  a.softcap = (score_mod == ATTN_SCORE_SOFTCAP) ? softcap : 0.0f;
  a.items_per_qb = bsattn::plan_never_splits(form.kind, bm->window, bm->num_kv_blocks) ? 1 : bsattn::kMaxChunks;
  if (a.pack_split == 0 && a.kv_split == 0) {
    a.chain = bsattn::chain_grid(dtype, form.kind, bm->window, key_start != nullptr || key_end != nullptr,
                                 (int64_t)B * H, bm->num_q_blocks, S);
    if (a.chain > 0) a.split = 0;  // no plan entry of such a window is split
  }
  if (clear_counters && need > 0) {
    const int n = (int)(bsattn::kCountersBytes / sizeof(int32_t));
    hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<int32_t*>(workspace), n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e, "scratch counter clear launch");
  }
  return hip_status(bsattn::launch_forward(dtype, a, static_cast<hipStream_t>(stream)),
                    "forward launch");
}

}  // namespace

extern "C" {

attn_status attn_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                         int32_t dtype, int32_t B, int32_t H, int32_t L, int32_t S, int32_t E,
                         const int64_t* q_strides, const int64_t* k_strides,
                         const int64_t* v_strides, const int64_t* o_strides,
                         const attn_block_mask* bm, int32_t score_mod, float softcap, float scale,
                         void* workspace, size_t workspace_size, void* stream) {
  return forward_impl(q, k, v, o, lse, dtype, B, H, H, L, S, E, q_strides, k_strides, v_strides,
                      o_strides, bm, score_mod, softcap, scale, nullptr, nullptr, workspace,
                      workspace_size, stream);
}

attn_status attn_forward_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                             int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t L, int32_t S,
                             int32_t E, const int64_t* q_strides, const int64_t* k_strides,
                             const int64_t* v_strides, const int64_t* o_strides,
                             const attn_block_mask* bm, int32_t score_mod, float softcap,
                             float scale, void* workspace, size_t workspace_size, void* stream) {
  return forward_impl(q, k, v, o, lse, dtype, B, H, H_kv, L, S, E, q_strides, k_strides, v_strides,
                      o_strides, bm, score_mod, softcap, scale, nullptr, nullptr, workspace,
                      workspace_size, stream);
}

attn_status attn_forward_padded(const void* q, const void* k, const void* v, void* o, float* lse,
                                int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t L,
                                int32_t S, int32_t E, const int64_t* q_strides,
                                const int64_t* k_strides, const int64_t* v_strides,
                                const int64_t* o_strides, const attn_block_mask* bm,
                                int32_t score_mod, float softcap, float scale,
                                const int32_t* key_start, const int32_t* key_end, void* workspace,
                                size_t workspace_size, void* stream) {
  return forward_impl(q, k, v, o, lse, dtype, B, H, H_kv, L, S, E, q_strides, k_strides, v_strides,
                      o_strides, bm, score_mod, softcap, scale, key_start, key_end, workspace,
                      workspace_size, stream);
}

}  // extern "C"

namespace {

// Scratch memory of attn_forward_noalloc: one copy per GPU, allocated with
// the library's code object when it is loaded on that GPU and held until the
// process ends. In host code `scratch` names a host-side stand-in, not the
// GPU's copy, so it is never passed to a kernel or a copy: each device's
// address comes from hipGetSymbolAddress with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up once per device).
attn_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_ERR_UNSUPPORTED, "device %d: the no-alloc scratch tracks %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0)
      return fail(ATTN_ERR_HIP, "scratch symbol has no usable device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_forward_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t L,
                                 int32_t S, int32_t E, const int64_t* q_strides,
                                 const int64_t* k_strides, const int64_t* v_strides,
                                 const int64_t* o_strides, const attn_block_mask* bm,
                                 int32_t score_mod, float softcap, float scale,
                                 const int32_t* key_start, const int32_t* key_end, void* stream) {
  g_last_error[0] = '\0';
  if (bm == nullptr) return fail(ATTN_ERR_INVALID_ARGUMENT, "block mask is null");
  if (B < 1 || H < 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "bad sizes B=%d H=%d", B, H);
  const size_t need =
      bsattn::workspace_bytes(dtype, (int64_t)B * H, bm->num_q_blocks, bm->num_kv_blocks);
  if (need > kNoAllocScratchBytes)
    return fail(ATTN_ERR_UNSUPPORTED,
                "this shape needs %zu bytes of scratch; attn_forward_noalloc holds %zu "
                "(use attn_forward_padded with a workspace)",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    attn_status st = scratch_of_current_device(&ws);
    if (st != ATTN_OK) return st;
  }
  // The shared body validates everything attn_forward_padded does before it
  // enqueues anything; split work items then start from zeroed counters.
  return forward_impl(q, k, v, o, lse, dtype, B, H, H_kv, L, S, E, q_strides, k_strides, v_strides,
                      o_strides, bm, score_mod, softcap, scale, key_start, key_end, ws,
                      need > 0 ? kNoAllocScratchBytes : 0, stream, /*clear_counters=*/true);
}

attn_status attn_backward_workspace_size(int32_t B, int32_t H, int32_t H_kv, const attn_block_mask* bm,
                                         size_t* bytes) {
  g_last_error[0] = '\0';
  if (bm == nullptr || bytes == nullptr)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "block mask and bytes must be non-null");
  if (B < 1 || H < 1 || H_kv < 1 || H % H_kv != 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "bad sizes B=%d H=%d H_kv=%d", B, H, H_kv);
  *bytes = bsattn::bwd_workspace_bytes((int64_t)B * H, (int64_t)B * H_kv, bm->q_len, bm->num_q_blocks,
                                       bm->num_kv_blocks);
  return ATTN_OK;
}

attn_status attn_backward(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          int32_t dtype, int32_t B, int32_t H, int32_t H_kv, int32_t L, int32_t S,
                          int32_t E, const attn_block_mask* bm, int32_t score_mod, float softcap,
                          float scale, const int32_t* key_start, const int32_t* key_end,
                          void* workspace, size_t workspace_size, void* stream) {
  g_last_error[0] = '\0';
  if (bm == nullptr) return fail(ATTN_ERR_INVALID_ARGUMENT, "block mask is null");
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_F16)
    return fail(ATTN_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (B < 1 || H < 1 || L < 0 || S < 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "bad sizes B=%d H=%d L=%d S=%d", B, H, L, S);
  if (H_kv < 1 || H % H_kv != 0)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "H=%d query heads cannot share H_kv=%d K/V heads", H, H_kv);
  if (E != bsattn::kHeadDim)
    return fail(ATTN_ERR_UNSUPPORTED, "head dim %d: only %d is supported", E, bsattn::kHeadDim);
  if ((L > 0 && (!q || !o || !lse || !dout || !dq)) || (S > 0 && (!k || !v || !dk || !dv)))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "q, k, v, o, lse, dout, dq, dk and dv must be non-null");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "tensors must be 16-byte aligned");
  if (bm->q_len != L || bm->kv_len != S || bm->block_size != ATTN_BLOCK_SIZE)
    return fail(ATTN_ERR_INVALID_ARGUMENT,
                "block mask was built for q_len=%d kv_len=%d block=%d, tensors have L=%d S=%d",
                bm->q_len, bm->kv_len, bm->block_size, L, S);
  if (bm->num_q_blocks != attn_num_blocks(L, ATTN_BLOCK_SIZE) ||
      bm->num_kv_blocks != attn_num_blocks(S, ATTN_BLOCK_SIZE) ||
      !arrays_present(bm, bm->num_q_blocks, bm->num_kv_blocks))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "block mask is not built");
  if (bm->kind < ATTN_MASK_NONE || bm->kind > ATTN_MASK_CUSTOM ||
      ((bm->kind == ATTN_MASK_SLIDING_WINDOW || bm->kind == ATTN_MASK_SLIDING_WINDOW_LOWER_RIGHT) &&
       bm->window < 1) ||
      ((bm->kind == ATTN_MASK_DOCUMENT || bm->kind == ATTN_MASK_DOCUMENT_BIDIRECTIONAL) &&
       bm->document_id == nullptr) ||
      (bm->kind == ATTN_MASK_CUSTOM && ((bm->mask_bits == nullptr && (int64_t)L * S > 0) ||
                                        (reinterpret_cast<uintptr_t>(bm->mask_bits) & 15u) != 0)))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "block mask fields are inconsistent");
  if (score_mod != ATTN_SCORE_NONE && score_mod != ATTN_SCORE_SOFTCAP)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "unknown score_mod %d", score_mod);
  if (score_mod == ATTN_SCORE_SOFTCAP && !(std::isfinite(softcap) && softcap > 0.0f))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "soft-cap must be finite and > 0");
  if (!(std::isfinite(scale) && scale > 0.0f))
    return fail(ATTN_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
  if ((int64_t)B * H * (bm->num_q_blocks > bm->num_kv_blocks ? bm->num_q_blocks : bm->num_kv_blocks) >
      0x7fffffffLL)
    return fail(ATTN_ERR_UNSUPPORTED, "too many work items");
  const bsattn::BwdLayout lay =
      bsattn::bwd_layout((int64_t)B * H, (int64_t)B * H_kv, L, bm->num_q_blocks, bm->num_kv_blocks);
  const size_t need = lay.total;
  if (need > 0 && (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
                   workspace_size < need))
    return fail(ATTN_ERR_INVALID_ARGUMENT,
                "workspace must be 256-byte aligned and hold %zu bytes (got %zu)", need,
                workspace == nullptr ? (size_t)0 : workspace_size);

  bsattn::BwdArgs a{};
  bsattn::FwdArgs& f = a.f;
  f.q = q, f.k = k, f.v = v, f.o = const_cast<void*>(o), f.lse = const_cast<float*>(lse);
  f.B = B, f.H = H, f.L = L, f.S = S;
  f.kv_group = H / H_kv;
  f.key_start = key_start;
  f.key_end = key_end;
  // contiguous [B, heads, len, E]
  f.q_sl = f.o_sl = E, f.q_sh = f.o_sh = (int64_t)L * E, f.q_sb = f.o_sb = (int64_t)H * L * E;
  f.k_sl = f.v_sl = E, f.k_sh = f.v_sh = (int64_t)S * E, f.k_sb = f.v_sb = (int64_t)H_kv * S * E;
  f.m.kv_num = bm->kv_num_blocks;
  f.m.kv_idx = bm->kv_indices;
  f.m.full_num = bm->full_kv_num_blocks;
  f.m.full_idx = bm->full_kv_indices;
  f.m.schedule = bm->schedule;
  f.m.doc = bm->document_id;
  f.m.bits = bm->mask_bits;
  f.m.bits_w = 4 * bm->num_kv_blocks;
  f.m.nq = bm->num_q_blocks;
  f.m.nk = bm->num_kv_blocks;
  const bsattn::MaskForm form = bsattn::mask_form(bm->kind, L, S);
  f.m.kind = form.kind;
  f.m.q_off = form.q_off;
  f.m.window = bm->window;
  f.scale = scale;
  f.softcap = (score_mod == ATTN_SCORE_SOFTCAP) ? softcap : 0.0f;
  a.dout = dout, a.dq = dq, a.dk = dk, a.dv = dv;
  char* w = static_cast<char*>(workspace);
  a.D = reinterpret_cast<float*>(w + lay.D);
  a.lse2 = reinterpret_cast<float*>(w + lay.lse2);
  a.tq_num = reinterpret_cast<int32_t*>(w + lay.tq_num);
  a.tf_num = reinterpret_cast<int32_t*>(w + lay.tf_num);
  a.tq_idx = reinterpret_cast<int32_t*>(w + lay.tq_idx);
  a.tf_idx = reinterpret_cast<int32_t*>(w + lay.tf_idx);
  a.tplan = reinterpret_cast<int32_t*>(w + lay.tplan);
  a.split_kv = lay.split_kv ? 1 : 0;
  f.split = lay.split_q ? 1 : 0;
  a.counters_kv = reinterpret_cast<int32_t*>(w + lay.counters_kv);
  a.counters_q = reinterpret_cast<int32_t*>(w + lay.counters_q);
  a.part_kv = reinterpret_cast<float*>(w + lay.part_kv);
  a.part_q = reinterpret_cast<float*>(w + lay.part_q);
  return hip_status(bsattn::launch_backward(dtype, a, static_cast<hipStream_t>(stream)),
                    "backward launch");
}

attn_status attn_forward_workspace_size(int32_t dtype, int32_t B, int32_t H,
                                        const attn_block_mask* bm, size_t* bytes) {
  g_last_error[0] = '\0';
  if (bm == nullptr || bytes == nullptr)
    return fail(ATTN_ERR_INVALID_ARGUMENT, "block mask and bytes must be non-null");
  if (B < 1 || H < 1) return fail(ATTN_ERR_INVALID_ARGUMENT, "bad sizes B=%d H=%d", B, H);
  *bytes = bsattn::workspace_bytes(dtype, (int64_t)B * H, bm->num_q_blocks, bm->num_kv_blocks);
  return ATTN_OK;
}

const char* attn_status_string(attn_status status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported";
    case ATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_last_error; }

}  // extern "C"
