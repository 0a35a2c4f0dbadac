// C-ABI entry points (include/idx.h): argument validation, the gfx950 gate, and the
// hand-off to the kernel launchers.  Validation is plain host code that runs before
// any HIP call, so every error path can be exercised on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "idx.h"
#include "launch.hpp"

#define IDX_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxDevices = 64;
// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_arch_state[kMaxDevices];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return IDX_EUNSUPPORTED;
  }
  if (dev < kMaxDevices) {
    const int st = g_arch_state[dev].load(std::memory_order_relaxed);
    if (st == 1) return IDX_OK;
    if (st == 2) return IDX_EUNSUPPORTED;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return IDX_EUNSUPPORTED;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? IDX_OK : IDX_EUNSUPPORTED;
}

// Compute units of the current device (cached per device; 256 if the query fails).
int num_cus() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return 256;
  }
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

int64_t bytes_per_token(int32_t fmt) { return fmt == IDX_KV_MXFP4 ? 68 : (fmt == IDX_KV_FP8_E4M3 ? 132 : -1); }

// Pool checks shared by every entry point that takes a pool.
int check_pool(const idx_pool* p, int32_t want_fmt) {
  if (!p || !p->base) return IDX_EINVAL;
  if (p->kv_format != IDX_KV_MXFP4 && p->kv_format != IDX_KV_FP8_E4M3) return IDX_EINVAL;
  if (want_fmt >= 0 && p->kv_format != want_fmt) return IDX_EINVAL;
  if (p->page_size < 16 || p->page_size > 1024 || (p->page_size & (p->page_size - 1)) != 0) return IDX_EUNSUPPORTED;
  if (p->offset_bytes < 0 || p->num_pages <= 0 || p->page_stride_bytes <= 0) return IDX_EINVAL;
  if (p->page_stride_bytes < bytes_per_token(p->kv_format) * p->page_size) return IDX_EINVAL;
  if (p->offset_bytes % 256 != 0 || p->page_stride_bytes % 256 != 0) return IDX_EALIGN;
  if ((reinterpret_cast<uintptr_t>(p->base) & 255u) != 0) return IDX_EALIGN;
  // the pool's byte span must fit in a signed 64-bit offset
  if (p->num_pages > (INT64_MAX - p->offset_bytes) / p->page_stride_bytes) return IDX_EINVAL;
  return IDX_OK;
}

idx::PoolView view_of(const idx_pool* p) {
  idx::PoolView v;
  v.base = static_cast<uint8_t*>(p->base) + p->offset_bytes;
  v.stride = p->page_stride_bytes;
  v.num_pages = p->num_pages;
  v.page_size = p->page_size;
  v.page_shift = __builtin_ctz((unsigned)p->page_size);
  v.kv_format = p->kv_format;
  return v;
}

int hip_status(hipError_t e) { return e == hipSuccess ? IDX_OK : IDX_EHIP; }

// Scratch the fused decode step takes: one block counter per sequence.
size_t step_workspace_bytes(int32_t B) { return B < 1 ? 0 : ((size_t)B * sizeof(int32_t) + 255) / 256 * 256; }

// A (workspace, ws_bytes) pair for a call that uses `need` bytes of it: NULL only with
// ws_bytes == 0 and need == 0; a buffer must be 256-byte aligned and large enough.
int check_workspace(const void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return (ws_bytes == 0 && need == 0) ? IDX_OK : IDX_EINVAL;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return IDX_EALIGN;
  return ws_bytes >= need ? IDX_OK : IDX_EINVAL;
}

int k_store_common(const idx_pool* pool, int32_t fmt, const void* k_bf16, int64_t n_rows, int64_t row_stride_elems,
                   const float* gamma, float eps, const int32_t* positions, const float* cos_sin, int32_t max_pos,
                   const int64_t* slot_mapping, void* stream) {
  int st = check_pool(pool, fmt);
  if (st != IDX_OK) return st;
  if (n_rows < 0 || row_stride_elems < 128) return IDX_EINVAL;
  if (n_rows > 0 && (!k_bf16 || !gamma || !positions || !cos_sin || !slot_mapping)) return IDX_EINVAL;
  if (!(eps > 0.0f) || max_pos <= 0) return IDX_EINVAL;
  if (n_rows > (int64_t)UINT32_MAX * 4) return IDX_EINVAL;
  if ((st = check_device()) != IDX_OK) return st;
  idx::KStoreArgs a;
  a.pool = view_of(pool);
  a.k = static_cast<const uint16_t*>(k_bf16);
  a.n_rows = n_rows;
  a.row_stride = row_stride_elems;
  a.gamma = gamma;
  a.eps = (double)eps;
  a.positions = positions;
  a.cos_sin = cos_sin;
  a.max_pos = max_pos;
  a.slots = slot_mapping;
  return hip_status(idx::launch_k_store(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

IDX_EXPORT int idx_k_store_mxfp4(const idx_pool* pool, const void* k_bf16, int64_t n_rows, int64_t row_stride_elems,
                                 const float* gamma, float eps, const int32_t* positions, const float* cos_sin,
                                 int32_t max_pos, const int64_t* slot_mapping, void* stream) {
  return k_store_common(pool, IDX_KV_MXFP4, k_bf16, n_rows, row_stride_elems, gamma, eps, positions, cos_sin,
                        max_pos, slot_mapping, stream);
}

IDX_EXPORT int idx_k_store_fp8(const idx_pool* pool, const void* k_bf16, int64_t n_rows, int64_t row_stride_elems,
                               const float* gamma, float eps, const int32_t* positions, const float* cos_sin,
                               int32_t max_pos, const int64_t* slot_mapping, void* stream) {
  return k_store_common(pool, IDX_KV_FP8_E4M3, k_bf16, n_rows, row_stride_elems, gamma, eps, positions, cos_sin,
                        max_pos, slot_mapping, stream);
}

IDX_EXPORT int idx_qk_prep_fp8(const idx_pool* pool, const void* q_bf16, const void* k_bf16, int64_t n_tokens,
                               int32_t H, const float* w, const int32_t* positions, const float* cos_sin,
                               int32_t max_pos, int32_t rope_neox, const float* ln_gamma, const float* ln_beta,
                               float eps, const int64_t* slot_mapping, uint8_t* q_fp8, float* w_out, void* stream) {
  int st = check_pool(pool, IDX_KV_FP8_E4M3);
  if (st != IDX_OK) return st;
  if (n_tokens < 0 || H < 1 || max_pos <= 0 || !(eps > 0.0f) || (rope_neox != 0 && rope_neox != 1))
    return IDX_EINVAL;
  if (H > idx::kMaxHeads) return IDX_EUNSUPPORTED;
  if (n_tokens > 0 && (!q_bf16 || !k_bf16 || !w || !positions || !cos_sin || !ln_gamma || !ln_beta ||
                       !slot_mapping || !q_fp8 || !w_out))
    return IDX_EINVAL;
  // one wave per vector: the grid's work-items (64 per vector) must fit in 32 bits
  if (n_tokens > (int64_t)(UINT32_MAX / 64) / (H + 1)) return IDX_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q_fp8) & 3u) != 0 || (reinterpret_cast<uintptr_t>(q_bf16) & 15u) != 0)
    return IDX_EALIGN;
  if ((st = check_device()) != IDX_OK) return st;
  idx::QKPrepArgs a;
  a.pool = view_of(pool);
  a.q = static_cast<const uint16_t*>(q_bf16);
  a.k = static_cast<const uint16_t*>(k_bf16);
  a.n_tokens = n_tokens;
  a.H = H;
  a.w = w;
  a.positions = positions;
  a.cos_sin = cos_sin;
  a.max_pos = max_pos;
  a.neox = rope_neox;
  a.ln_gamma = ln_gamma;
  a.ln_beta = ln_beta;
  a.eps = (double)eps;
  a.slots = slot_mapping;
  a.q_out = q_fp8;
  a.w_out = w_out;
  return hip_status(idx::launch_qk_prep_fp8(a, static_cast<hipStream_t>(stream)));
}

IDX_EXPORT int idx_q_prep_mxfp4(const void* q_bf16, int64_t n_tokens, int32_t H, const int32_t* positions,
                                const float* cos_sin, int32_t max_pos, const float* w, float w_scale,
                                uint8_t* q_packed, uint8_t* q_scale, float* w_out, void* stream) {
  if (n_tokens < 0 || H < 1 || max_pos <= 0) return IDX_EINVAL;
  if (H > idx::kMaxHeads) return IDX_EUNSUPPORTED;
  if (n_tokens > 0 && (!q_bf16 || !positions || !cos_sin || !w || !q_packed || !q_scale || !w_out))
    return IDX_EINVAL;
  if (n_tokens > (int64_t)UINT32_MAX / H) return IDX_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q_packed) & 3u) != 0 || (reinterpret_cast<uintptr_t>(q_scale) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(q_bf16) & 15u) != 0)
    return IDX_EALIGN;
  int st = check_device();
  if (st != IDX_OK) return st;
  idx::QPrepArgs a;
  a.q = static_cast<const uint16_t*>(q_bf16);
  a.n_vecs = n_tokens * H;
  a.H = H;
  a.positions = positions;
  a.cos_sin = cos_sin;
  a.max_pos = max_pos;
  a.w = w;
  a.w_scale = w_scale;
  a.q_out = q_packed;
  a.q_scale = q_scale;
  a.w_out = w_out;
  return hip_status(idx::launch_q_prep_mxfp4(a, static_cast<hipStream_t>(stream)));
}

IDX_EXPORT int idx_q_quant_mxfp4(const void* q_bf16, int64_t n_vecs, uint8_t* q_packed, uint8_t* q_scale,
                                 void* stream) {
  if (n_vecs < 0) return IDX_EINVAL;
  if (n_vecs > 0 && (!q_bf16 || !q_packed || !q_scale)) return IDX_EINVAL;
  if (n_vecs > (int64_t)UINT32_MAX * 64) return IDX_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q_packed) & 15u) != 0) return IDX_EALIGN;
  int st = check_device();
  if (st != IDX_OK) return st;
  return hip_status(idx::launch_q_quant_mxfp4(static_cast<const uint16_t*>(q_bf16), n_vecs, q_packed, q_scale,
                                              static_cast<hipStream_t>(stream)));
}

IDX_EXPORT int idx_q_quant_fp8(const void* q_bf16, const float* w, int64_t n_vecs, uint8_t* q_fp8, float* w_out,
                               void* stream) {
  if (n_vecs < 0) return IDX_EINVAL;
  if (n_vecs > 0 && (!q_bf16 || !w || !q_fp8 || !w_out)) return IDX_EINVAL;
  if (n_vecs > (int64_t)UINT32_MAX * 256) return IDX_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q_fp8) & 3u) != 0) return IDX_EALIGN;
  int st = check_device();
  if (st != IDX_OK) return st;
  return hip_status(idx::launch_q_quant_fp8(static_cast<const uint16_t*>(q_bf16), w, n_vecs, q_fp8, w_out,
                                            static_cast<hipStream_t>(stream)));
}

namespace {

// Scorer argument checks shared by idx_logits_paged and idx_decode_step.
int logits_args(const idx_pool* pool, const uint8_t* q, const uint8_t* q_scale, const float* w,
                const int32_t* page_table, int32_t max_pages_per_seq, const int32_t* ctx_lens, int32_t B, int32_t n_q,
                int32_t H, int32_t D, int32_t max_ctx, float* logits, int64_t logits_stride, idx::LogitsArgs& a) {
  int st = check_pool(pool, -1);
  if (st != IDX_OK) return st;
  if (D != 128) return IDX_EUNSUPPORTED;
  if (H < 1 || H > idx::kMaxHeads) return H < 1 ? IDX_EINVAL : IDX_EUNSUPPORTED;
  if (B < 1 || n_q < 1 || max_ctx < 0 || max_pages_per_seq < 1 || logits_stride < 1) return IDX_EINVAL;
  if (!q || !w || !page_table || !ctx_lens || !logits) return IDX_EINVAL;
  if (pool->kv_format == IDX_KV_MXFP4 && !q_scale) return IDX_EINVAL;
  if ((int64_t)max_ctx > (int64_t)max_pages_per_seq * pool->page_size) return IDX_EINVAL;
  if ((int64_t)max_ctx > logits_stride) return IDX_EINVAL;
  if ((reinterpret_cast<uintptr_t>(q) & 15u) != 0) return IDX_EALIGN;
  if ((int64_t)B * n_q > (int64_t)INT32_MAX) return IDX_EINVAL;
  if ((int64_t)max_ctx > idx::logits_max_ctx(n_q, H, pool->page_size)) return IDX_EUNSUPPORTED;
  a.pool = view_of(pool);
  a.q = q;
  a.q_scale = q_scale;
  a.w = w;
  a.page_table = page_table;
  a.max_pages = max_pages_per_seq;
  a.ctx = ctx_lens;
  a.B = B;
  a.n_q = n_q;
  a.H = H;
  a.max_ctx = max_ctx;
  a.logits = logits;
  a.lstride = logits_stride;
  return IDX_OK;
}

}  // namespace

IDX_EXPORT int idx_logits_paged(const idx_pool* pool, const uint8_t* q, const uint8_t* q_scale, const float* w,
                                const int32_t* page_table, int32_t max_pages_per_seq, const int32_t* ctx_lens,
                                int32_t B, int32_t n_q, int32_t H, int32_t D, int32_t max_ctx, float* logits,
                                int64_t logits_stride, void* workspace, size_t ws_bytes, void* stream) {
  idx::LogitsArgs a;
  int st = logits_args(pool, q, q_scale, w, page_table, max_pages_per_seq, ctx_lens, B, n_q, H, D, max_ctx, logits,
                       logits_stride, a);
  if (st != IDX_OK) return st;
  if ((st = check_workspace(workspace, ws_bytes, 0)) != IDX_OK) return st;
  if ((st = check_device()) != IDX_OK) return st;
  return hip_status(idx::launch_logits(a, static_cast<hipStream_t>(stream), num_cus()));
}

IDX_EXPORT int idx_topk(const float* logits, int64_t logits_stride, const int32_t* ctx_lens, int32_t B, int32_t n_q,
                        int32_t k, int32_t* out_idx, void* workspace, size_t ws_bytes, void* stream) {
  if (!logits || !ctx_lens || !out_idx) return IDX_EINVAL;
  if (B < 1 || n_q < 1 || k < 1 || logits_stride < 1) return IDX_EINVAL;
  if ((int64_t)B * n_q > (int64_t)INT32_MAX) return IDX_EINVAL;
  // the row capacity bounds the row length and sizes the launch
  if (logits_stride > idx::kTopkMaxCtx) return IDX_EUNSUPPORTED;
  int st = check_workspace(workspace, ws_bytes, 0);
  if (st != IDX_OK) return st;
  if ((st = check_device()) != IDX_OK) return st;
  idx::TopkArgs a;
  a.logits = logits;
  a.lstride = logits_stride;
  a.ctx = ctx_lens;
  a.B = B;
  a.n_q = n_q;
  a.max_ctx = (int32_t)logits_stride;
  a.k = k;
  a.out = out_idx;
  return hip_status(idx::launch_topk(a, static_cast<hipStream_t>(stream)));
}

IDX_EXPORT int idx_logits_candidates(const idx_pool* pool, const uint8_t* q, const uint8_t* q_scale, const float* w,
                                     const int32_t* page_table, int32_t max_pages_per_seq, const int32_t* ctx_lens,
                                     int32_t B, int32_t n_q, int32_t H, int32_t D, const int32_t* cand_blocks,
                                     int32_t n_cand, float* logits, int64_t logits_stride, void* stream) {
  if (!pool) return IDX_EINVAL;
  if (n_cand < 0 || (n_cand > 0 && !cand_blocks)) return IDX_EINVAL;
  const int64_t cells = (int64_t)n_cand * pool->page_size;
  if (cells > logits_stride) return IDX_EINVAL;
  // token indices (block id * P + row) must fit an int32
  if ((int64_t)max_pages_per_seq * pool->page_size > (int64_t)INT32_MAX) return IDX_EINVAL;
  if (cells > idx::kTopkMaxCtx) return IDX_EUNSUPPORTED;
  idx::LogitsArgs a;
  // max_ctx is not used by this entry point (cells are bounded by the candidate count)
  int st = logits_args(pool, q, q_scale, w, page_table, max_pages_per_seq, ctx_lens, B, n_q, H, D, 0, logits,
                       logits_stride, a);
  if (st != IDX_OK) return st;
  if ((st = check_device()) != IDX_OK) return st;
  idx::CandArgs c;
  c.cand = cand_blocks;
  c.n_cand = n_cand;
  return hip_status(idx::launch_logits_candidates(a, c, static_cast<hipStream_t>(stream)));
}

IDX_EXPORT int idx_topk_candidates(const float* logits, int64_t logits_stride, const int32_t* cand_blocks,
                                   int32_t n_cand, int32_t page_size, int32_t B, int32_t n_q, int32_t k,
                                   int32_t* out_idx, void* stream) {
  if (!logits || !out_idx || n_cand < 0 || (n_cand > 0 && !cand_blocks)) return IDX_EINVAL;
  if (B < 1 || n_q < 1 || k < 1 || logits_stride < 1) return IDX_EINVAL;
  if (page_size < 16 || page_size > 1024 || (page_size & (page_size - 1)) != 0) return IDX_EUNSUPPORTED;
  const int64_t cells = (int64_t)n_cand * page_size;
  if (cells > logits_stride) return IDX_EINVAL;
  if ((int64_t)B * n_q > (int64_t)INT32_MAX) return IDX_EINVAL;
  if (cells > idx::kTopkMaxCtx) return IDX_EUNSUPPORTED;
  int st = check_device();
  if (st != IDX_OK) return st;
  idx::TopkCandArgs a;
  a.logits = logits;
  a.lstride = logits_stride;
  a.cand = cand_blocks;
  a.n_cand = n_cand;
  a.page_shift = __builtin_ctz((unsigned)page_size);
  a.rows = (int64_t)B * n_q;
  a.k = k;
  a.out = out_idx;
  return hip_status(idx::launch_topk_candidates(a, static_cast<hipStream_t>(stream)));
}

IDX_EXPORT int idx_decode_step_fused(int32_t B, int32_t n_q, int32_t H, int32_t max_ctx) {
  if (B < 1 || n_q < 1 || H < 1 || max_ctx < 0) return IDX_EINVAL;
  if (H > idx::kMaxHeads || !idx::decode_step_supported(n_q, H, max_ctx)) return IDX_EUNSUPPORTED;
  const int st = check_device();
  if (st != IDX_OK) return st;
  return idx::decode_step_fuses(B, n_q, H, max_ctx, num_cus()) ? 1 : 0;
}

IDX_EXPORT size_t idx_workspace_bytes(int32_t B, int32_t n_q, int32_t H, int32_t max_ctx, int32_t k) {
  if (B < 1 || n_q < 1 || H < 1 || k < 1 || max_ctx < 0) return 0;
  return step_workspace_bytes(B);
}

namespace {

// Everything idx_decode_step and idx_decode_step_noalloc share: the argument checks, all
// but the scratch's; fills `a` but the counters.
int decode_step_common(const idx_pool* pool, const void* k_bf16, int64_t row_stride_elems, const float* gamma,
                       float eps, const int32_t* positions, const float* cos_sin, int32_t max_pos,
                       const int64_t* slot_mapping, const uint8_t* q, const uint8_t* q_scale, const float* w,
                       const int32_t* page_table, int32_t max_pages_per_seq, const int32_t* ctx_lens, int32_t B,
                       int32_t n_q, int32_t H, int32_t D, int32_t max_ctx, float* logits, int64_t logits_stride,
                       int32_t k, int32_t* out_idx, idx::StepArgs& a) {
  int st = logits_args(pool, q, q_scale, w, page_table, max_pages_per_seq, ctx_lens, B, n_q, H, D, max_ctx, logits,
                       logits_stride, a.s);
  if (st != IDX_OK) return st;
  if (!k_bf16 || !gamma || !positions || !cos_sin || !slot_mapping || !out_idx) return IDX_EINVAL;
  if (row_stride_elems < 128 || !(eps > 0.0f) || max_pos <= 0 || k < 1) return IDX_EINVAL;
  if (!idx::decode_step_supported(n_q, H, max_ctx)) return IDX_EUNSUPPORTED;
  a.k = static_cast<const uint16_t*>(k_bf16);
  a.row_stride = row_stride_elems;
  a.gamma = gamma;
  a.eps = (double)eps;
  a.positions = positions;
  a.cos_sin = cos_sin;
  a.max_pos = max_pos;
  a.slots = slot_mapping;
  a.k_top = k;
  a.out = out_idx;
  return IDX_OK;
}

}  // namespace

IDX_EXPORT int idx_decode_step(const idx_pool* pool, const void* k_bf16, int64_t row_stride_elems, const float* gamma,
                               float eps, const int32_t* positions, const float* cos_sin, int32_t max_pos,
                               const int64_t* slot_mapping, const uint8_t* q, const uint8_t* q_scale, const float* w,
                               const int32_t* page_table, int32_t max_pages_per_seq, const int32_t* ctx_lens,
                               int32_t B, int32_t n_q, int32_t H, int32_t D, int32_t max_ctx, float* logits,
                               int64_t logits_stride, int32_t k, int32_t* out_idx, void* workspace,
                               size_t workspace_bytes, void* stream) {
  idx::StepArgs a;
  int st = decode_step_common(pool, k_bf16, row_stride_elems, gamma, eps, positions, cos_sin, max_pos, slot_mapping,
                              q, q_scale, w, page_table, max_pages_per_seq, ctx_lens, B, n_q, H, D, max_ctx, logits,
                              logits_stride, k, out_idx, a);
  if (st != IDX_OK) return st;
  if (!workspace) return IDX_EINVAL;
  if ((st = check_workspace(workspace, workspace_bytes, step_workspace_bytes(B))) != IDX_OK) return st;
  if ((st = check_device()) != IDX_OK) return st;
  a.counters = static_cast<int32_t*>(workspace);
  return hip_status(idx::launch_decode_step(a, static_cast<hipStream_t>(stream), num_cus()));
}

// ---------------------------------------------------------------------------------------
// The decode step for callers that cannot allocate: its block counters live in this
// library's own device array.  The array has static storage (zero when the code object
// loads), every device holds its own copy at its own address, and its device address is
// taken once per device with hipGetSymbolAddress on the entry point's first call there.
// Every call leaves the counters it used at zero (the last block of each sequence resets
// its counter), so each call finds them cleared.  Calls that overlap on one device share
// the array and race.
// ---------------------------------------------------------------------------------------
namespace {

static __device__ __align__(256) int32_t scratch[IDX_NOALLOC_MAX_SEQS];

std::atomic<int32_t*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (nullptr if it cannot be had).
int32_t* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  int32_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) {
    (void)hipGetLastError();
    return nullptr;
  }
  p = static_cast<int32_t*>(addr);
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

IDX_EXPORT int idx_decode_step_noalloc(const idx_pool* pool, const void* k_bf16, int64_t row_stride_elems,
                                       const float* gamma, float eps, const int32_t* positions, const float* cos_sin,
                                       int32_t max_pos, const int64_t* slot_mapping, const uint8_t* q,
                                       const uint8_t* q_scale, const float* w, const int32_t* page_table,
                                       int32_t max_pages_per_seq, const int32_t* ctx_lens, int32_t B, int32_t n_q,
                                       int32_t H, int32_t D, int32_t max_ctx, float* logits, int64_t logits_stride,
                                       int32_t k, int32_t* out_idx, void* stream) {
  idx::StepArgs a;
  int st = decode_step_common(pool, k_bf16, row_stride_elems, gamma, eps, positions, cos_sin, max_pos, slot_mapping,
                              q, q_scale, w, page_table, max_pages_per_seq, ctx_lens, B, n_q, H, D, max_ctx, logits,
                              logits_stride, k, out_idx, a);
  if (st != IDX_OK) return st;
  if (B > IDX_NOALLOC_MAX_SEQS) return IDX_ESCRATCH;
  if ((st = check_device()) != IDX_OK) return st;
  int32_t* counters = scratch_for_current_device();
  if (!counters) return IDX_EHIP;
  a.counters = counters;
  return hip_status(idx::launch_decode_step(a, static_cast<hipStream_t>(stream), num_cus()));
}

IDX_EXPORT int idx_diag_fp64(const double* a, const double* b, double* quot, double* root, int64_t n, void* stream) {
  if (n < 0 || (n > 0 && (!a || !b || !quot || !root))) return IDX_EINVAL;
  if (n > (int64_t)UINT32_MAX * 256) return IDX_EINVAL;
  int st = check_device();
  if (st != IDX_OK) return st;
  return hip_status(idx::launch_diag_fp64(a, b, quot, root, n, static_cast<hipStream_t>(stream)));
}

IDX_EXPORT int idx_diag_mfma(int32_t fmt, int32_t blocks, int32_t rounds, float* out, void* stream) {
  if ((fmt != 0 && fmt != 1) || blocks < 1 || rounds < 0 || !out) return IDX_EINVAL;
  int st = check_device();
  if (st != IDX_OK) return st;
  return hip_status(idx::launch_diag_mfma(fmt, blocks, rounds, out, static_cast<hipStream_t>(stream)));
}

IDX_EXPORT int idx_diag_hbm_read(const void* buf, int64_t bytes, int32_t blocks, float* out, void* stream) {
  if (!buf || !out || bytes < 16 || bytes % 16 != 0 || blocks < 1) return IDX_EINVAL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return IDX_EALIGN;
  int st = check_device();
  if (st != IDX_OK) return st;
  return hip_status(idx::launch_diag_read(buf, bytes, blocks, out, static_cast<hipStream_t>(stream)));
}

IDX_EXPORT int idx_device_info(int32_t* cus, int32_t* clock_khz) {
  if (!cus || !clock_khz) return IDX_EINVAL;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return IDX_EHIP;
  }
  int c = 0, k = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&k, hipDeviceAttributeClockRate, dev) != hipSuccess) {
    (void)hipGetLastError();
    return IDX_EHIP;
  }
  *cus = c;
  *clock_khz = k;
  return IDX_OK;
}

IDX_EXPORT int64_t idx_bytes_per_token(int32_t kv_format) { return bytes_per_token(kv_format); }

IDX_EXPORT int idx_device_check(void) { return check_device(); }

IDX_EXPORT const char* idx_status_string(int status) {
  switch (status) {
    case IDX_OK: return "ok";
    case IDX_EINVAL: return "invalid argument";
    case IDX_EUNSUPPORTED: return "unsupported shape, page size or device (needs gfx950, head dim 128)";
    case IDX_EALIGN: return "misaligned pool offset, page stride or buffer";
    case IDX_EHIP: return "HIP runtime error while enqueueing";
    case IDX_ESCRATCH: return "more sequences than the library's static scratch holds (idx_decode_step_noalloc)";
    default: return "unknown status";
  }
}
