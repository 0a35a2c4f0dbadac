// Host-side launchers of the gfx950 kernels (defined next to each kernel) and the
// argument bundles they take.  Arguments reaching these functions have already been
// validated by the C-ABI layer (api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idx {

// A validated view of a physical page pool: page pid lives at
// base + offset + pid * stride (64-bit arithmetic on the host and in the kernels).
struct PoolView {
  uint8_t* base;        // base + offset_bytes, pre-added
  int64_t stride;       // bytes between pages
  int64_t num_pages;
  int32_t page_size;    // tokens per page (a power of two)
  int32_t page_shift;   // log2(page_size)
  int32_t kv_format;    // 0 MXFP4, 1 FP8
};

struct KStoreArgs {
  PoolView pool;
  const uint16_t* k;
  int64_t n_rows;
  int64_t row_stride;
  const float* gamma;
  double eps;
  const int32_t* positions;
  const float* cos_sin;
  int32_t max_pos;
  const int64_t* slots;
  // Decode-step rows (optional): row i = b*step_n_q + j is token
  // clamp(ctx[b], 0, step_max_ctx) - step_n_q + j and is skipped when that is negative.
  const int32_t* step_ctx = nullptr;
  int32_t step_n_q = 0;
  int32_t step_max_ctx = 0;
};

// FP8 QK preparation: T tokens, H query heads per token.
struct QKPrepArgs {
  PoolView pool;          // FP8 pool
  const uint16_t* q;      // bf16 [T][H][128]
  const uint16_t* k;      // bf16 [T][128]
  int64_t n_tokens;
  int32_t H;
  const float* w;         // [T][H]
  const int32_t* positions;
  const float* cos_sin;   // [max_pos][64]
  int32_t max_pos;
  int32_t neox;           // 1: pairs (i, i+32); 0: pairs (2i, 2i+1)
  const float* ln_gamma;  // [128]
  const float* ln_beta;   // [128]
  double eps;
  const int64_t* slots;
  uint8_t* q_out;         // e4m3 [T][H][128]
  float* w_out;           // [T][H]
};
hipError_t launch_qk_prep_fp8(const QKPrepArgs& a, hipStream_t s);

struct LogitsArgs {
  PoolView pool;
  const uint8_t* q;
  const uint8_t* q_scale;
  const float* w;
  const int32_t* page_table;
  int32_t max_pages;
  const int32_t* ctx;
  int32_t B, n_q, H, max_ctx;
  float* logits;
  int64_t lstride;
};

struct TopkArgs {
  const float* logits;
  int64_t lstride;
  const int32_t* ctx;
  int32_t B, n_q, max_ctx, k;
  int32_t* out;
};

// MXFP4 Q preparation: vector v = t*H + h (head h of token t), rotated at positions[t].
struct QPrepArgs {
  const uint16_t* q;  // [n_vecs][128] bf16
  int64_t n_vecs;
  int32_t H;
  const int32_t* positions;  // [n_vecs / H]
  const float* cos_sin;
  int32_t max_pos;
  const float* w;  // [n_vecs]
  float w_scale;
  uint8_t* q_out;    // [n_vecs][64]
  uint8_t* q_scale;  // [n_vecs][4]
  float* w_out;      // [n_vecs]
};

hipError_t launch_k_store(const KStoreArgs& a, hipStream_t s);
hipError_t launch_q_prep_mxfp4(const QPrepArgs& a, hipStream_t s);
hipError_t launch_q_quant_mxfp4(const uint16_t* q, int64_t n_vecs, uint8_t* qp, uint8_t* qs, hipStream_t s);
hipError_t launch_q_quant_fp8(const uint16_t* q, const float* w, int64_t n_vecs, uint8_t* q8, float* wo,
                              hipStream_t s);
hipError_t launch_logits(const LogitsArgs& a, hipStream_t s, int num_cus = 256);
// Streaming decode scorer: workers (a wave for n_q = 1, a block of n_q row waves for
// n_q = 2..4) take balanced contiguous runs of 64-token chunks of one sequence, the next
// chunk's K in flight while the current one is scored.
hipError_t launch_logits_stream(const LogitsArgs& a, int num_cus, hipStream_t s);
// Whether the streaming scorer takes this shape (n_q <= 4, B <= 1024, chunk counts in int32).
bool logits_stream_takes(int B, int n_q, int max_ctx);
// Whether the scorer takes its decode form (all query rows of a sequence in registers).
bool logits_uses_decode_kernel(int n_q, int H);
// Largest max_ctx the scorer accepts for this shape (the prefill form splits the context
// into at most 256 chunks of at most 64 pages).
int64_t logits_max_ctx(int n_q, int H, int page_size);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

// Candidate blocks of each query row: cand[r][c] is a block (page-table) index of row
// r's sequence, negative = padding.  Cell c*P + i of the row's logits is token
// cand[r][c]*P + i.
struct CandArgs {
  const int32_t* cand;  // [rows][n_cand]
  int32_t n_cand;
};
hipError_t launch_logits_candidates(const LogitsArgs& a, const CandArgs& c, hipStream_t s);

// Top-k over candidate cells: row r has n_cand*P cells; -inf cells are not candidates.
struct TopkCandArgs {
  const float* logits;
  int64_t lstride;
  const int32_t* cand;
  int32_t n_cand;
  int32_t page_shift;
  int64_t rows;
  int32_t k;
  int32_t* out;
};
hipError_t launch_topk_candidates(const TopkCandArgs& a, hipStream_t s);

// The fused decode step: K store of the B*n_q new rows, scorer, top-k, in one launch.
// Row i = b*n_q + j of k/positions/slots is token ctx[b] - n_q + j of sequence b.
struct StepArgs {
  LogitsArgs s;
  const uint16_t* k;
  int64_t row_stride;
  const float* gamma;
  double eps;
  const int32_t* positions;
  const float* cos_sin;
  int32_t max_pos;
  const int64_t* slots;
  int32_t k_top;
  int32_t* out;
  int32_t* counters;  // [B] block counters: zero on entry, left zero on exit
};
// Whether the decode step takes this shape: the scorer's decode form (n_q * ceil(H/16) <=
// 16 query head tiles per sequence) and rows the top-k takes (max_ctx <= 65536).  It runs
// fused for up to 2 head tiles and rows of up to 16384 tokens, else as three kernels.
bool decode_step_supported(int n_q, int H, int64_t max_ctx);
// Whether a supported step runs as the one fused kernel (else as three kernels).
bool decode_step_fuses(int B, int n_q, int H, int max_ctx, int num_cus);
hipError_t launch_decode_step(const StepArgs& a, hipStream_t s, int num_cus);
// 8 * rounds MFMAs (16x16x128, fmt 0: E2M1 x E2M1, 1: e4m3 x e4m3) per wave on register
// operands; out gets blocks * 256 floats.
hipError_t launch_diag_mfma(int fmt, int blocks, int rounds, float* out, hipStream_t s);
// Plain streaming read of `bytes` (a multiple of 16) at buf; out gets blocks * 256 floats.
hipError_t launch_diag_read(const void* buf, int64_t bytes, int blocks, float* out, hipStream_t s);
hipError_t launch_diag_fp64(const double* a, const double* b, double* quot, double* root, int64_t n,
                            hipStream_t s);

// Largest context the top-k kernel supports (registers hold a row: 1024 threads x 64).
constexpr int32_t kTopkMaxCtx = 65536;
// Largest head count the scorer supports (8 head tiles of 16).
constexpr int32_t kMaxHeads = 128;

}  // namespace idx
