/*
 * idx.h — C ABI of the MI355X (gfx950) lightning-indexer hot path.
 *
 * The method (DeepSeek sparse attention's lightning indexer, as run on ROCm in the
 * pages "[ROCm][Perf] Add AITER paged MXFP4 sparse indexing on gfx950" (vllm PR 57517)
 * and "Dense MXFP4 indexer for DeepSeek-V4 on ROCm" (vllm PR 60834)) scores every
 * cached token s against every query token t:
 *
 *     logits[t,s] = sum_h w[t,h] * ReLU( deq(q[t,h]) . deq(k[s]) )
 *
 * with one K row per cached token shared by all heads (MQA), K read in place from a
 * paged cache through a page table (no gather pass), a causal / length mask, and a
 * per-query top-k of the logits.
 *
 * Conventions for every entry point:
 *  - Pointers named as device memory must point to device memory of the current HIP
 *    device; the caller owns all of it.  The library never allocates, frees or
 *    synchronises, and keeps no state between calls apart from a per-device
 *    architecture check done on first use.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the null
 *    stream) and returns before it finishes.  No entry point reads device memory on
 *    the host, so every call can be captured in a HIP graph.
 *  - Return value: IDX_OK, or a negative idx_status.  Argument problems are detected
 *    on the host before anything is enqueued: IDX_EINVAL (null pointer, bad size or
 *    range), IDX_EALIGN (misaligned pool offset / stride), IDX_EUNSUPPORTED (head dim
 *    other than 128, page size not a power of two in [16, 1024], or no gfx950 device,
 *    so the caller can fall back as the pages' FP8 default does).  IDX_EHIP reports a
 *    HIP runtime error while enqueueing.
 *  - Device data that breaks the stated contract (a page id outside the pool, a
 *    context length above max_ctx) is never read out of bounds: such pages score
 *    as NaN and lengths are clamped to max_ctx.
 *  - Scratch memory is the caller's too: the calls that take a (workspace, ws_bytes)
 *    pair use device memory of at least idx_workspace_bytes(...) bytes, zero-filled
 *    once before its first use; every call leaves it zero again, so one buffer serves
 *    every layer and every step (calls sharing it must not overlap in time).
 */
#ifndef IDX_H
#define IDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IDX_OK = 0,
  IDX_EINVAL = -1,
  IDX_EUNSUPPORTED = -2,
  IDX_EALIGN = -3,
  IDX_EHIP = -4,
  IDX_ESCRATCH = -5 /* the call needs more scratch than the library's static array holds */
} idx_status;

/* Indexer K-cache formats.
 *  IDX_KV_MXFP4: 68 B per token — 128 E2M1 values (64 B) and four E8M0 block-32 scales
 *                (page "Dense MXFP4 indexer for DeepSeek-V4 on ROCm", Purpose, gives the
 *                MXFP4 indexer row as 68 B against FP8's 132 B).
 *  IDX_KV_FP8_E4M3: 132 B per token — 128 OCP e4m3 codes and one fp32 per-token scale
 *                (the default FP8 cache that passage compares with). */
typedef enum { IDX_KV_MXFP4 = 0, IDX_KV_FP8_E4M3 = 1 } idx_kv_format;

/* A zero-copy view of a caller-owned physical page pool.  Page "[ROCm][Perf] Add AITER
 * paged MXFP4 sparse indexing on gfx950", Purpose, lists views of the cache taken without
 * copies, explicit page strides into a shared pool, and page rebasing in 64 bits.
 *
 * Physical page `pid` starts at byte  base + offset_bytes + pid * page_stride_bytes,
 * computed in 64 bits, so pools larger than 4 GiB work.  Inside a page of P tokens:
 *   MXFP4: a nibble plane of P rows x 64 B (row r = token r; element 2j in the low
 *          nibble of byte j, 2j+1 in the high nibble), then a scale plane of
 *          P rows x 4 B (E8M0 byte of elements 32b..32b+31 at byte b).
 *   FP8:   a code plane of P rows x 128 B (e4m3, element i at byte i), then P fp32
 *          per-token scales.
 * Bytes of a page beyond 68P (132P) and between pages are never touched. */
typedef struct {
  void* base;                /* device allocation holding the pool */
  int64_t offset_bytes;      /* start of page 0 inside base; >= 0, multiple of 256 */
  int64_t page_stride_bytes; /* distance between pages; >= page bytes, multiple of 256 */
  int64_t num_pages;         /* physical pages addressable through the view; > 0 */
  int32_t page_size;         /* tokens per page P: a power of two in [16, 1024] */
  int32_t kv_format;         /* idx_kv_format */
} idx_pool;

/* ---------------------------------------------------------------------------------
 * K-cache store (MXFP4): per row, RMSNorm over 128 dims, NeoX RoPE on the leading 64
 * dims at the row's position, MXFP4 quantisation per 32-element block, and a store
 * into the row's page slot.  Follows page "Dense MXFP4 indexer for DeepSeek-V4 on
 * ROCm", Changes / K write (normalisation, rotation, MXFP4 packing and the page store
 * happen in one pass with no intermediate written out) and page "[ROCm][Perf] Fuse DSA
 * indexer QK preprocessing with AITER", Purpose (rotation covers the leading 64 dims;
 * rows mapped to the padding slot are skipped).
 *
 * Arithmetic (all fp64; bit-exact against a CPU implementation of the same steps):
 *   r = sqrt(S/128 + eps) with S summed as s_l = x_l^2 + x_{l+64}^2 (l < 64), then
 *   halving s_l += s_{l+w} for w = 32..1;  y_i = (x_i / r) * gamma_i;
 *   z_i = y_i c_i - y_{i+32} n_i,  z_{i+32} = y_{i+32} c_i + y_i n_i  (i < 32),
 *   c_i = cos_sin[pos][i], n_i = cos_sin[pos][32+i];  z_i = y_i for i >= 64;
 *   block scale X = clamp(floor(log2 amax) - 2, -127, 127), E8M0 byte X + 127
 *   (byte 0 when amax = 0); element code = E2M1 round-to-nearest-even of z / 2^X,
 *   saturating at 6, sign bit = IEEE sign of z.
 *
 * pool            IDX_KV_MXFP4 pool (see idx_pool).
 * k_bf16          device, bf16 [n_rows][row_stride_elems] (first 128 elements used).
 * n_rows          >= 0 (0 is a no-op); row_stride_elems >= 128.
 * gamma           device, fp32 [128] RMSNorm weight; eps > 0 (fp32, widened to fp64).
 * positions       device, int32 [n_rows], each in [0, max_pos).
 * cos_sin         device, fp32 [max_pos][64]: 32 cosines then 32 sines per position.
 * slot_mapping    device, int64 [n_rows]: page * P + row; negative = skip the row.
 *                 Rows with a slot outside the pool, or a position outside
 *                 [0, max_pos), are skipped as well.
 * ------------------------------------------------------------------------------- */
int idx_k_store_mxfp4(const idx_pool* pool, const void* k_bf16, int64_t n_rows, int64_t row_stride_elems,
                      const float* gamma, float eps, const int32_t* positions, const float* cos_sin,
                      int32_t max_pos, const int64_t* slot_mapping, void* stream);

/* K-cache store (FP8 e4m3): the same normed, rotated row z, then one fp32 per-token
 * scale sk = fp32(amax(|z|) / 448) and codes e4m3(z_i / sk), round-to-nearest-even,
 * saturating at 448 (sk = 0 and sign-only zero codes for an all-zero row).  The FP8
 * arm of the pages' MXFP4-versus-FP8 comparison (132 B per token).  Arguments as for
 * idx_k_store_mxfp4, with an IDX_KV_FP8_E4M3 pool. */
int idx_k_store_fp8(const idx_pool* pool, const void* k_bf16, int64_t n_rows, int64_t row_stride_elems,
                    const float* gamma, float eps, const int32_t* positions, const float* cos_sin,
                    int32_t max_pos, const int64_t* slot_mapping, void* stream);

/* ---------------------------------------------------------------------------------
 * Q packing for the scorer (page "[ROCm][Perf] Add AITER paged MXFP4 sparse indexing on
 * gfx950", Purpose: the integration produces packed MXFP4 Q with its scale layout).  Quantises n_vecs head vectors of 128
 * bf16 values with the MXFP4 block rule above (no RoPE: the vectors are taken as
 * already rotated).
 * q_bf16   device, bf16 [n_vecs][128].
 * q_packed device, uint8 [n_vecs][64] (element 2j in the low nibble of byte j).
 * q_scale  device, uint8 [n_vecs][4] (E8M0 of blocks 0..3).
 * ------------------------------------------------------------------------------- */
int idx_q_quant_mxfp4(const void* q_bf16, int64_t n_vecs, uint8_t* q_packed, uint8_t* q_scale, void* stream);

/* ---------------------------------------------------------------------------------
 * MXFP4 Q preparation for the scorer: rotation, packing and the weight fold in one op.
 * Page "Dense MXFP4 indexer for DeepSeek-V4 on ROCm", Changes / Q quant: the Q op rotates
 * and packs Q to MXFP4 and emits fp32 weights with the softmax and head scales folded in;
 * page "[ROCm][Perf] Fuse DSA indexer QK preprocessing with AITER", Purpose: RoPE covers
 * the leading rope dims of q as of k.
 *
 * Vector v = t * H + h is head h of token t.  Its leading 64 dims are rotated at
 * positions[t] with the K store's NeoX rotation (pairs (i, i+32), fp64, no fused
 * operations, the same cos_sin table), dims 64..127 pass through, and the result is
 * packed exactly as idx_q_quant_mxfp4 packs a vector (bit-exact against a CPU
 * implementation).  A position outside [0, max_pos) leaves its token's vectors
 * unrotated.  w_out[v] = fp32(w[v] * w_scale), where w_scale is the product of the
 * factors folded in (for example head_dim^-1/2 * H^-1/2).
 *
 * q_bf16     device bf16 [n_tokens][H][128], 16-byte aligned;  positions device int32 [n_tokens];
 * cos_sin    device fp32 [max_pos][64] (32 cosines, 32 sines per position);
 * w          device fp32 [n_tokens][H];  w_out device fp32 [n_tokens][H];
 * q_packed   device uint8 [n_tokens][H][64], 4-byte aligned;
 * q_scale    device uint8 [n_tokens][H][4], 4-byte aligned.
 * n_tokens >= 0 (0 is a no-op); H in [1, 128].
 * ------------------------------------------------------------------------------- */
int idx_q_prep_mxfp4(const void* q_bf16, int64_t n_tokens, int32_t H, const int32_t* positions, const float* cos_sin,
                     int32_t max_pos, const float* w, float w_scale, uint8_t* q_packed, uint8_t* q_scale, float* w_out,
                     void* stream);

/* ---------------------------------------------------------------------------------
 * FP8 QK preparation in one launch (page "[ROCm][Perf] Fuse DSA indexer QK preprocessing
 * with AITER", Purpose: the indexer's five pre-processing steps — LayerNorm on k, RoPE on
 * the leading rope dims of q and k, per-token-group FP8 quantisation of q, the q scale
 * folded into the weights, FP8 quantisation of k with the paged cache write — as one
 * kernel; Test Plan: NeoX and interleaved rotation layouts, and the rows the op skips
 * left at zero).  For token t (all arithmetic fp64, no fused operations):
 *   k: mu = S(x)/128, d = x - mu, r = sqrt(S(d^2)/128 + eps), y = (d / r) * ln_gamma +
 *      ln_beta (S sums in the K store's fold-then-halve order); dims 0..63 rotated at
 *      positions[t] (below); FP8 row as idx_k_store_fp8 (sk = fp32(amax/448), e4m3
 *      codes) stored at slot_mapping[t] of the FP8 pool;
 *   q: each head vector [t][h] rotated as loaded, then sq = fp32(amax/448), codes
 *      e4m3(q/sq) to q_fp8[t][h], w_out[t][h] = fp32(w[t][h] * sq) (idx_q_quant_fp8);
 *   rotation: pairs (i, i+32) when rope_neox = 1, (2i, 2i+1) when 0, i < 32; pair i
 *      turns by (cos_sin[pos][i], cos_sin[pos][32+i]): a' = a c - b n, b' = b c + a n;
 *   a token whose slot is negative (padding), outside the pool, or whose position is
 *      outside [0, max_pos) is skipped: no K is stored, its q_fp8 bytes and w_out are 0.
 * pool: FP8 (IDX_EINVAL otherwise).  q_bf16 device bf16 [n_tokens][H][128], 16-byte aligned; k_bf16 device
 * bf16 [n_tokens][128]; w, w_out device fp32 [n_tokens][H] (w_out may alias w);
 * positions int32 [n_tokens]; cos_sin fp32 [max_pos][64]; ln_gamma, ln_beta fp32 [128];
 * eps > 0; slot_mapping int64 [n_tokens]; q_fp8 device uint8 [n_tokens][H][128], 4-byte
 * aligned.  n_tokens >= 0 (0 is a no-op); H in [1, 128]; n_tokens * (H + 1) < 2^26.
 * ------------------------------------------------------------------------------- */
int idx_qk_prep_fp8(const idx_pool* pool, const void* q_bf16, const void* k_bf16, int64_t n_tokens, int32_t H,
                    const float* w, const int32_t* positions, const float* cos_sin, int32_t max_pos,
                    int32_t rope_neox, const float* ln_gamma, const float* ln_beta, float eps,
                    const int64_t* slot_mapping, uint8_t* q_fp8, float* w_out, void* stream);

/* FP8 Q with one scale per 128-dim head vector, multiplied into that head's weight
 * (page "[ROCm][Perf] Fuse DSA indexer QK preprocessing with AITER", Purpose: q is FP8
 * quantised per token group and its scale is then folded into the indexer weights):
 * sq = fp32(amax / 448), q_fp8[i] = e4m3(q[i] / sq), w_out = fp32(w * sq).
 * q_bf16 device bf16 [n_vecs][128]; w device fp32 [n_vecs]; q_fp8 device uint8
 * [n_vecs][128]; w_out device fp32 [n_vecs] (may alias w). */
int idx_q_quant_fp8(const void* q_bf16, const float* w, int64_t n_vecs, uint8_t* q_fp8, float* w_out,
                    void* stream);

/* ---------------------------------------------------------------------------------
 * Paged MQA logits with the causal / length mask — the scorer.  Page "Dense MXFP4
 * indexer for DeepSeek-V4 on ROCm", Purpose: the MQA-logits kernel reads the paged
 * cache where it lies, so prefill needs no K gather; page "[ROCm][Perf] Add AITER paged
 * MXFP4 sparse indexing on gfx950", Performance and accuracy: the isolated scorer
 * timed at decode and prefill shapes.
 *
 * Rows: r = b * n_q + j is query token j of sequence b; its valid length is
 *   n_r = clamp(ctx_lens[b] - n_q + 1 + j, 0, ctx_lens[b])
 * (the n_q query tokens are the sequence's last n_q tokens, causal among
 * themselves: decode n_q = 1, speculative verification n_q > 1, prefill n_q = ctx).
 * For s < n_r:  logits[r * logits_stride + s] =
 *   sum_h w[r*H + h] * max(0, sum_i deq(q[r,h])_i * deq(k_b[s])_i),
 * k_b[s] read from physical page page_table[b * max_pages_per_seq + s / P], row s % P.
 * Cells s >= n_r are not written.  Accumulation is fp32 (MFMA), results fp32.
 *
 * pool             MXFP4 or FP8 pool.
 * q                device.  MXFP4: uint8 [B][n_q][H][64] packed E2M1;
 *                  FP8: uint8 [B][n_q][H][128] e4m3.
 * q_scale          device uint8 [B][n_q][H][4] E8M0 for MXFP4; ignored (may be NULL) for FP8.
 * w                device fp32 [B][n_q][H] with every per-head factor already
 *                  multiplied in (page "Dense MXFP4 indexer for DeepSeek-V4 on ROCm",
 *                  Changes / Q quant: the Q op emits fp32 weights that carry the
 *                  softmax and head scales).
 * page_table       device int32 [B][max_pages_per_seq] physical page ids.
 * ctx_lens         device int32 [B], each in [0, max_ctx].
 * B, n_q >= 1; H in [1, 128]; D must be 128.
 * max_ctx          host upper bound of ctx_lens (sizes the launch; no device read on
 *                  the host); 0 <= max_ctx <= max_pages_per_seq * P and <= logits_stride.
 *                  When n_q * ceil(H/16) > 16 (the prefill form) max_ctx is limited to
 *                  16384 * P (IDX_EUNSUPPORTED beyond).
 * logits           device fp32 [B * n_q][logits_stride].
 * workspace        device scratch of ws_bytes bytes, sized by idx_workspace_bytes.  No
 *                  shape this call takes today uses it, so workspace = NULL with
 *                  ws_bytes = 0 is accepted; a non-NULL workspace must be 256-byte
 *                  aligned (IDX_EALIGN), and NULL with ws_bytes > 0 is IDX_EINVAL.
 * ------------------------------------------------------------------------------- */
int idx_logits_paged(const idx_pool* pool, const uint8_t* q, const uint8_t* q_scale, const float* w,
                     const int32_t* page_table, int32_t max_pages_per_seq, const int32_t* ctx_lens, int32_t B,
                     int32_t n_q, int32_t H, int32_t D, int32_t max_ctx, float* logits, int64_t logits_stride,
                     void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Per-row top-k of the logits (page "Dense MXFP4 indexer for DeepSeek-V4 on ROCm",
 * Purpose: the V4 indexer keeps the best 1024 tokens per query; page "[ROCm][Perf]
 * Fuse DSA indexer QK preprocessing with AITER", Purpose: the selected indices land in
 * a top-k index buffer).  For row r with valid length n_r (rule above):
 *   n_r <= k: out_idx[r][0..n_r) = 0..n_r-1, the rest -1;
 *   n_r >  k: the k token indices with the largest logits, equal logits broken
 *             toward the smaller index (-0.0 equals +0.0).  The order of the k indices
 *             within the row is unspecified but deterministic (the same input gives the
 *             same bytes).
 * Only cells s < n_r are read.  NaN logits are outside the contract.
 * logits   device fp32 [B * n_q][logits_stride]; logits_stride is also the host bound
 *          of the row length that sizes the launch (no device read on the host):
 *          ctx_lens above it are clamped to it; at most 65536 (IDX_EUNSUPPORTED beyond).
 * ctx_lens device int32 [B];  k >= 1;  out_idx device int32 [B * n_q][k].
 * workspace, ws_bytes  scratch, with the same rules as for idx_logits_paged (no shape
 *          this call takes today uses it).
 * ------------------------------------------------------------------------------- */
int idx_topk(const float* logits, int64_t logits_stride, const int32_t* ctx_lens, int32_t B, int32_t n_q,
             int32_t k, int32_t* out_idx, void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Device scratch the hot path's calls need for one shape: the largest of what
 * idx_logits_paged, idx_topk and idx_decode_step take for B sequences of n_q query
 * rows, H heads, contexts up to max_ctx and top-k k (a multiple of 256; 0 when B, n_q,
 * H or k is below 1 or max_ctx is negative).  Page "[ROCm][Perf] Add AITER paged MXFP4
 * sparse indexing on gfx950", Purpose: the cache is read through views with no copies
 * and the schedule stays fixed under graph replay; page "Dense MXFP4 indexer for
 * DeepSeek-V4 on ROCm" review discussion: one persistent scratch buffer shared by the
 * indexer layers.  The buffer is zero-filled once by the caller and every call leaves
 * it zero (see the conventions above).  Today only idx_decode_step uses it (one block
 * counter per sequence); the scorer and the top-k keep the pair so that a form needing
 * scratch changes no caller.
 * ------------------------------------------------------------------------------- */
size_t idx_workspace_bytes(int32_t B, int32_t n_q, int32_t H, int32_t max_ctx, int32_t k);

/* ---------------------------------------------------------------------------------
 * Candidate-block scorer: the second level of a two-level indexer, where each query
 * row scores only the blocks a first level chose for it (page "Dense MXFP4 indexer for
 * DeepSeek-V4 on ROCm", Purpose: the candidate-pool path beside the dense one, which is
 * the same scorer called with no candidate blocks).  The pages do not define a candidate
 * block; here it is one page-sized run of the row's sequence, named by its index in the
 * sequence's page table, and read in place from the page that entry names.
 *
 * Row r = b * n_q + j (valid length n_r as for idx_logits_paged) has candidate ids
 * cand_blocks[r * n_cand + c], c < n_cand (negative = padding).  Every cell
 * c * P + i (i < P) of the row's logits is written:
 *   logits[r * logits_stride + c*P + i] = the idx_logits_paged logit of token
 *       s = cand * P + i  when 0 <= cand < max_pages_per_seq and s < n_r,
 *   = -inf otherwise (padding ids, ids past the page table, tokens past n_r).
 * A page id outside the pool scores NaN, as in idx_logits_paged.  The ids of a row
 * should be distinct (a repeated id repeats its cells).
 * Arguments as for idx_logits_paged (max_ctx is not taken: the candidate count bounds
 * the cells), plus cand_blocks device int32 [B * n_q][n_cand] and n_cand >= 0;
 * n_cand * P <= logits_stride, n_cand * P <= 65536 (IDX_EUNSUPPORTED beyond) and
 * max_pages_per_seq * P < 2^31.
 * ------------------------------------------------------------------------------- */
int idx_logits_candidates(const idx_pool* pool, const uint8_t* q, const uint8_t* q_scale, const float* w,
                          const int32_t* page_table, int32_t max_pages_per_seq, const int32_t* ctx_lens, int32_t B,
                          int32_t n_q, int32_t H, int32_t D, const int32_t* cand_blocks, int32_t n_cand,
                          float* logits, int64_t logits_stride, void* stream);

/* Per-row top-k over candidate cells (the logits idx_logits_candidates writes): cells
 * holding -inf are not candidates; among the others, the k with the largest logits, as
 * token indices cand_blocks[r][c] * P + i.  A row with at most k candidate cells outputs
 * all of their tokens, then -1.  Equal logits go to the earlier cell (the smaller token
 * when a row's ids ascend); the order within a row is unspecified but deterministic.  NaN
 * logits (a page id outside the pool) are outside the contract, as for idx_topk.
 * logits device fp32 [B * n_q][logits_stride]; cand_blocks device int32 [B * n_q][n_cand];
 * page_size P as the pool's; n_cand * P <= logits_stride and <= 65536; k >= 1;
 * out_idx device int32 [B * n_q][k]. */
int idx_topk_candidates(const float* logits, int64_t logits_stride, const int32_t* cand_blocks, int32_t n_cand,
                        int32_t page_size, int32_t B, int32_t n_q, int32_t k, int32_t* out_idx, void* stream);

/* ---------------------------------------------------------------------------------
 * Fused decode step: the K store of the step's new rows, the scorer and the top-k in
 * one launch.  The pages run these as separate launches per indexer layer (page "Dense
 * MXFP4 indexer for DeepSeek-V4 on ROCm", Changes: the K write, then the MQA-logits
 * kernel; Purpose: top-k 1024), and at decode sizes each is dominated by launch and
 * dependency latency.  The result equals
 *   idx_k_store_{mxfp4|fp8}(rows 0..B*n_q-1)  then  idx_logits_paged  then  idx_topk
 * on the same arguments (the same pool bytes, the same logits bits, the same indices),
 * given the contract below.
 *
 * New rows: row i = b * n_q + j of k_bf16 / positions / slot_mapping is the K row of
 * token t = ctx_lens[b] - n_q + j of sequence b (the sequence's newest n_q tokens, as in
 * a decode step where ctx_lens already counts them).  A non-negative slot must be the
 * slot the page table maps token t to: page_table[b][t / P] * P + t % P (other slots
 * give unspecified logits for the step and may race with reads of the pool).  Rows with
 * t < 0, a negative slot, a slot outside the pool or a position outside [0, max_pos)
 * are not stored, exactly as idx_k_store skips them.
 *
 * Arguments are those of idx_k_store_* (the pool's format selects MXFP4 or FP8),
 * idx_logits_paged and idx_topk, plus:
 * workspace        device memory of at least idx_workspace_bytes(B, n_q, H, max_ctx, k)
 *                  bytes, 256-byte aligned, zero-filled before its first use; every call
 *                  leaves it zero again.  Calls that share a workspace must not overlap
 *                  (the per-sequence block counters live there).
 * Supported shapes (else IDX_EUNSUPPORTED, before anything is enqueued): the scorer's
 * decode form, n_q * ceil(H/16) <= 16, and max_ctx <= 65536.
 * Execution: one kernel of 1024-thread blocks, each scoring 2048 tokens of a sequence,
 * when n_q * ceil(H/16) <= 2, max_ctx <= 16384 and that grid (ceil(max_ctx / 2048) * B
 * blocks) fits the device's CU count; otherwise the K store, scorer and top-k kernels run
 * one after another, with the same results (the fused launch pays off only while every
 * block has a CU to itself and its registers hold the query tiles).
 * ------------------------------------------------------------------------------- */
int idx_decode_step(const idx_pool* pool, const void* k_bf16, int64_t row_stride_elems, const float* gamma,
                    float eps, const int32_t* positions, const float* cos_sin, int32_t max_pos,
                    const int64_t* slot_mapping, const uint8_t* q, const uint8_t* q_scale, const float* w,
                    const int32_t* page_table, int32_t max_pages_per_seq, const int32_t* ctx_lens, int32_t B,
                    int32_t n_q, int32_t H, int32_t D, int32_t max_ctx, float* logits, int64_t logits_stride,
                    int32_t k, int32_t* out_idx, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * The fused decode step for callers that cannot allocate device memory (code under HIP
 * graph capture that must not call hipMalloc, tight serving loops, harnesses that forbid
 * allocation): idx_decode_step with the same arguments and results, minus the workspace.
 * Its per-sequence block counters live in a static device array inside this library
 * (IDX_NOALLOC_MAX_SEQS int32 counters, 64 KiB per device, held by every device the
 * library runs on until the process ends); the caller still passes every input and
 * output.  The array starts zero and every call leaves it zero.  Calls that overlap in
 * time on one device share the array and race: serialise them (one stream, or events).
 * IDX_ESCRATCH when B > IDX_NOALLOC_MAX_SEQS; IDX_EHIP if the array's device address
 * cannot be obtained; otherwise the statuses of idx_decode_step.  Allocates nothing.
 * ------------------------------------------------------------------------------- */
#define IDX_NOALLOC_MAX_SEQS 16384
int idx_decode_step_noalloc(const idx_pool* pool, const void* k_bf16, int64_t row_stride_elems, const float* gamma,
                            float eps, const int32_t* positions, const float* cos_sin, int32_t max_pos,
                            const int64_t* slot_mapping, const uint8_t* q, const uint8_t* q_scale, const float* w,
                            const int32_t* page_table, int32_t max_pages_per_seq, const int32_t* ctx_lens, int32_t B,
                            int32_t n_q, int32_t H, int32_t D, int32_t max_ctx, float* logits, int64_t logits_stride,
                            int32_t k, int32_t* out_idx, void* stream);

/* How idx_decode_step runs this shape on the current device: 1 = the one fused kernel,
 * 0 = the K store, scorer and top-k kernels in sequence; IDX_EUNSUPPORTED for a shape it
 * does not take (or no gfx950 device), IDX_EINVAL for B, n_q or H below 1 or max_ctx < 0.
 * Host-only; for callers and benchmarks that report which kernels ran. */
int idx_decode_step_fused(int32_t B, int32_t n_q, int32_t H, int32_t max_ctx);


/* Diagnostic: quot[i] = a[i] / b[i] and root[i] = sqrt(a[i]) in fp64 on the device,
 * with the same division and square-root operations the K store uses, so a test can
 * confirm that they round exactly as IEEE-754 prescribes (the K store's bit-exactness
 * rests on it).  Device fp64 arrays of n elements. */
int idx_diag_fp64(const double* a, const double* b, double* quot, double* root, int64_t n, void* stream);

/* Diagnostic: blocks x 256 threads, every wave running 8 * rounds independent scaled
 * 16x16x128 MFMAs on register operands (fmt 0: E2M1 x E2M1, 1: e4m3 x e4m3), so a
 * caller timing it gets the sustained matrix rate next to the nominal peak (each MFMA is
 * 2 * 16 * 16 * 128 flops).  out: device fp32 [blocks * 256] (values meaningless, written
 * so nothing is dead).  IDX_EINVAL for another fmt, blocks < 1, rounds < 0 or out NULL. */
int idx_diag_mfma(int32_t fmt, int32_t blocks, int32_t rounds, float* out, void* stream);

/* Diagnostic: a plain streaming read of `bytes` bytes at buf (device, 16-byte aligned,
 * bytes a positive multiple of 16) by blocks x 256 threads, 16-byte non-temporal loads
 * with eight in flight per thread and no arithmetic to speak of, so a caller timing it gets
 * the HBM read rate a kernel can reach on this device next to the nominal 8 TB/s (and the
 * rate for a transfer of a given size, start-up included).  out: device fp32
 * [blocks * 256] (values meaningless).  IDX_EINVAL / IDX_EALIGN for bad arguments. */
int idx_diag_hbm_read(const void* buf, int64_t bytes, int32_t blocks, float* out, void* stream);

/* The current device's compute-unit count and peak shader clock (kHz), as the runtime
 * reports them.  IDX_EINVAL for a NULL pointer, IDX_EHIP when the runtime query fails. */
int idx_device_info(int32_t* cus, int32_t* clock_khz);

/* Bytes per token of a format (68, 132), or -1 for an unknown format. */
int64_t idx_bytes_per_token(int32_t kv_format);

/* IDX_OK when the current HIP device is gfx950, IDX_EUNSUPPORTED otherwise
 * (including when no device is present). */
int idx_device_check(void);

/* Static description of a status code; never NULL. */
const char* idx_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* IDX_H */
