/*
 * Oracle for the lightning-indexer hot path: a plain, slow, fp64 CPU implementation.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code, header,
 * table or helper with the HIP library; the two meet only through the byte layouts
 * and formulas written out below, each taken from the pages that define the method:
 *
 *   [p1] "[ROCm][Perf] Add AITER paged MXFP4 sparse indexing on gfx950"
 *        (vllm PR 57517) — Purpose; Performance and accuracy (isolated scorer table
 *        and its accuracy column).
 *   [p2] "Dense MXFP4 indexer for DeepSeek-V4 on ROCm" (vllm PR 60834) — Purpose
 *        (an MXFP4 indexer row is 68 B against FP8's 132 B; the MQA-logits kernel
 *        reads the cache in place; V4's packer uses cvt.rn.satfinite.e2m1x2);
 *        Changes / K write (normalise, rotate, pack, store to the page in one pass);
 *        Changes / Q quant (the fp32 weights arrive with softmax and head scales
 *        multiplied in).
 *   [p3] "[ROCm][Perf] Fuse DSA indexer QK preprocessing with AITER" (vllm PR 53094)
 *        — Purpose (RoPE on the leading rope dims; per-token-group FP8 quantisation
 *        of q with the q scale folded into the weights; rows with a pad slot skipped).
 *
 * The logits formula logits[t,s] = sum_h w[t,h] * ReLU(deq(q[t,h]) . deq(k[s])) is the
 * lightning-indexer MQA score the pages name (p2 Purpose: "mqa_logits"; one K row per
 * cached token shared by every head).  Where the pages leave a step open, the reading
 * taken is stated at the function that implements it.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared (no fast-math: every
 * floating-point operation below is one IEEE double operation, in the order written).
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL -1

#define HEAD_DIM 128
#define ROPE_DIM 64
#define MX_BLOCK 32

/* ------------------------------------------------------------------------------ */
/* Codecs                                                                          */
/* ------------------------------------------------------------------------------ */

/* E2M1 (OCP MX FP4): bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Exponent 0 is subnormal: magnitude m * 0.5.  Otherwise 2^(e-1) * (1 + m/2).
 * [p2 Purpose: the K cache is MXFP4; cvt...e2m1x2 packs two E2M1 values per byte] */
double orc_e2m1_decode(unsigned nibble) {
  unsigned e = (nibble >> 1) & 3u, m = nibble & 1u;
  double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return (nibble & 8u) ? -mag : mag;
}

/* E8M0 block scale: byte b stands for 2^(b-127); 0xFF is NaN in the MX format and is
 * never produced by the quantiser below. */
double orc_e8m0_decode(unsigned byte) {
  if (byte == 0xFFu) return NAN;
  return ldexp(1.0, (int)byte - 127);
}

/* OCP FP8 e4m3 ("e4m3fn"): bias 7, no infinities, S.1111.111 is NaN, largest finite
 * magnitude 448; exponent field 0 is subnormal with magnitude m/8 * 2^-6.
 * [p1 Purpose: FP8 remains the default indexer cache; p2 Purpose: 132 B per token] */
double orc_e4m3_decode(unsigned byte) {
  unsigned e = (byte >> 3) & 15u, m = byte & 7u;
  if (e == 15u && m == 7u) return NAN;
  double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return (byte & 0x80u) ? -mag : mag;
}

/* Round |u| to the E2M1 magnitude grid {0, .5, 1, 1.5, 2, 3, 4, 6}: the nearest grid
 * value, an exact midpoint going to the code with an even mantissa bit ("rn"), and
 * anything beyond 6 held at 6 ("satfinite") [p2 Purpose: cvt.rn.satfinite.e2m1x2].
 * Written as a search over the eight codes so it reads as the definition. */
static unsigned e2m1_code_of_magnitude(double a) {
  unsigned best = 0;
  double best_d = INFINITY;
  for (unsigned c = 0; c < 8; ++c) {
    double d = fabs(a - orc_e2m1_decode(c));
    if (d < best_d || (d == best_d && (c & 1u) == 0u)) { best = c; best_d = d; }
  }
  return best;
}

/* Quantise one block of 32 values to MXFP4.
 * Scale: X = floor(log2(amax)) - 2, clamped to [-127, 127], stored as E8M0 byte X+127
 * (the MX rule that puts amax/2^X in [4, 8), i.e. just above the largest E2M1 value
 * 6, so the largest element may saturate).  amax == 0 gives byte 0.
 * Element: u = v / 2^X (exact scaling by a power of two), code = rn-satfinite(|u|),
 * sign bit = the IEEE sign bit of v (so -0.0 and small negatives that round to zero
 * keep bit 3 set).  Output: 16 bytes, element 2j in the low nibble of byte j. */
void orc_mxfp4_quant_block(const double* v, uint8_t* nib16, uint8_t* scale_byte) {
  double amax = 0.0;
  for (int i = 0; i < MX_BLOCK; ++i) {
    double a = fabs(v[i]);
    if (a > amax) amax = a;
  }
  int X;
  if (amax == 0.0) {
    X = -127;
  } else {
    int e;
    (void)frexp(amax, &e); /* amax = f * 2^e with f in [0.5, 1): floor(log2 amax) = e-1 */
    X = (e - 1) - 2;
    if (X < -127) X = -127;
    if (X > 127) X = 127;
  }
  *scale_byte = (uint8_t)(X + 127);
  for (int j = 0; j < MX_BLOCK / 2; ++j) {
    unsigned nib[2];
    for (int t = 0; t < 2; ++t) {
      double x = v[2 * j + t];
      double u = ldexp(x, -X);
      unsigned c = e2m1_code_of_magnitude(fabs(u));
      if (signbit(x)) c |= 8u;
      nib[t] = c;
    }
    nib16[j] = (uint8_t)(nib[0] | (nib[1] << 4));
  }
}

/* e4m3 round-to-nearest-even with saturation at +-448: the nearest finite e4m3 value,
 * ties to the code with an even last bit, magnitudes beyond 448 held at 448.  Searched
 * over all 127 finite non-negative codes.  Sign bit copied from v. */
uint8_t orc_e4m3_encode(double v) {
  double a = fabs(v);
  unsigned best = 0;
  double best_d = INFINITY;
  for (unsigned c = 0; c < 0x7Fu; ++c) {
    double d = fabs(a - orc_e4m3_decode(c));
    if (d < best_d || (d == best_d && (c & 1u) == 0u)) { best = c; best_d = d; }
  }
  return (uint8_t)(best | (signbit(v) ? 0x80u : 0u));
}

static double bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ------------------------------------------------------------------------------ */
/* Page layout of the indexer K cache (this library's own; the pages leave it to   */
/* the implementation, AITER's preshuffled order being prior art only)             */
/* ------------------------------------------------------------------------------ */
/* A physical page holding P tokens starts at  base + offset + pid * stride.
 *  MXFP4 (68 B/token [p2 Purpose]): nibble plane of P rows x 64 B (row r = token r,
 *         element 2j in the low nibble of byte j), then a scale plane of P rows x 4 B
 *         (E8M0 of blocks 0..3).  Page bytes 68 P.
 *  FP8   (132 B/token [p2 Purpose, Test Result]): code plane of P rows x 128 B e4m3,
 *         then P fp32 per-token scales.  Page bytes 132 P. */
#define FMT_MXFP4 0
#define FMT_FP8 1

/* Threads the parallel loops below use (for reporting the CPU baseline honestly). */
int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int64_t orc_bytes_per_token(int fmt) { return fmt == FMT_MXFP4 ? 68 : (fmt == FMT_FP8 ? 132 : -1); }

/* ------------------------------------------------------------------------------ */
/* K store: RMSNorm -> NeoX RoPE on the leading 64 dims -> quantise -> page store    */
/* [p2 Changes / K write; p3 Purpose for RoPE on the leading rope dims and the pad  */
/* slot skip]                                                                       */
/* ------------------------------------------------------------------------------ */
/* Reading of the steps the pages leave open (all arithmetic in fp64, never narrowed
 * before the quantiser decides a code):
 *   RMSNorm over the 128 dims: r = sqrt(mean(x^2) + eps), y_i = (x_i / r) * gamma_i.
 *   The sum of squares is taken in a fixed order: s_l = x_l^2 + x_{l+64}^2 for l < 64,
 *   then halving: for w = 32, 16, 8, 4, 2, 1: s_l = s_l + s_{l+w} (l < w).
 *   NeoX RoPE on dims 0..63 with pairs (i, i+32), i < 32, at the row's position:
 *     z_i = y_i c_i - y_{i+32} n_i,  z_{i+32} = y_{i+32} c_i + y_i n_i  (no fused ops),
 *   with c_i = cos_sin[pos][i], n_i = cos_sin[pos][32+i] (a caller-supplied fp32 table);
 *   dims 64..127 pass through.
 *   slot = page * P + row; a negative slot is a padding row and writes nothing. */
static void k_row_normed_roped(const uint16_t* xrow, const float* gamma, float eps, const float* cs_row,
                               double* z) {
  double x[HEAD_DIM], s[64], y[HEAD_DIM];
  for (int i = 0; i < HEAD_DIM; ++i) x[i] = bf16_to_double(xrow[i]);
  for (int l = 0; l < 64; ++l) s[l] = x[l] * x[l] + x[l + 64] * x[l + 64];
  for (int w = 32; w >= 1; w /= 2)
    for (int l = 0; l < w; ++l) s[l] = s[l] + s[l + w];
  double r = sqrt(s[0] / 128.0 + (double)eps);
  for (int i = 0; i < HEAD_DIM; ++i) y[i] = (x[i] / r) * (double)gamma[i];
  for (int i = 0; i < ROPE_DIM / 2; ++i) {
    double c = (double)cs_row[i], n = (double)cs_row[32 + i];
    double a = y[i], b = y[i + 32];
    double ac = a * c, bn = b * n, bc = b * c, an = a * n;
    z[i] = ac - bn;
    z[i + 32] = bc + an;
  }
  for (int i = ROPE_DIM; i < HEAD_DIM; ++i) z[i] = y[i];
}

/* FP8 arm of the K store: the same normed, rotated row, then one fp32 per-token scale
 * sk = fp32(amax / 448) and codes e4m3_rne_sat(z_i / sk) (reading: the pages give
 * FP8 K as e4m3 codes plus one fp32 scale per token, 132 B, without the scale rule;
 * amax/448 maps the row's largest magnitude onto e4m3's largest finite value).
 * amax == 0 (or a scale that underflows fp32) stores sk = 0 and sign-only zero codes. */
static void fp8_quant_row(const double* z, uint8_t* codes, float* sk_out) {
  double amax = 0.0;
  for (int i = 0; i < HEAD_DIM; ++i)
    if (fabs(z[i]) > amax) amax = fabs(z[i]);
  float sk = (float)(amax / 448.0);
  *sk_out = sk;
  for (int i = 0; i < HEAD_DIM; ++i) {
    if (sk == 0.0f) codes[i] = signbit(z[i]) ? 0x80 : 0x00;
    else codes[i] = orc_e4m3_encode(z[i] / (double)sk);
  }
}

int orc_k_store(uint8_t* pool, int64_t offset, int64_t stride, int64_t num_pages, int32_t page_size, int32_t fmt,
                const uint16_t* k_bf16, int64_t n_rows, int64_t row_stride, const float* gamma, float eps,
                const int32_t* positions, const float* cos_sin, int32_t max_pos, const int64_t* slots) {
  if (fmt != FMT_MXFP4 && fmt != FMT_FP8) return ORC_EINVAL;
  for (int64_t i = 0; i < n_rows; ++i) {
    if (slots[i] >= 0 && (slots[i] / page_size >= num_pages || positions[i] < 0 || positions[i] >= max_pos))
      return ORC_EINVAL;
  }
  /* rows are independent (each owns its slot), so they may run in any order */
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t slot = slots[i];
    if (slot < 0) continue;
    int64_t pid = slot / page_size, row = slot % page_size;
    int32_t pos = positions[i];
    double z[HEAD_DIM];
    k_row_normed_roped(k_bf16 + i * row_stride, gamma, eps, cos_sin + (int64_t)pos * 64, z);
    uint8_t* page = pool + offset + pid * stride;
    if (fmt == FMT_MXFP4) {
      for (int b = 0; b < HEAD_DIM / MX_BLOCK; ++b)
        orc_mxfp4_quant_block(z + MX_BLOCK * b, page + row * 64 + 16 * b, page + (int64_t)page_size * 64 + row * 4 + b);
    } else {
      float sk;
      fp8_quant_row(z, page + row * 128, &sk);
      memcpy(page + (int64_t)page_size * 128 + row * 4, &sk, 4);
    }
  }
  return ORC_OK;
}

/* The normed, rotated, unquantised K rows (fp64) — the reference point for the same-run
 * precision comparison of the MXFP4 and FP8 arms. */
void orc_k_rows_exact(const uint16_t* k_bf16, int64_t n_rows, int64_t row_stride, const float* gamma, float eps,
                      const int32_t* positions, const float* cos_sin, double* z_out) {
  for (int64_t i = 0; i < n_rows; ++i)
    k_row_normed_roped(k_bf16 + i * row_stride, gamma, eps, cos_sin + (int64_t)positions[i] * 64, z_out + i * HEAD_DIM);
}

/* ------------------------------------------------------------------------------ */
/* Q quantisation (input preparation for the scorer)                                */
/* ------------------------------------------------------------------------------ */
/* MXFP4 Q: each 128-dim head vector split into four 32-blocks, each quantised with the
 * block rule above; 64 B of nibbles and 4 E8M0 bytes per head [p1 Purpose: packed Q
 * production and scale layout; p2 Changes / Q quant].  No RoPE here (reading: the
 * scorer's inputs are already-rotated head vectors). */
void orc_q_quant_mxfp4(const uint16_t* q_bf16, int64_t n_vecs, uint8_t* q_out, uint8_t* scale_out) {
  for (int64_t v = 0; v < n_vecs; ++v) {
    double x[HEAD_DIM];
    for (int i = 0; i < HEAD_DIM; ++i) x[i] = bf16_to_double(q_bf16[v * HEAD_DIM + i]);
    for (int b = 0; b < 4; ++b) orc_mxfp4_quant_block(x + 32 * b, q_out + v * 64 + 16 * b, scale_out + v * 4 + b);
  }
}

/* MXFP4 Q preparation: rotation, packing and the weight fold in one op [p2 Changes / Q
 * quant: the Q op rotates and packs Q to MXFP4 and emits fp32 weights with the softmax
 * and head scales folded in; p3 Purpose: RoPE covers the leading rope dims of q as of k].
 * Reading of what the pages leave open:
 *   - vector v = t * H + h is head h of token t; it is rotated at positions[t] with the
 *     K store's NeoX rotation (pairs (i, i+32), i < 32, the same cos/sin table, no fused
 *     operations) applied to the bf16 values as they are (Q gets no normalisation);
 *     a position outside [0, max_pos) leaves the vector unrotated;
 *   - the rotated fp64 values are packed exactly as orc_q_quant_mxfp4 packs a vector;
 *   - w_out[v] = fp32(w[v] * w_scale), w_scale being the product of the factors the
 *     caller folds in (e.g. head_dim^-1/2 * H^-1/2). */
void orc_q_prep_mxfp4(const uint16_t* q_bf16, int64_t n_tokens, int32_t H, const int32_t* positions,
                      const float* cos_sin, int32_t max_pos, const float* w, float w_scale, uint8_t* q_out,
                      uint8_t* scale_out, float* w_out) {
  for (int64_t t = 0; t < n_tokens; ++t) {
    const int32_t pos = positions[t];
    const int rot = pos >= 0 && pos < max_pos;
    for (int32_t h = 0; h < H; ++h) {
      const int64_t v = t * H + h;
      double x[HEAD_DIM], z[HEAD_DIM];
      for (int i = 0; i < HEAD_DIM; ++i) x[i] = bf16_to_double(q_bf16[v * HEAD_DIM + i]);
      for (int i = 0; i < HEAD_DIM; ++i) z[i] = x[i];
      if (rot) {
        const float* cs = cos_sin + (int64_t)pos * 64;
        for (int i = 0; i < ROPE_DIM / 2; ++i) {
          double c = (double)cs[i], n = (double)cs[32 + i];
          double a = x[i], b = x[i + 32];
          double ac = a * c, bn = b * n, bc = b * c, an = a * n;
          z[i] = ac - bn;
          z[i + 32] = bc + an;
        }
      }
      for (int b = 0; b < 4; ++b) orc_mxfp4_quant_block(z + 32 * b, q_out + v * 64 + 16 * b, scale_out + v * 4 + b);
      w_out[v] = (float)((double)w[v] * (double)w_scale);
    }
  }
}

/* FP8 Q, per-token-group quantisation with group = one 128-dim head vector [p3
 * Purpose: per-token-group FP8 quantisation of q, then the q scale folded into the
 * indexer weights]: sq = fp32(amax / 448), codes e4m3_rne_sat(q_i / sq), and
 * w_out[v] = fp32(w[v] * sq).  A zero vector gives sq = 0, zero codes, w_out = 0. */
void orc_q_quant_fp8(const uint16_t* q_bf16, const float* w, int64_t n_vecs, uint8_t* q_out, float* w_out) {
  for (int64_t v = 0; v < n_vecs; ++v) {
    double x[HEAD_DIM], amax = 0.0;
    for (int i = 0; i < HEAD_DIM; ++i) {
      x[i] = bf16_to_double(q_bf16[v * HEAD_DIM + i]);
      if (fabs(x[i]) > amax) amax = fabs(x[i]);
    }
    float sq = (float)(amax / 448.0);
    for (int i = 0; i < HEAD_DIM; ++i)
      q_out[v * HEAD_DIM + i] = (sq == 0.0f) ? (signbit(x[i]) ? 0x80 : 0x00) : orc_e4m3_encode(x[i] / (double)sq);
    w_out[v] = (float)((double)w[v] * (double)sq);
  }
}

/* ------------------------------------------------------------------------------ */
/* FP8 QK preparation: the indexer's five pre-processing steps as one op             */
/* [p3 Purpose: LayerNorm on k, RoPE on the leading rope dims of q and k, per-token-  */
/* group FP8 quantisation of q, the q scale folded into the weights, FP8 k written    */
/* to the paged cache; Test Plan: NeoX and interleaved rotation layouts, page sizes,  */
/* and the rows the op skips pinned to zero]                                          */
/* ------------------------------------------------------------------------------ */
/* Rotation of dims 0..63 of y at the factors cs (32 cosines, then 32 sines); dims
 * 64..127 pass through.  NeoX pairs (i, i+32); interleaved pairs (2i, 2i+1); pair i
 * turns by (c_i, n_i) = (cs[i], cs[32+i]), no fused operations:
 *   first' = first * c - second * n,  second' = second * c + first * n. */
static void rope64(const double* y, const float* cs, int neox, double* z) {
  for (int i = 0; i < HEAD_DIM; ++i) z[i] = y[i];
  for (int i = 0; i < ROPE_DIM / 2; ++i) {
    const int a_i = neox ? i : 2 * i, b_i = neox ? i + 32 : 2 * i + 1;
    double c = (double)cs[i], n = (double)cs[32 + i];
    double a = y[a_i], b = y[b_i];
    double ac = a * c, bn = b * n, bc = b * c, an = a * n;
    z[a_i] = ac - bn;
    z[b_i] = bc + an;
  }
}

/* Reading of the steps the page leaves open (fp64 throughout, nothing narrowed before a
 * code is decided):
 *   LayerNorm over the 128 dims of k: mu = S(x) / 128, d_i = x_i - mu, var = S(d^2) / 128,
 *   r = sqrt(var + eps), y_i = (d_i / r) * gamma_i + beta_i, where S sums in the K
 *   store's fixed order (s_l = v_l + v_{l+64} for l < 64, then s_l = s_l + s_{l+w} for
 *   w = 32, 16, 8, 4, 2, 1);
 *   k: rope64, then the FP8 K store's row quantiser (one fp32 scale per token), stored
 *   at its slot in the 132 B/token page layout;
 *   q: each head vector of the token rotated as loaded (no normalisation), then
 *   quantised per 128-dim vector exactly as orc_q_quant_fp8 does, w_out = fp32(w * sq);
 *   a token whose slot is negative (padding), outside the pool, or whose position is
 *   outside [0, max_pos) is skipped: no K is stored, and its q codes and weights are
 *   zero. */
static double fold_sum(const double* v) {
  double s[64];
  for (int l = 0; l < 64; ++l) s[l] = v[l] + v[l + 64];
  for (int w = 32; w >= 1; w /= 2)
    for (int l = 0; l < w; ++l) s[l] = s[l] + s[l + w];
  return s[0];
}

int orc_qk_prep_fp8(uint8_t* pool, int64_t offset, int64_t stride, int64_t num_pages, int32_t page_size,
                    const uint16_t* q_bf16, const uint16_t* k_bf16, int64_t n_tokens, int32_t H, const float* w,
                    const int32_t* positions, const float* cos_sin, int32_t max_pos, int32_t neox,
                    const float* ln_gamma, const float* ln_beta, float eps, const int64_t* slots, uint8_t* q_out,
                    float* w_out) {
  if (page_size <= 0 || H <= 0) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n_tokens; ++t) {
    const int64_t slot = slots[t];
    const int32_t pos = positions[t];
    const int skip = slot < 0 || slot / page_size >= num_pages || pos < 0 || pos >= max_pos;
    if (skip) {
      memset(q_out + t * H * HEAD_DIM, 0, (size_t)H * HEAD_DIM);
      for (int32_t h = 0; h < H; ++h) w_out[t * H + h] = 0.0f;
      continue;
    }
    const float* cs = cos_sin + (int64_t)pos * 64;
    /* k: LayerNorm, rotation, FP8 row, page store */
    double x[HEAD_DIM], d[HEAD_DIM], sq[HEAD_DIM], y[HEAD_DIM], z[HEAD_DIM];
    for (int i = 0; i < HEAD_DIM; ++i) x[i] = bf16_to_double(k_bf16[t * HEAD_DIM + i]);
    const double mu = fold_sum(x) / 128.0;
    for (int i = 0; i < HEAD_DIM; ++i) {
      d[i] = x[i] - mu;
      sq[i] = d[i] * d[i];
    }
    const double r = sqrt(fold_sum(sq) / 128.0 + (double)eps);
    for (int i = 0; i < HEAD_DIM; ++i) {
      const double nrm = (d[i] / r) * (double)ln_gamma[i];
      y[i] = nrm + (double)ln_beta[i];
    }
    rope64(y, cs, neox, z);
    uint8_t* page = pool + offset + (slot / page_size) * stride;
    const int64_t row = slot % page_size;
    float sk;
    fp8_quant_row(z, page + row * 128, &sk);
    memcpy(page + (int64_t)page_size * 128 + row * 4, &sk, 4);
    /* q: rotation, per-vector FP8, weight fold */
    for (int32_t h = 0; h < H; ++h) {
      const int64_t v = t * H + h;
      double qx[HEAD_DIM], qz[HEAD_DIM], amax = 0.0;
      for (int i = 0; i < HEAD_DIM; ++i) qx[i] = bf16_to_double(q_bf16[v * HEAD_DIM + i]);
      rope64(qx, cs, neox, qz);
      for (int i = 0; i < HEAD_DIM; ++i)
        if (fabs(qz[i]) > amax) amax = fabs(qz[i]);
      const float s = (float)(amax / 448.0);
      for (int i = 0; i < HEAD_DIM; ++i)
        q_out[v * HEAD_DIM + i] = (s == 0.0f) ? (signbit(qz[i]) ? 0x80 : 0x00) : orc_e4m3_encode(qz[i] / (double)s);
      w_out[v] = (float)((double)w[v] * (double)s);
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------------ */
/* Scorer: paged MQA logits with the causal / length mask                           */
/* ------------------------------------------------------------------------------ */
/* Row r = b * n_q + j holds query token j of sequence b.  Its valid length is
 *   n_r = clamp(ctx[b] - n_q + 1 + j, 0, ctx[b])
 * (reading: the n_q query tokens of a sequence are its last n_q tokens and are causal
 * among themselves — decode has n_q = 1, speculative verification n_q > 1 [p2 Test
 * Plan: MTP speculative tokens], prefill n_q = ctx).  For s < n_r:
 *   logit[r,s] = sum_h w[r,h] * max(d_h, 0),  d_h = sum_i deq(q[r,h])_i * deq(k[s])_i,
 * k[s] read in place from page pt[b][s / P], row s % P [p2 Purpose: scored in place,
 * no gather].  Heads are summed in order h = 0..H-1.  Cells s >= n_r are not computed
 * (left as NaN here).  `rows` selects which rows to compute (all of them when NULL),
 * so that full-size configurations can be checked on a sample; out row i is rows[i].
 * MXFP4: deq(x)_i = e2m1(code_i) * 2^(E8M0 of i's block - 127) for both q and k.
 * FP8:   deq(k)_i = sk[s] * e4m3(code_i), deq(q)_i = e4m3(code_i) with the q scale
 *        already folded into w. */
int64_t orc_valid_len(const int32_t* ctx, int32_t n_q, int64_t r) {
  int64_t b = r / n_q, j = r % n_q;
  int64_t n = (int64_t)ctx[b] - n_q + 1 + j;
  if (n < 0) n = 0;
  if (n > ctx[b]) n = ctx[b];
  return n;
}

static void deq_k_token(const uint8_t* page, int32_t page_size, int64_t row, int fmt, double* k) {
  if (fmt == FMT_MXFP4) {
    const uint8_t* nib = page + row * 64;
    const uint8_t* sc = page + (int64_t)page_size * 64 + row * 4;
    for (int i = 0; i < HEAD_DIM; ++i) {
      unsigned byte = nib[i / 2];
      unsigned code = (i % 2 == 0) ? (byte & 15u) : (byte >> 4);
      k[i] = orc_e2m1_decode(code) * orc_e8m0_decode(sc[i / 32]);
    }
  } else {
    float sk;
    memcpy(&sk, page + (int64_t)page_size * 128 + row * 4, 4);
    for (int i = 0; i < HEAD_DIM; ++i) k[i] = (double)sk * orc_e4m3_decode(page[row * 128 + i]);
  }
}

int orc_logits_paged(const uint8_t* pool, int64_t offset, int64_t stride, int64_t num_pages, int32_t page_size,
                     int32_t fmt, const uint8_t* q, const uint8_t* q_scale, const float* w, const int32_t* page_table,
                     int32_t max_pages_per_seq, const int32_t* ctx, int32_t B, int32_t n_q, int32_t H,
                     const int64_t* rows, int64_t n_rows, double* out, int64_t out_stride) {
  if (fmt != FMT_MXFP4 && fmt != FMT_FP8) return ORC_EINVAL;
  if (rows == NULL) n_rows = (int64_t)B * n_q;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t r = rows ? rows[i] : i;
    int64_t b = r / n_q;
    int64_t n = orc_valid_len(ctx, n_q, r);
    double* o = out + i * out_stride;
    for (int64_t s = 0; s < out_stride; ++s) o[s] = NAN;
    double* qd = (double*)malloc(sizeof(double) * (size_t)H * HEAD_DIM);
    for (int h = 0; h < H; ++h) {
      int64_t v = r * H + h;
      for (int ii = 0; ii < HEAD_DIM; ++ii) {
        if (fmt == FMT_MXFP4) {
          unsigned byte = q[v * 64 + ii / 2];
          unsigned code = (ii % 2 == 0) ? (byte & 15u) : (byte >> 4);
          qd[h * HEAD_DIM + ii] = orc_e2m1_decode(code) * orc_e8m0_decode(q_scale[v * 4 + ii / 32]);
        } else {
          qd[h * HEAD_DIM + ii] = orc_e4m3_decode(q[v * HEAD_DIM + ii]);
        }
      }
    }
    for (int64_t s = 0; s < n; ++s) {
      int64_t pid = page_table[b * max_pages_per_seq + s / page_size];
      if (pid < 0 || pid >= num_pages) { bad = 1; continue; }
      double k[HEAD_DIM];
      deq_k_token(pool + offset + pid * stride, page_size, s % page_size, fmt, k);
      double logit = 0.0;
      for (int h = 0; h < H; ++h) {
        double d = 0.0;
        for (int ii = 0; ii < HEAD_DIM; ++ii) d += qd[h * HEAD_DIM + ii] * k[ii];
        logit += (double)w[r * H + h] * (d > 0.0 ? d : 0.0);
      }
      o[s] = logit;
    }
    free(qd);
  }
  return bad ? ORC_EINVAL : ORC_OK;
}

/* Unquantised logits from fp64 head vectors and fp64 K rows laid out by logical token:
 * the reference point for the MXFP4 / FP8 precision comparison (not a parity target).
 * k_rows[b][s][128], q_rows[r][h][128]. */
void orc_logits_exact(const double* q_rows, const float* w, const double* k_rows, int64_t k_seq_stride,
                      const int32_t* ctx, int32_t B, int32_t n_q, int32_t H, const int64_t* rows, int64_t n_rows,
                      double* out, int64_t out_stride) {
  (void)B;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t r = rows[i], b = r / n_q, n = orc_valid_len(ctx, n_q, r);
    double* o = out + i * out_stride;
    for (int64_t s = 0; s < out_stride; ++s) o[s] = NAN;
    for (int64_t s = 0; s < n; ++s) {
      const double* k = k_rows + b * k_seq_stride + s * HEAD_DIM;
      double logit = 0.0;
      for (int h = 0; h < H; ++h) {
        const double* qq = q_rows + (r * H + h) * HEAD_DIM;
        double d = 0.0;
        for (int ii = 0; ii < HEAD_DIM; ++ii) d += qq[ii] * k[ii];
        logit += (double)w[r * H + h] * (d > 0.0 ? d : 0.0);
      }
      o[s] = logit;
    }
  }
}

/* ------------------------------------------------------------------------------ */
/* Per-row top-k [p2 Purpose: top-k 1024; p3 Purpose: topk_indices_buffer]          */
/* ------------------------------------------------------------------------------ */
/* Reading: rank the valid tokens s < n_r by (logit descending, s ascending) and keep
 * the first min(k, n_r); the remaining output slots hold -1.  When n_r <= k the result
 * is every valid token.  Output is in rank order. */
typedef struct { double v; int64_t s; } ranked;

static int cmp_ranked(const void* a, const void* b) {
  const ranked* x = (const ranked*)a;
  const ranked* y = (const ranked*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->s < y->s) ? -1 : (x->s > y->s);
}

void orc_topk(const double* logits, int64_t stride, const int32_t* ctx, int32_t n_q, int32_t k, const int64_t* rows,
              int64_t n_rows, int32_t* out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t r = rows[i];
    int64_t n = orc_valid_len(ctx, n_q, r);
    const double* row = logits + i * stride;
    int32_t* o = out + i * (int64_t)k;
    ranked* buf = (ranked*)malloc(sizeof(ranked) * (size_t)(n > 0 ? n : 1));
    for (int64_t s = 0; s < n; ++s) { buf[s].v = row[s]; buf[s].s = s; }
    qsort(buf, (size_t)n, sizeof(ranked), cmp_ranked);
    for (int64_t t = 0; t < k; ++t) o[t] = (t < n) ? (int32_t)buf[t].s : -1;
    free(buf);
  }
}
