// FP8 QK preparation of the indexer in one launch on gfx950 (page "[ROCm][Perf] Fuse DSA
// indexer QK preprocessing with AITER", Purpose: LayerNorm on k, RoPE on the leading rope
// dims of q and k, per-token-group FP8 quantisation of q, the q scale folded into the
// weights, FP8 k written to the paged cache; Test Plan: NeoX and interleaved layouts, and
// the rows the op skips left at zero).
//
// Query heads go four to a wave (a 16-lane group per head vector, lane j of the group
// holding dims 8j..8j+7: the NeoX partner of dim d < 32 is in lane j ^ 4, an interleaved
// pair lies within one lane); then one wave per K row, lane l holding dims l and l+64 (as
// in the K store), so LayerNorm's sums are the two-half fold followed by a halving tree.
// fp64 throughout with no fused multiply-adds (a maximum does not depend on its order), so
// the bytes equal a CPU implementation of the same steps.
#include "kstore_row.hpp"

namespace idx {
namespace {

// Rotation of dims 0..63 for the value y0 this lane holds (dim `lane`); pair i turns by
// (cs[i], cs[32+i]): first' = first c - second n, second' = second c + first n.
__device__ __forceinline__ double rope_lane(double y0, int lane, const float* __restrict__ cs, bool neox) {
#pragma clang fp contract(off)
  if (neox) return rope_neox_lane(y0, lane, cs);
  const int i = lane >> 1;
  const double c = (double)cs[i], n = (double)cs[32 + i];
  const double partner = shfl_xor(y0, 1);
  if ((lane & 1) == 0) {
    const double ac = y0 * c, bn = partner * n;
    return ac - bn;
  }
  const double bc = y0 * c, an = partner * n;
  return bc + an;
}

// The fold-then-halve sum of v0 + v1 over the wave (lane 0's order), on every lane.
__device__ __forceinline__ double wave_fold_sum(double v0, double v1) {
#pragma clang fp contract(off)
  double s = v0 + v1;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const double o = __shfl_down(s, w, 64);
    s = s + o;
  }
  return __shfl(s, 0, 64);
}

// Four query head vectors of one wave: rotation, per-vector FP8 codes and the weight fold.
__device__ __forceinline__ void qk_prep_q4(const QKPrepArgs& a, int64_t wq, int lane) {
#pragma clang fp contract(off)
  const int j = lane & 15;
  const int64_t nq = a.n_tokens * a.H;
  const int64_t v_raw = wq * 4 + (lane >> 4);
  const bool live = v_raw < nq;
  const int64_t v = live ? v_raw : nq - 1;  // lanes past the end compute a copy, store nothing
  const int64_t t = v / a.H;
  const int64_t slot = a.slots[t];
  const int32_t pos = a.positions[t];
  const bool skip = slot < 0 || slot >= a.pool.num_pages * (int64_t)a.pool.page_size || pos < 0 || pos >= a.max_pos;
  const float* __restrict__ cs = a.cos_sin + (int64_t)(skip ? 0 : pos) * 64;
  const uint4 raw = *(const uint4*)(a.q + v * 128 + 8 * j);
  const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
  double y[8];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    y[2 * m] = bf16_to_f64((uint16_t)(wds[m] & 0xFFFFu));
    y[2 * m + 1] = bf16_to_f64((uint16_t)(wds[m] >> 16));
  }
  double z[8];
  double m = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // pair index i; whether this dim is the pair's first member; the other member
    const bool is_first = a.neox ? j < 4 : (e & 1) == 0;
    const int i = a.neox ? 8 * (j & 3) + e : 4 * j + (e >> 1);
    const double partner = a.neox ? shfl_xor(y[e], 4) : y[e ^ 1];
    const double c = (double)cs[i & 31], n = (double)cs[32 + (i & 31)];
    double zr;
    if (is_first) {
      const double ac = y[e] * c, bn = partner * n;
      zr = ac - bn;
    } else {
      const double bc = y[e] * c, an = partner * n;
      zr = bc + an;
    }
    z[e] = j < 8 ? zr : y[e];
    m = fmax(m, fabs(z[e]));
  }
#pragma unroll
  for (int w = 1; w <= 8; w <<= 1) m = fmax(m, shfl_xor(m, w));
  const float sq = (float)(m / 448.0);
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t code = sq == 0.0f ? (signbit(z[e]) ? 0x80u : 0u) : e4m3_code(z[e] / (double)sq);
    if (e < 4) w0 |= code << (8 * e);
    else w1 |= code << (8 * (e - 4));
  }
  if (!live) return;
  uint32_t* q_words = reinterpret_cast<uint32_t*>(a.q_out + v * 128) + 2 * j;
  q_words[0] = skip ? 0u : w0;  // a skipped token's query is zero codes and a zero weight
  q_words[1] = skip ? 0u : w1;
  if (j == 0) a.w_out[v] = skip ? 0.0f : (float)((double)a.w[v] * (double)sq);
}

__global__ __launch_bounds__(256) void qk_prep_fp8_kernel(QKPrepArgs a, int64_t q_waves) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wv < q_waves) {
    qk_prep_q4(a, wv, lane);
    return;
  }
  const int64_t t = wv - q_waves;
  if (t >= a.n_tokens) return;
  const int64_t slot = a.slots[t];
  const int32_t pos = a.positions[t];
  const bool skip = slot < 0 || slot >= a.pool.num_pages * (int64_t)a.pool.page_size || pos < 0 || pos >= a.max_pos;
  if (skip) return;  // no K for a skipped token
  const float* cs = a.cos_sin + (int64_t)pos * 64;
  const double x0 = bf16_to_f64(a.k[t * 128 + lane]);
  const double x1 = bf16_to_f64(a.k[t * 128 + 64 + lane]);
  const double mu = wave_fold_sum(x0, x1) / 128.0;
  const double d0 = x0 - mu, d1 = x1 - mu;
  const double r = sqrt(wave_fold_sum(d0 * d0, d1 * d1) / 128.0 + a.eps);
  const double n0 = (d0 / r) * (double)a.ln_gamma[lane];
  const double n1 = (d1 / r) * (double)a.ln_gamma[lane + 64];
  const double y0 = n0 + (double)a.ln_beta[lane];
  const double y1 = n1 + (double)a.ln_beta[lane + 64];
  const double z0 = rope_lane(y0, lane, cs, a.neox != 0);
  const int64_t P = a.pool.page_size;
  const int64_t pid = slot >> a.pool.page_shift, prow = slot & (P - 1);
  uint8_t* page = a.pool.base + pid * a.pool.stride;
  (void)pack_fp8_row(z0, y1, lane, (uint32_t*)(page + prow * 128), (float*)(page + P * 128 + prow * 4), nullptr);
}

}  // namespace

hipError_t launch_qk_prep_fp8(const QKPrepArgs& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  const int64_t q_waves = (a.n_tokens * a.H + 3) / 4;
  const int64_t waves = q_waves + a.n_tokens;
  hipLaunchKernelGGL(qk_prep_fp8_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a, q_waves);
  return hipGetLastError();
}

}  // namespace idx
