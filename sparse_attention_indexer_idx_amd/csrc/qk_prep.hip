// FP8 QK preparation of the indexer in one launch on gfx950 (page "[ROCm][Perf] Fuse DSA
// indexer QK preprocessing with AITER", Purpose: LayerNorm on k, RoPE on the leading rope
// dims of q and k, per-token-group FP8 quantisation of q, the q scale folded into the
// weights, FP8 k written to the paged cache; Test Plan: NeoX and interleaved layouts, and
// the rows the op skips left at zero).
//
// One wave per 128-dim vector: the H query heads of every token, then the K row of every
// token.  Lane l holds dims l and l+64 (as in the K store): sums are the two-half fold
// followed by a halving tree, the NeoX partner of dim l is lane l^32 and the interleaved
// partner lane l^1.  fp64 throughout with no fused multiply-adds, so the bytes equal a
// CPU implementation of the same steps.
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

__global__ __launch_bounds__(256) void qk_prep_fp8_kernel(QKPrepArgs a) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int64_t v = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nq = a.n_tokens * a.H;
  if (v >= nq + a.n_tokens) return;
  const bool is_q = v < nq;
  const int64_t t = is_q ? v / a.H : v - nq;
  const int64_t slot = a.slots[t];
  const int32_t pos = a.positions[t];
  const bool skip = slot < 0 || slot >= a.pool.num_pages * (int64_t)a.pool.page_size || pos < 0 || pos >= a.max_pos;
  const float* cs = a.cos_sin + (int64_t)(skip ? 0 : pos) * 64;
  if (is_q) {
    uint32_t* q_words = reinterpret_cast<uint32_t*>(a.q_out + v * 128);
    if (skip) {  // a skipped token's query is zero codes and a zero weight
      if (lane < 32) q_words[lane] = 0u;
      if (lane == 0) a.w_out[v] = 0.0f;
      return;
    }
    const double x0 = bf16_to_f64(a.q[v * 128 + lane]);
    const double x1 = bf16_to_f64(a.q[v * 128 + 64 + lane]);
    const double z0 = rope_lane(x0, lane, cs, a.neox != 0);
    const float sq = pack_fp8_row(z0, x1, lane, q_words, nullptr, nullptr);
    if (lane == 0) a.w_out[v] = (float)((double)a.w[v] * (double)sq);
    return;
  }
  if (skip) return;  // no K for a skipped token
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
  const int64_t vecs = a.n_tokens * (a.H + 1);
  if (vecs == 0) return hipSuccess;
  hipLaunchKernelGGL(qk_prep_fp8_kernel, dim3((unsigned)((vecs + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace idx
