// K-cache store, Q preparation and Q packing for the indexer (gfx950).
//
// K store (page "Dense MXFP4 indexer for DeepSeek-V4 on ROCm", Changes / K write:
// normalise, rotate, pack to MXFP4 and store into the pages in one pass; page
// "[ROCm][Perf] Fuse DSA indexer QK preprocessing with AITER", Purpose: the rotation
// covers the leading 64 dims and padding-slot rows are skipped).
// One wave per row (kstore_row.hpp); the Q packing below is fp64 as well, with no fused
// multiply-adds.
#include "kstore_row.hpp"

#pragma clang fp contract(off)

namespace idx {
namespace {

constexpr int kRowsPerBlock = 4;  // 4 waves of 64 per 256-thread block

template <int FMT>
__global__ __launch_bounds__(256) void k_store_kernel(KStoreArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.n_rows) return;
  const int64_t slot = a.slots[row];
  const int32_t pos = a.positions[row];
  const int64_t P = a.pool.page_size;
  if (slot < 0 || slot >= a.pool.num_pages * P || pos < 0 || pos >= a.max_pos) return;
  if (a.step_ctx) {  // a decode step's row: its token index must be >= 0
    const int64_t bq = row / a.step_n_q, j = row % a.step_n_q;
    const int n_b = min(max(a.step_ctx[bq], 0), a.step_max_ctx);
    if (n_b - a.step_n_q + j < 0) return;
  }
  kstore_row<FMT>(a.pool, a.k + row * a.row_stride, a.gamma, a.eps, a.cos_sin + (int64_t)pos * 64, slot, lane,
                  nullptr);
}

// Q preparation for the MXFP4 scorer: rotation of the leading 64 dims at the token's
// position (the K store's rotation), MXFP4 packing, and the fold of the caller's factor
// into the weights.  Four head vectors per wave: a 16-lane group per vector, lane j of
// the group holding dims 8j..8j+7 (one 16-byte load), so the NeoX partner of dim d < 32
// (dim d + 32) sits in lane j ^ 4 of the same group and each 32-block is four lanes.
// The arithmetic is the K store's (fp64, no fused operations; the block maximum does not
// depend on its order), so the bytes equal the row routine's.  A position outside
// [0, max_pos) leaves the vector unrotated.
constexpr int kQVecsPerBlock = 16;

__global__ __launch_bounds__(256) void q_prep_mxfp4_kernel(QPrepArgs a) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63, j = lane & 15;
  const int64_t v_raw = (int64_t)blockIdx.x * kQVecsPerBlock + (threadIdx.x >> 4);
  const bool live = v_raw < a.n_vecs;
  const int64_t v = live ? v_raw : a.n_vecs - 1;  // lanes past the end compute a copy, store nothing
  const int32_t pos = a.positions[v / a.H];
  const bool rot = pos >= 0 && pos < a.max_pos && j < 8;
  const uint4 raw = *(const uint4*)(a.q + v * 128 + 8 * j);
  const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
  double y[8];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    y[2 * m] = bf16_to_f64((uint16_t)(wds[m] & 0xFFFFu));
    y[2 * m + 1] = bf16_to_f64((uint16_t)(wds[m] >> 16));
  }
  const float* __restrict__ cs = a.cos_sin + (int64_t)(rot ? pos : 0) * 64;
  double z[8];
  double amax = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double partner = shfl_xor(y[e], 4);
    const int i = 8 * (j & 3) + e;
    const double c = (double)cs[i], n = (double)cs[32 + i];
    double zr;
    if (j < 4) {
      const double ac = y[e] * c, bn = partner * n;
      zr = ac - bn;
    } else {
      const double bc = y[e] * c, an = partner * n;
      zr = bc + an;
    }
    z[e] = rot ? zr : y[e];
    amax = fmax(amax, fabs(z[e]));
  }
  amax = fmax(amax, shfl_xor(amax, 1));
  amax = fmax(amax, shfl_xor(amax, 2));
  const int X = mx_block_exponent(amax);
  uint32_t word = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) word |= mxfp4_code(z[e], X) << (4 * e);
  // scale bytes of blocks 0..3 from lanes 0, 4, 8, 12 of the group
  const uint32_t sb = (uint32_t)(X + 127);
  const int g0 = lane & 48;
  const uint32_t sw = __shfl(sb, g0, 64) | (__shfl(sb, g0 + 4, 64) << 8) | (__shfl(sb, g0 + 8, 64) << 16) |
                      (__shfl(sb, g0 + 12, 64) << 24);
  if (live) {
    reinterpret_cast<uint32_t*>(a.q_out + v * 64)[j] = word;
    if (j == 0) {
      *reinterpret_cast<uint32_t*>(a.q_scale + v * 4) = sw;
      a.w_out[v] = (float)((double)a.w[v] * (double)a.w_scale);
    }
  }
}

// MXFP4 packing of head vectors: one thread per 32-element block.
__global__ __launch_bounds__(256) void q_quant_mxfp4_kernel(const uint16_t* q, int64_t n_blocks, uint8_t* qp,
                                                            uint8_t* qs) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= n_blocks) return;
  const uint16_t* src = q + blk * 32;
  double v[32];
  double amax = 0.0;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    v[e] = bf16_to_f64(src[e]);
    amax = fmax(amax, fabs(v[e]));
  }
  const int X = mx_block_exponent(amax);
  uint32_t words[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t acc = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc |= mxfp4_code(v[8 * w + e], X) << (4 * e);
    words[w] = acc;
  }
  *(uint4*)(qp + blk * 16) = make_uint4(words[0], words[1], words[2], words[3]);
  qs[blk] = (uint8_t)(X + 127);
}

// FP8 per-vector (128 elements) quantisation with the scale folded into the weight.
__global__ __launch_bounds__(256) void q_quant_fp8_kernel(const uint16_t* q, const float* w, int64_t n_vecs,
                                                          uint8_t* q8, float* wo) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= n_vecs) return;
  const uint16_t* src = q + v * 128;
  double amax = 0.0;
  for (int e = 0; e < 128; ++e) amax = fmax(amax, fabs(bf16_to_f64(src[e])));
  const float sq = (float)(amax / 448.0);
  for (int g = 0; g < 32; ++g) {
    uint32_t acc = 0;
    for (int e = 0; e < 4; ++e) {
      const double x = bf16_to_f64(src[4 * g + e]);
      const uint32_t c = (sq == 0.0f) ? (signbit(x) ? 0x80u : 0u) : e4m3_code(x / (double)sq);
      acc |= c << (8 * e);
    }
    *(uint32_t*)(q8 + v * 128 + 4 * g) = acc;
  }
  const float wv = w[v];
  wo[v] = (float)((double)wv * (double)sq);
}

__global__ void diag_fp64_kernel(const double* a, const double* b, double* quot, double* root, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  quot[i] = a[i] / b[i];
  root[i] = sqrt(a[i]);
}

}  // namespace

hipError_t launch_k_store(const KStoreArgs& a, hipStream_t s) {
  if (a.n_rows == 0) return hipSuccess;
  const int64_t blocks = (a.n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (a.pool.kv_format == 0)
    hipLaunchKernelGGL(k_store_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_store_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_q_prep_mxfp4(const QPrepArgs& a, hipStream_t s) {
  if (a.n_vecs == 0) return hipSuccess;
  const int64_t blocks = (a.n_vecs + kQVecsPerBlock - 1) / kQVecsPerBlock;
  hipLaunchKernelGGL(q_prep_mxfp4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_q_quant_mxfp4(const uint16_t* q, int64_t n_vecs, uint8_t* qp, uint8_t* qs, hipStream_t s) {
  if (n_vecs == 0) return hipSuccess;
  const int64_t nb = n_vecs * 4;
  hipLaunchKernelGGL(q_quant_mxfp4_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, q, nb, qp, qs);
  return hipGetLastError();
}

hipError_t launch_q_quant_fp8(const uint16_t* q, const float* w, int64_t n_vecs, uint8_t* q8, float* wo,
                              hipStream_t s) {
  if (n_vecs == 0) return hipSuccess;
  hipLaunchKernelGGL(q_quant_fp8_kernel, dim3((unsigned)((n_vecs + 255) / 256)), dim3(256), 0, s, q, w, n_vecs,
                     q8, wo);
  return hipGetLastError();
}

hipError_t launch_diag_fp64(const double* a, const double* b, double* quot, double* root, int64_t n,
                            hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(diag_fp64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, b, quot, root, n);
  return hipGetLastError();
}

}  // namespace idx
