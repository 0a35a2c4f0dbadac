// K-cache store and Q packing for the indexer (gfx950).
//
// K store (page "Dense MXFP4 indexer for DeepSeek-V4 on ROCm", Changes / K write:
// normalise, rotate, pack to MXFP4 and store into the pages in one pass; page
// "[ROCm][Perf] Fuse DSA indexer QK preprocessing with AITER", Purpose: the rotation
// covers the leading 64 dims and padding-slot rows are skipped).
// One wave per row: lane l holds dims l and l+64, which makes the sum of squares a
// fold of the two halves followed by a halving tree, the NeoX partner of dim l the
// lane l^32, and each 32-block of the row one half-wave.  Everything is fp64 with
// no fused multiply-adds, so the bytes equal a CPU implementation of the same steps.
#include "device_common.hpp"
#include "launch.hpp"

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

  const uint16_t* xr = a.k + row * a.row_stride;
  const double x0 = bf16_to_f64(xr[lane]);
  const double x1 = bf16_to_f64(xr[lane + 64]);

  // Sum of squares: s_l = x_l^2 + x_{l+64}^2, then s_l += s_{l+w} for w = 32..1.
  double s = x0 * x0 + x1 * x1;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    double o = __shfl_down(s, w, 64);
    s = s + o;
  }
  s = __shfl(s, 0, 64);
  const double r = sqrt(s / 128.0 + a.eps);
  const double y0 = (x0 / r) * (double)a.gamma[lane];
  const double y1 = (x1 / r) * (double)a.gamma[lane + 64];

  // NeoX rotation of dims 0..63 (pairs i, i+32); dims 64..127 pass through.
  const int i = lane & 31;
  const float* cs = a.cos_sin + (int64_t)pos * 64;
  const double c = (double)cs[i], n = (double)cs[32 + i];
  const double partner = shfl_xor(y0, 32);
  double z0;
  if (lane < 32) {
    const double ac = y0 * c, bn = partner * n;
    z0 = ac - bn;
  } else {
    const double bc = y0 * c, an = partner * n;
    z0 = bc + an;
  }
  const double z1 = y1;

  const int64_t pid = slot >> a.pool.page_shift, prow = slot & (P - 1);
  uint8_t* page = a.pool.base + pid * a.pool.stride;

  if (FMT == 0) {
    // MXFP4: blocks are dims [0,32) [32,64) (z0 in the two half-waves) and [64,96)
    // [96,128) (z1 in the two half-waves).
    double m0 = fabs(z0), m1 = fabs(z1);
#pragma unroll
    for (int w = 16; w >= 1; w >>= 1) {
      m0 = fmax(m0, shfl_xor(m0, w));
      m1 = fmax(m1, shfl_xor(m1, w));
    }
    const int X0 = mx_block_exponent(m0), X1 = mx_block_exponent(m1);
    uint32_t n0 = mxfp4_code(z0, X0) << (4 * (lane & 7));
    uint32_t n1 = mxfp4_code(z1, X1) << (4 * (lane & 7));
#pragma unroll
    for (int w = 1; w <= 4; w <<= 1) {
      n0 |= shfl_xor(n0, w);
      n1 |= shfl_xor(n1, w);
    }
    // scale bytes of blocks 0,2 live in half-wave 0 and 1,3 in half-wave 1
    const uint32_t sb_lo = (uint32_t)(X0 + 127) | ((uint32_t)(X1 + 127) << 16);
    const uint32_t sb_hi = shfl_xor(sb_lo, 32);
    uint32_t* nib_row = (uint32_t*)(page + prow * 64);
    if ((lane & 7) == 0) {
      nib_row[lane >> 3] = n0;        // bytes (lane/2)..(lane/2+3): dims lane..lane+7
      nib_row[8 + (lane >> 3)] = n1;  // dims 64+lane..64+lane+7
    }
    if (lane == 0) *(uint32_t*)(page + P * 64 + prow * 4) = sb_lo | (sb_hi << 8);
  } else {
    // FP8: one fp32 scale per token, sk = fp32(amax / 448), codes e4m3(z / sk).
    double m = fmax(fabs(z0), fabs(z1));
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) m = fmax(m, shfl_xor(m, w));
    const float sk = (float)(m / 448.0);
    uint32_t c0, c1;
    if (sk == 0.0f) {
      c0 = signbit(z0) ? 0x80u : 0u;
      c1 = signbit(z1) ? 0x80u : 0u;
    } else {
      c0 = e4m3_code(z0 / (double)sk);
      c1 = e4m3_code(z1 / (double)sk);
    }
    c0 <<= 8 * (lane & 3);
    c1 <<= 8 * (lane & 3);
#pragma unroll
    for (int w = 1; w <= 2; w <<= 1) {
      c0 |= shfl_xor(c0, w);
      c1 |= shfl_xor(c1, w);
    }
    uint32_t* code_row = (uint32_t*)(page + prow * 128);
    if ((lane & 3) == 0) {
      code_row[lane >> 2] = c0;
      code_row[16 + (lane >> 2)] = c1;
    }
    if (lane == 0) *(float*)(page + P * 128 + prow * 4) = sk;
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
