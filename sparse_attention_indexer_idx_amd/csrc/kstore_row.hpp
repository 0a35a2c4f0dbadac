// K-cache store of one row by one wave (gfx950), shared by the K-store kernel and the
// fused decode step (page "Dense MXFP4 indexer for DeepSeek-V4 on ROCm", Changes / K write:
// normalise, rotate, pack to MXFP4 and store into the pages in one pass; page "[ROCm][Perf]
// Fuse DSA indexer QK preprocessing with AITER", Purpose: the rotation covers the leading
// 64 dims).
// Lane l holds dims l and l+64, which makes the sum of squares a fold of the two halves
// followed by a halving tree, the NeoX partner of dim l the lane l^32, and each 32-block of
// the row one half-wave.  Everything is fp64 with no fused multiply-adds, so the bytes
// equal a CPU implementation of the same steps.
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace idx {

// NeoX rotation of dims 0..63 (pairs i, i+32) for the value y0 this lane holds (dim
// `lane`), with cs = cos_sin[position] (32 cosines, 32 sines); no fused operations.
__device__ __forceinline__ double rope_neox_lane(double y0, int lane, const float* __restrict__ cs) {
#pragma clang fp contract(off)
  const int i = lane & 31;
  const double c = (double)cs[i], n = (double)cs[32 + i];
  const double partner = shfl_xor(y0, 32);
  if (lane < 32) {
    const double ac = y0 * c, bn = partner * n;
    return ac - bn;
  }
  const double bc = y0 * c, an = partner * n;
  return bc + an;
}

// MXFP4 packing of a 128-dim row held as (z0 = dim lane, z1 = dim 64 + lane): blocks are
// dims [0,32) [32,64) (z0 in the two half-waves) and [64,96) [96,128) (z1).  Writes the
// 16 nibble words and the scale word (E8M0 bytes of blocks 0..3), and the same 17 words
// to `copy` when it is non-null.  All 64 lanes call it.
__device__ __forceinline__ void pack_mxfp4_row(double z0, double z1, int lane, uint32_t* __restrict__ nib_words,
                                               uint32_t* __restrict__ scale_word, uint32_t* copy) {
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
  if ((lane & 7) == 0) {
    nib_words[lane >> 3] = n0;        // bytes (lane/2)..(lane/2+3): dims lane..lane+7
    nib_words[8 + (lane >> 3)] = n1;  // dims 64+lane..64+lane+7
    if (copy) {
      copy[lane >> 3] = n0;
      copy[8 + (lane >> 3)] = n1;
    }
  }
  if (lane == 0) {
    *scale_word = sb_lo | (sb_hi << 8);
    if (copy) copy[16] = sb_lo | (sb_hi << 8);
  }
}

// FP8 row: one fp32 scale, sk = fp32(amax / 448), codes e4m3(z / sk) (sign-only zeros
// when sk == 0).  Writes the 32 code words and (when `scale` is non-null) the scale, and
// the same 33 words to `copy` when it is non-null; returns sk on every lane.
__device__ __forceinline__ float pack_fp8_row(double z0, double z1, int lane, uint32_t* __restrict__ code_words,
                                              float* __restrict__ scale, uint32_t* copy) {
#pragma clang fp contract(off)
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
  if ((lane & 3) == 0) {
    code_words[lane >> 2] = c0;
    code_words[16 + (lane >> 2)] = c1;
    if (copy) {
      copy[lane >> 2] = c0;
      copy[16 + (lane >> 2)] = c1;
    }
  }
  if (lane == 0) {
    if (scale) *scale = sk;
    if (copy) copy[32] = __float_as_uint(sk);
  }
  return sk;
}

// Store row xr (128 bf16) at pool slot `slot` (already checked to lie in the pool), with
// RoPE factors cs = cos_sin[position] (32 cosines, 32 sines).  With `copy` non-null the
// row's bytes are also written there in the page layout: MXFP4 — 16 nibble words then the
// scale word; FP8 — 32 code words then the fp32 scale.  All 64 lanes of the wave call it.
template <int FMT>
__device__ __forceinline__ void kstore_row(const PoolView& pool, const uint16_t* __restrict__ xr,
                                           const float* __restrict__ gamma, double eps, const float* __restrict__ cs,
                                           int64_t slot, int lane, uint32_t* copy) {
#pragma clang fp contract(off)
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
  const double r = sqrt(s / 128.0 + eps);
  const double y0 = (x0 / r) * (double)gamma[lane];
  const double y1 = (x1 / r) * (double)gamma[lane + 64];

  // NeoX rotation of dims 0..63; dims 64..127 pass through.
  const double z0 = rope_neox_lane(y0, lane, cs);
  const double z1 = y1;

  const int64_t P = pool.page_size;
  const int64_t pid = slot >> pool.page_shift, prow = slot & (P - 1);
  uint8_t* page = pool.base + pid * pool.stride;
  if (FMT == 0)
    pack_mxfp4_row(z0, z1, lane, (uint32_t*)(page + prow * 64), (uint32_t*)(page + P * 64 + prow * 4), copy);
  else
    pack_fp8_row(z0, z1, lane, (uint32_t*)(page + prow * 128), (float*)(page + P * 128 + prow * 4), copy);
}

}  // namespace idx
