// Device-side helpers shared by the gfx950 kernels of the indexer hot path:
// bf16 widening, the MXFP4 / e4m3 encoders (fp64, bit-exact by construction), the
// scaled-MFMA operand types and wave-level lane exchanges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// MFMA operand format codes of v_mfma_scale_f32_16x16x128_f8f6f4 (cbsz / blgp).
constexpr int kMfmaFmtFp8 = 0;  // OCP e4m3
constexpr int kMfmaFmtFp4 = 4;  // E2M1
constexpr uint32_t kE8m0One = 0x7F7F7F7Fu;  // every scale byte = 2^0

// XCDs of an MI355X.  The device hands the linear block ids of a launch to its XCDs in turn
// (block n to XCD n % kXcds), and each XCD has its own L2, so kernels whose blocks share
// inputs lay their work out per XCD.  A power of two.
constexpr int kXcds = 8;

// Fourth word of a raw buffer descriptor on the gfx9 family (gfx950 included): 32-bit
// data format, no swizzle; with a zero stride, a load whose offset is at or past the
// descriptor's byte count returns 0 instead of touching memory, and such a store is dropped.
constexpr int kBufferRsrcFlags = 0x00020000;

__device__ __forceinline__ double bf16_to_f64(uint16_t h) {
  return (double)__uint_as_float((uint32_t)h << 16);
}

// E2M1 code of a magnitude a = |z| / 2^X (an exact fp64 value): round to nearest
// with exact midpoints going to the even code, held at 6 (code 7) above the grid.
// The grid is {0, .5, 1, 1.5, 2, 3, 4, 6}; its midpoints are .25 .75 1.25 1.75 2.5
// 3.5 5, and the even neighbour of each is code 0 2 2 4 4 6 6 — so a midpoint counts
// toward the upper code exactly when that upper code is even (">=" below).
__device__ __forceinline__ unsigned e2m1_code(double a) {
  return (unsigned)(a > 0.25) + (unsigned)(a >= 0.75) + (unsigned)(a > 1.25) + (unsigned)(a >= 1.75) +
         (unsigned)(a > 2.5) + (unsigned)(a >= 3.5) + (unsigned)(a > 5.0);
}

// MXFP4 block exponent for a block maximum: clamp(floor(log2 amax) - 2, -127, 127);
// -127 for amax == 0.  frexp gives amax = f * 2^e with f in [0.5, 1).
__device__ __forceinline__ int mx_block_exponent(double amax) {
  if (amax == 0.0) return -127;
  int e;
  (void)frexp(amax, &e);
  int X = e - 3;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// Signed E2M1 code of z under block exponent X (z / 2^X is exact: a power-of-two scale).
__device__ __forceinline__ unsigned mxfp4_code(double z, int X) {
  unsigned c = e2m1_code(fabs(ldexp(z, -X)));
  return c | (signbit(z) ? 8u : 0u);
}

// OCP e4m3 code of u: nearest finite value, ties to the even code, held at 448.
// Below 2^-6 the grid is the subnormal step 2^-9; above it each binade [2^E, 2^(E+1))
// has 8 steps of 2^(E-3).  rint() rounds half to even, and since the code is
// 8*(E+7) + q - 8 its parity is q's, so an even q is an even code; q == 16 carries
// into the next binade's first code.
__device__ __forceinline__ unsigned e4m3_code(double u) {
  double a = fabs(u);
  unsigned code;
  if (!(a < 448.0)) {
    code = 0x7Eu;
  } else if (a < 0.015625) {
    code = (unsigned)rint(a * 512.0);
  } else {
    int e;
    (void)frexp(a, &e);
    int E = e - 1;
    unsigned q = (unsigned)rint(ldexp(a, 3 - E));
    code = (unsigned)(8 * (E + 7)) + q - 8u;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code | (signbit(u) ? 0x80u : 0u);
}

// Lane exchange within a wave of 64.
template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// v_permlane32_swap / v_permlane16_swap (gfx950).  For X, Y split into 16-lane rows
// r0..r3:  swap32 -> X' = [X.r0 X.r1 Y.r0 Y.r1], Y' = [X.r2 X.r3 Y.r2 Y.r3];
//          swap16 -> X' = [X.r0 Y.r0 X.r2 Y.r2], Y' = [X.r1 Y.r1 X.r3 Y.r3].
__device__ __forceinline__ void swap32(float& x, float& y) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& x, float& y) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}

// Inclusive prefix sum of an int over the 64 lanes of a wave, in lane order: DPP row
// shifts by 1, 2, 4, 8 scan each row of 16 lanes, then row_bcast:15 / row_bcast:31 carry
// the row totals into the following rows.  All VALU, no LDS round trip.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Four partial sums p_t (t = 0..3) per lane, where lane (g = lane/16, c = lane%16)
// holds the part of column c contributed by head group g.  Returns, in lane (g, c),
// the full sum over the four head groups of p_g at column c: the head reduction and
// a 4x16 transpose in three swaps and three adds.
__device__ __forceinline__ float reduce4_transpose(float p0, float p1, float p2, float p3) {
  swap32(p0, p2);
  swap32(p1, p3);
  float u02 = p0 + p2;  // [p0.r0+p0.r2, p0.r1+p0.r3, p2.r0+p2.r2, p2.r1+p2.r3]
  float u13 = p1 + p3;
  swap16(u02, u13);
  return u02 + u13;     // row g holds p_g summed over all four rows
}

}  // namespace idx
