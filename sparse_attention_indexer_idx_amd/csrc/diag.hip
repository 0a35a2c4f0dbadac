// Diagnostic kernels, which a measurement reports next to the nominal peaks: the sustained
// rate of the scaled 16x16x128 MFMA on register operands (no memory traffic), and the rate
// of a plain streaming read (no compute) of a device buffer.
#include "device_common.hpp"
#include "launch.hpp"

namespace idx {
namespace {

// Every wave runs `rounds` rounds of 8 independent accumulating MFMAs (A and B formats
// FMT: 4 = E2M1, 0 = e4m3) and writes one float per lane so nothing is dead.
template <int FMT>
__global__ __launch_bounds__(256) void diag_mfma_kernel(float* out, int rounds) {
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (int)(0x3A3A3A3Au ^ (threadIdx.x * 0x01010101u + i));
    b[i] = (int)(0x22222222u + i * 0x01000100u);
  }
  v4f c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < rounds; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[j], FMT, FMT, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (c[j][0] + c[j][1]) + (c[j][2] + c[j][3]);
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Plain streaming read: every thread reads 16-byte words at a grid stride, eight loads in
// flight per iteration (non-temporal, as the scorer's K loads), and folds them into one
// value it stores, so no load is dead.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void diag_read_kernel(const u32x4_t* __restrict__ buf, int64_t n16, float* out) {
  constexpr int kUnroll = 8;
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(buf + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = (float)acc;
}

}  // namespace

hipError_t launch_diag_read(const void* buf, int64_t bytes, int blocks, float* out, hipStream_t s) {
  hipLaunchKernelGGL(diag_read_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const u32x4_t*>(buf),
                     bytes / 16, out);
  return hipGetLastError();
}

hipError_t launch_diag_mfma(int fmt, int blocks, int rounds, float* out, hipStream_t s) {
  if (fmt == 0)
    hipLaunchKernelGGL(diag_mfma_kernel<kMfmaFmtFp4>, dim3((unsigned)blocks), dim3(256), 0, s, out, rounds);
  else
    hipLaunchKernelGGL(diag_mfma_kernel<kMfmaFmtFp8>, dim3((unsigned)blocks), dim3(256), 0, s, out, rounds);
  return hipGetLastError();
}

}  // namespace idx
