// Per-row top-k of the indexer logits on gfx950: one workgroup per row (topk_row.hpp),
// the block size chosen by the number of rows per CU.
#include "launch.hpp"
#include "topk_row.hpp"

namespace idx {
namespace {

template <int NT, int EPT>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
  __shared__ TopkShared<NT, EPT> sh;
  const int64_t r = blockIdx.x;
  const int b = (int)(r / a.n_q), j = (int)(r % a.n_q);
  const int n_b = min(max(a.ctx[b], 0), a.max_ctx);
  int n = n_b - a.n_q + 1 + j;
  n = n < 0 ? 0 : (n > n_b ? n_b : n);
  topk_row<NT, EPT>(a.logits + r * a.lstride, n, a.k, a.out + r * a.k, sh);
}

template <int NT>
hipError_t launch_nt(const TopkArgs& a, int ept, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.B * a.n_q));
  switch (ept) {
#define IDX_TOPK_CASE(E) \
  case E: hipLaunchKernelGGL((topk_kernel<NT, E>), grid, dim3(NT), 0, s, a); break;
    IDX_TOPK_CASE(1) IDX_TOPK_CASE(2) IDX_TOPK_CASE(4) IDX_TOPK_CASE(8) IDX_TOPK_CASE(16) IDX_TOPK_CASE(32)
    IDX_TOPK_CASE(64)
#undef IDX_TOPK_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.n_q;
  if (rows == 0) return hipSuccess;
  // Rows per CU decides the block size: with many rows, 256-thread blocks let several
  // rows share a CU; with about one row per CU, 1024 threads shorten each row's chain.
  int nt = 1024;
  if (rows >= 4 * 256 && a.max_ctx <= 256 * 32) nt = 256;
  else if (rows > 256 && a.max_ctx <= 512 * 32) nt = 512;
  int ept = 1;
  while ((int64_t)ept * nt < a.max_ctx) ept *= 2;
  if (nt == 256) return launch_nt<256>(a, ept, s);
  if (nt == 512) return launch_nt<512>(a, ept, s);
  return launch_nt<1024>(a, ept, s);
}

}  // namespace idx
