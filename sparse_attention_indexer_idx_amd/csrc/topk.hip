// Per-row top-k of the indexer logits on gfx950: one workgroup per row (topk_row.hpp),
// the block size chosen by the number of rows per CU.
#include "launch.hpp"
#include "topk_row.hpp"

namespace idx {
namespace {

// Rows are taken last first: the query rows of a sequence are its newest tokens, so later
// rows are at least as long (causal prefill: row j has j + 1 cells), and the longest rows
// then start first instead of forming a tail.  The 256-thread form (many rows per CU) is
// held to 96 registers, five waves per SIMD instead of four (it fits without spills).
template <int NT, int EPT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT == 256 && EPT <= 32 ? 5 : 1)))
void topk_kernel(TopkArgs a) {
  __shared__ TopkShared<NT, EPT> sh;
  const int64_t r = (int64_t)gridDim.x - 1 - blockIdx.x;
  const int b = (int)(r / a.n_q), j = (int)(r % a.n_q);
  const int n_b = min(max(a.ctx[b], 0), a.max_ctx);
  int n = n_b - a.n_q + 1 + j;
  n = n < 0 ? 0 : (n > n_b ? n_b : n);
  if constexpr (EPT > 32) topk_row_stream<NT, EPT>(a.logits + r * a.lstride, n, a.k, a.out + r * a.k, sh);
  else topk_row<NT, EPT>(a.logits + r * a.lstride, n, a.k, a.out + r * a.k, sh);
}

// Candidate rows: n_cand*P cells, -inf cells are not candidates, cells map to tokens
// through the row's candidate block ids.
template <int NT, int EPT>
__global__ __launch_bounds__(NT) void topk_cand_kernel(TopkCandArgs a) {
  __shared__ TopkShared<NT, EPT> sh;
  const int64_t r = blockIdx.x;
  CandidateRow map;
  map.cand = a.cand + r * a.n_cand;
  map.page_shift = a.page_shift;
  if constexpr (EPT > 32)
    topk_row_stream<NT, EPT, CandidateRow>(a.logits + r * a.lstride, a.n_cand << a.page_shift, a.k, a.out + r * a.k,
                                           sh, map);
  else
    topk_row<NT, EPT, CandidateRow>(a.logits + r * a.lstride, a.n_cand << a.page_shift, a.k, a.out + r * a.k, sh,
                                    map);
}

template <int NT>
hipError_t launch_cand_nt(const TopkCandArgs& a, int ept, hipStream_t s) {
  const dim3 grid((unsigned)a.rows);
  switch (ept) {
#define IDX_TOPK_CASE(E) \
  case E: hipLaunchKernelGGL((topk_cand_kernel<NT, E>), grid, dim3(NT), 0, s, a); break;
    IDX_TOPK_CASE(1) IDX_TOPK_CASE(2) IDX_TOPK_CASE(4) IDX_TOPK_CASE(8) IDX_TOPK_CASE(16) IDX_TOPK_CASE(32)
    IDX_TOPK_CASE(64)
#undef IDX_TOPK_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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

// Block size by rows per CU.  (The dense top-k keeps this rule as it is: the fused decode
// step runs the same rows with 1024 threads and must give the same index order.)
int topk_block_size(int64_t rows, int64_t cells) {
  if (rows >= 4 * 256 && cells <= 256 * 32) return 256;
  if (rows > 256 && cells <= 512 * 32) return 512;
  return 1024;
}

hipError_t launch_topk_candidates(const TopkCandArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  const int64_t cells = (int64_t)a.n_cand << a.page_shift;
  int nt = topk_block_size(a.rows, cells);
  // Candidate rows of at most 2048 cells take 512 threads even at about one row per CU:
  // fewer waves per barrier for the little work each holds (64 rows: 5.4 -> 4.9 us).
  if (nt == 1024 && cells <= 2048) nt = 512;
  int ept = 1;
  while ((int64_t)ept * nt < cells) ept *= 2;
  if (nt == 256) return launch_cand_nt<256>(a, ept, s);
  if (nt == 512) return launch_cand_nt<512>(a, ept, s);
  return launch_cand_nt<1024>(a, ept, s);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.n_q;
  if (rows == 0) return hipSuccess;
  // Rows per CU decides the block size: with many rows, 256-thread blocks let several
  // rows share a CU; with about one row per CU, 1024 threads shorten each row's chain.
  const int nt = topk_block_size(rows, a.max_ctx);
  int ept = 1;
  while ((int64_t)ept * nt < a.max_ctx) ept *= 2;
  if (nt == 256) return launch_nt<256>(a, ept, s);
  if (nt == 512) return launch_nt<512>(a, ept, s);
  return launch_nt<1024>(a, ept, s);
}

}  // namespace idx
