// Candidate-block scorer on gfx950: the second level of a two-level indexer, where each
// query row scores only the blocks a first level picked for it instead of its whole
// context (page "Dense MXFP4 indexer for DeepSeek-V4 on ROCm", Purpose: the candidate-
// pool path beside the dense one; the dense scorer is that path with no candidate
// blocks).  A candidate block is a page-sized run of the row's sequence, named by its
// index in the sequence's page table, so its tokens are read in place from that page.
//
//   cell (r, c*P + i) = logit of token cand[r][c]*P + i     when cand[r][c] is in
//                       [0, max_pages) and the token is below the row's valid length,
//                     = -inf                               otherwise.
//
// One wave per 64 cells of a row: the candidate ids of its four 16-cell tiles, then
// their page ids, then the K tiles (non-temporal: read once per call), the row's own Q
// and w, and the same MFMA / ReLU / head-sum epilogue as the dense decode form.
#include <algorithm>

#include "scorer.hpp"

namespace idx {
namespace {

constexpr int kCandWaves = 4;

template <int FMT, int HT>
__global__ __launch_bounds__(256) void logits_cand_kernel(LogitsArgs a, CandArgs c) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int64_t r = blockIdx.x;
  const int lgP = a.pool.page_shift, P = a.pool.page_size;
  const int n_cells = c.n_cand << lgP;
  const int c0 = (blockIdx.y * kCandWaves + wave) * 64;
  if (c0 >= n_cells) return;  // uniform: the wave holds no cell of the row
  const int b = (int)(r / a.n_q), j = (int)(r % a.n_q);

  v8i qa[HT];
  uint32_t qs[HT];
  v4f qw[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    load_q_tile<FMT>(a, r, ht, lane, qa[ht], qs[ht]);
    qw[ht] = load_w_tile(a, r, ht, lane);
  }

  // Candidate ids of the four tiles (a 16-cell tile lies in one block: P >= 16), then
  // the physical pages they name.  Tiles past the row's cells repeat its last cell.
  const int32_t* __restrict__ crow = c.cand + r * c.n_cand;
  const int32_t* __restrict__ ptb = a.page_table + (int64_t)b * a.max_pages;
  int32_t cb[4], pid[4];
  bool cok[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    cb[t] = uniform(crow[std::min(c0 + 16 * t, n_cells - 1) >> lgP]);
    cok[t] = cb[t] >= 0 && cb[t] < a.max_pages;
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) pid[t] = uniform(ptb[cok[t] ? cb[t] : 0]);
  const int64_t cap = (int64_t)a.max_pages << lgP;
  const int n_b = (int)std::min((int64_t)std::max(a.ctx[b], 0), cap);
  const int n_r = valid_len(n_b, a.n_q, j);

  KTile<FMT> kt[4];
  bool pok[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row0 = (c0 + 16 * t) & (P - 1);
    const bool live = cok[t] && (int64_t)cb[t] * P + row0 < n_r;  // some cell of the tile can be valid
    pok[t] = pid[t] >= 0 && (int64_t)pid[t] < a.pool.num_pages;
    const bool use = live && pok[t];
    const uint8_t* page = a.pool.base + (use ? (int64_t)pid[t] : 0) * a.pool.stride;
    kt[t] = load_k_tile<FMT, true>(page, P, use ? row0 : 0, lane);
  }

  float p[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float acc = 0.0f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) acc = relu_dot_acc(mfma<FMT>(qa[ht], qs[ht], kt[t]), qw[ht], acc, ht == 0);
    p[t] = FMT == 1 ? acc * __uint_as_float(kt[t].scale) : acc;
  }
  // lane l now holds cell c0 + l (tile l/16, column l%16)
  const float logit = reduce4_transpose(p[0], p[1], p[2], p[3]);
  const int g = lane >> 4, cell = c0 + lane;
  const int32_t my_cb = g == 0 ? cb[0] : (g == 1 ? cb[1] : (g == 2 ? cb[2] : cb[3]));
  const bool my_cok = g == 0 ? cok[0] : (g == 1 ? cok[1] : (g == 2 ? cok[2] : cok[3]));
  const bool my_pok = g == 0 ? pok[0] : (g == 1 ? pok[1] : (g == 2 ? pok[2] : pok[3]));
  if (cell < n_cells) {
    const bool valid = my_cok && (int64_t)my_cb * P + (cell & (P - 1)) < n_r;
    const float v = valid ? (my_pok ? logit : __builtin_nanf("")) : -__builtin_inff();
    a.logits[r * a.lstride + cell] = v;
  }
}

template <int FMT>
hipError_t launch_cand_fmt(const LogitsArgs& a, const CandArgs& c, int ht, hipStream_t s) {
  const int64_t cells = (int64_t)c.n_cand * a.pool.page_size;
  const dim3 grid((unsigned)((int64_t)a.B * a.n_q), (unsigned)((cells + 64 * kCandWaves - 1) / (64 * kCandWaves)));
  switch (ht) {
#define IDX_CAND_CASE(N) \
  case N: hipLaunchKernelGGL((logits_cand_kernel<FMT, N>), grid, dim3(256), 0, s, a, c); break;
    IDX_CAND_CASE(1) IDX_CAND_CASE(2) IDX_CAND_CASE(3) IDX_CAND_CASE(4)
    IDX_CAND_CASE(5) IDX_CAND_CASE(6) IDX_CAND_CASE(7) IDX_CAND_CASE(8)
#undef IDX_CAND_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_logits_candidates(const LogitsArgs& a, const CandArgs& c, hipStream_t s) {
  if (c.n_cand == 0) return hipSuccess;
  const int ht = (a.H + kHeadTile - 1) / kHeadTile;
  return a.pool.kv_format == 0 ? launch_cand_fmt<0>(a, c, ht, s) : launch_cand_fmt<1>(a, c, ht, s);
}

}  // namespace idx
