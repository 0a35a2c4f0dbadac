// Per-row top-k of the indexer logits on gfx950 (page "Dense MXFP4 indexer for
// DeepSeek-V4 on ROCm", Purpose: 1024 tokens kept per query; selection only matters
// once a row holds more than k valid tokens).
//
// One workgroup per row.  The row's valid cells are held in registers as order-
// preserving 32-bit keys (thread t holds cells t, t+NT, t+2NT, ...: every load is a
// contiguous 256-byte wave access).  A three-pass radix select (11, 11, 10 bits, LDS
// histogram) finds the k-th largest key K*; the output is every cell with key > K*
// plus the first (k - count_above) cells equal to K* in index order, written in
// ascending index order.  Index-order ranks come from wave ballots and per-wave
// counts, so ties are resolved deterministically toward the smaller index.
#include "device_common.hpp"
#include "launch.hpp"

namespace idx {
namespace {

__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks equal to +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }

template <int NT>
struct TopkShared {
  uint32_t hist[2048];
  int32_t wave_tot[NT / 64];
  int32_t sel_digit;
  int32_t sel_above;
};

// Inclusive prefix sum over the block (thread order), using LDS for wave totals.
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int32_t* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w)
    if (w < wave) before += wave_tot[w];
  __syncthreads();
  return v + before;
}

template <int NT, int EPT>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
  __shared__ TopkShared<NT> sh;
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r = blockIdx.x;
  const int b = (int)(r / a.n_q), j = (int)(r % a.n_q);
  const int n_b = min(max(a.ctx[b], 0), a.max_ctx);
  int n = n_b - a.n_q + 1 + j;
  n = n < 0 ? 0 : (n > n_b ? n_b : n);
  int32_t* out = a.out + r * a.k;
  if (n <= a.k) {
    for (int i = tid; i < a.k; i += NT) out[i] = (i < n) ? i : -1;
    return;
  }
  const float* row = a.logits + r * a.lstride;
  // Branch-free loads at an in-bounds index (cells past n read cell n-1 and are masked),
  // so all EPT loads are in flight together.
  float raw[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) raw[e] = row[min(e * NT + tid, n - 1)];
  uint32_t key[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) key[e] = (e * NT + tid < n) ? float_key(raw[e]) : 0u;

  // ---- radix select of the k-th largest key ----
  uint32_t prefix = 0, pmask = 0;
  int kk = a.k;  // rank still to place inside the current prefix
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int sh_ = shifts[pass];
    const uint32_t dmask = (1u << widths[pass]) - 1u;
    for (int i = tid; i < 2048; i += NT) sh.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int i = e * NT + tid;
      if (i < n && (key[e] & pmask) == prefix) atomicAdd(&sh.hist[(key[e] >> sh_) & dmask], 1u);
    }
    __syncthreads();
    // Suffix counts from the top digit down: thread t owns digits 2047 - per*t - q.
    constexpr int per = 2048 / NT;  // digits per thread (2 for NT = 1024, 8 for NT = 256)
    int cnt[per];
    int local = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) {
      cnt[q] = (int)sh.hist[2047 - per * tid - q];
      local += cnt[q];
    }
    const int incl = block_inclusive_scan<NT>(local, sh.wave_tot);
    int before = incl - local;
    if (before < kk && kk <= incl) {
#pragma unroll
      for (int q = 0; q < per; ++q) {
        if (before < kk && kk <= before + cnt[q]) {
          sh.sel_digit = 2047 - per * tid - q;
          sh.sel_above = before;
        }
        before += cnt[q];
      }
    }
    __syncthreads();
    const uint32_t d = (uint32_t)sh.sel_digit;
    kk -= sh.sel_above;
    prefix |= d << sh_;
    pmask |= dmask << sh_;
    __syncthreads();
  }
  const uint32_t kstar = prefix;
  const int need_eq = kk;  // how many cells equal to K* are taken (>= 1)

  // ---- ranks in index order: per (round e, wave) counts of >K* and ==K* cells ----
  // Cell i = e*NT + wave*64 + lane, so (e, wave) pairs in row-major order are index order.
  constexpr int NE = EPT * NW;
  __shared__ int32_t cnt_gt[NE];
  __shared__ int32_t cnt_eq[NE];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const bool v = e * NT + tid < n;
    const uint64_t bg = __ballot(v && key[e] > kstar);
    const uint64_t be = __ballot(v && key[e] == kstar);
    if (lane == 0) {
      cnt_gt[e * NW + wave] = __popcll(bg);
      cnt_eq[e * NW + wave] = __popcll(be);
    }
  }
  __syncthreads();
  if (wave == 0) {  // exclusive scan of both count arrays by one wave
    constexpr int PER = (NE + 63) / 64;
    int g[PER], q[PER], sg = 0, se = 0;
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const int f = lane * PER + t;
      g[t] = f < NE ? cnt_gt[f] : 0;
      q[t] = f < NE ? cnt_eq[f] : 0;
      sg += g[t];
      se += q[t];
    }
    int ig = sg, ie = se;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int og = __shfl_up(ig, d, 64), oe = __shfl_up(ie, d, 64);
      if (lane >= d) { ig += og; ie += oe; }
    }
    ig -= sg;
    ie -= se;
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const int f = lane * PER + t;
      if (f < NE) { cnt_gt[f] = ig; cnt_eq[f] = ie; }
      ig += g[t];
      ie += q[t];
    }
  }
  __syncthreads();
  const uint64_t lt = lanemask_lt(lane);
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = e * NT + tid;
    const bool v = i < n;
    const bool is_gt = v && key[e] > kstar;
    const bool is_eq = v && key[e] == kstar;
    const uint64_t bg = __ballot(is_gt);
    const uint64_t be = __ballot(is_eq);
    const int gt_before = cnt_gt[e * NW + wave] + __popcll(bg & lt);
    const int eq_before = cnt_eq[e * NW + wave] + __popcll(be & lt);
    const int pos = gt_before + min(eq_before, need_eq);
    if ((is_gt || (is_eq && eq_before < need_eq)) && pos < a.k) out[pos] = i;
  }
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
  if ((int64_t)a.B * a.n_q == 0) return hipSuccess;
  // Many rows: smaller blocks so several rows share a CU; few rows: one wide block each.
  const int64_t rows = (int64_t)a.B * a.n_q;
  const int nt = (rows >= 2048 && a.max_ctx <= 256 * 32) ? 256 : 1024;
  int ept = 1;
  while ((int64_t)ept * nt < a.max_ctx) ept *= 2;
  if (nt == 256) return launch_nt<256>(a, ept, s);
  return launch_nt<1024>(a, ept, s);
}

}  // namespace idx
