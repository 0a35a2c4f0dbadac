// Streaming form of the decode scorer (gfx950): each wave scores one query row over a
// strided set of 64-token chunks of its sequence, with the next chunk's K tiles in
// flight while the current one is scored (two register buffers used alternately, so no
// register copy waits on a load).  For shapes where one pass of short-lived waves leaves
// the memory system idle while they compute: several query rows with many heads (e.g. 3
// speculative tokens x 64 heads) over mixed context lengths.
//
// Blocks of 4 waves; wave w takes row w % n_q and chunk lane w / n_q of its block (n_q <= 4;
// waves past n_q * floor(4 / n_q) leave at once), so the rows of a chunk run on one CU and
// all but one read its K from the cache.  Chunk c of row j covers tokens [64c, 64c + 64);
// block x's chunk lane l takes chunks x*L + l, x*L + l + S, ... (L lanes per block, S =
// gridDim.x * L) below the row's valid length.  Loads are issued for every step, past the
// end too (page 0 row 0), so the outstanding-load count is the same on every path.
#include <algorithm>

#include "scorer.hpp"

namespace idx {
namespace {

template <int FMT, int HT, bool NT_LOADS>
__global__ __launch_bounds__(256) void logits_stream_kernel(LogitsArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int lanes_per_block = 4 / a.n_q;
  if (wave >= a.n_q * lanes_per_block) return;
  const int j = wave % a.n_q, cl = wave / a.n_q;
  const int b = blockIdx.y;
  const int stride = (int)gridDim.x * lanes_per_block;
  int c = (int)blockIdx.x * lanes_per_block + cl;
  const int64_t r = (int64_t)b * a.n_q + j;
  const int P = a.pool.page_size, lgP = a.pool.page_shift;
  const int last_page = (a.max_ctx - 1) >> lgP;
  const int32_t* __restrict__ ptb = a.page_table + (int64_t)b * a.max_pages;

  v8i qa[HT];
  uint32_t qs[HT];
  v4f qw[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    load_q_tile<FMT>(a, r, ht, lane, qa[ht], qs[ht]);
    qw[ht] = load_w_tile(a, r, ht, lane);
  }
  const int n_b = uniform(std::min(std::max(a.ctx[b], 0), a.max_ctx));
  const int n_r = valid_len(n_b, a.n_q, j);
  const int n_ch = (n_r + 63) >> 6;
  if (c >= n_ch) return;  // uniform: nothing to score

  const int32_t np32 = (int32_t)std::min<int64_t>(a.pool.num_pages, INT32_MAX);  // page ids are int32
  // Issue the four K tiles of chunk cc (any cc: past the row they read page 0 row 0).
  auto issue = [&](int cc, KTile<FMT>* K, bool* ok) {
    const bool live = cc < n_ch;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int s0 = 64 * cc + 16 * t;
      const int32_t pid = uniform(ptb[std::min(s0 >> lgP, last_page)]);
      const bool valid_page = pid >= 0 && pid < np32;
      const bool use = live && valid_page;
      const uint8_t* page = a.pool.base + (use ? (int64_t)pid : 0) * a.pool.stride;
      const uint32_t tok = (uint32_t)((use ? (s0 & (P - 1)) : 0) + (lane & 15)), g = (uint32_t)(lane >> 4);
      if (FMT == 0) {
        // 16 bytes of the token's nibbles; its four E8M0 bytes as one word (the lane's own
        // byte is shifted down when the tile is scored, so no byte load waits in the loop)
        const u32x4 x = ld<NT_LOADS>((const u32x4*)(page + (tok * 64u + 16u * g)));
        K[t].v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
        K[t].scale = ld<NT_LOADS>((const uint32_t*)(page + ((uint32_t)P * 64u + tok * 4u)));
      } else {
        K[t] = load_k_tile<FMT, NT_LOADS>(page, P, use ? (s0 & (P - 1)) : 0, lane);
      }
      ok[t] = valid_page;
    }
  };
  const float qnan = __builtin_nanf("");
  float* __restrict__ out_row = a.logits + r * a.lstride;
  // Score chunk cc from K: lane l of the result holds token 64cc + l.
  auto consume = [&](int cc, const KTile<FMT>* K, const bool* ok) {
    float p[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      KTile<FMT> kt = K[t];
      if (FMT == 0) kt.scale >>= 8 * (lane >> 4);  // the scale operand is its low byte
      float acc = 0.0f;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) acc = relu_dot_acc(mfma<FMT>(qa[ht], qs[ht], kt), qw[ht], acc, ht == 0);
      const float v = FMT == 1 ? acc * __uint_as_float(K[t].scale) : acc;
      p[t] = ok[t] ? v : qnan;
    }
    const float logit = reduce4_transpose(p[0], p[1], p[2], p[3]);
    const int s = 64 * cc + lane;
    if (s < n_r) out_row[s] = logit;
  };

  KTile<FMT> A[4], B[4];
  bool okA[4], okB[4];
  issue(c, A, okA);
  for (;;) {
    const int c2 = c + stride;
    issue(c2, B, okB);
    consume(c, A, okA);
    if (c2 >= n_ch) break;  // uniform
    const int c3 = c2 + stride;
    issue(c3, A, okA);
    consume(c2, B, okB);
    if (c3 >= n_ch) break;
    c = c3;
  }
}

template <int FMT>
hipError_t launch_stream_fmt(const LogitsArgs& a, dim3 grid, int ht, hipStream_t s) {
  switch (ht) {
#define IDX_STREAM_CASE(N) \
  case N: \
    if (a.n_q == 1) hipLaunchKernelGGL((logits_stream_kernel<FMT, N, true>), grid, dim3(256), 0, s, a); \
    else hipLaunchKernelGGL((logits_stream_kernel<FMT, N, false>), grid, dim3(256), 0, s, a); \
    break;
    IDX_STREAM_CASE(1) IDX_STREAM_CASE(2) IDX_STREAM_CASE(3) IDX_STREAM_CASE(4)
    IDX_STREAM_CASE(5) IDX_STREAM_CASE(6) IDX_STREAM_CASE(7) IDX_STREAM_CASE(8)
#undef IDX_STREAM_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_logits_stream(const LogitsArgs& a, int num_cus, hipStream_t s) {
  if (a.max_ctx == 0) return hipSuccess;
  if (a.n_q < 1 || a.n_q > 4) return hipErrorInvalidValue;
  const int ht = (a.H + kHeadTile - 1) / kHeadTile;
  const int lanes = 4 / a.n_q;
  const int chunks = (a.max_ctx + 63) / 64;
  // about eight waves per SIMD over the device, and at least four chunks per wave (measured
  // on 3 tokens x 64 heads: 13.3, 12.5 and 15.5 us for two, four and eight)
  const int64_t want_waves = (int64_t)num_cus * 32;
  const int64_t row_waves = (int64_t)a.B * a.n_q;
  int64_t bx = std::max<int64_t>(1, want_waves / std::max<int64_t>(1, row_waves * lanes));
  bx = std::min<int64_t>(bx, std::max(1, (chunks + 4 * lanes - 1) / (4 * lanes)));
  const dim3 grid((unsigned)bx, (unsigned)a.B);
  return a.pool.kv_format == 0 ? launch_stream_fmt<0>(a, grid, ht, s) : launch_stream_fmt<1>(a, grid, ht, s);
}

}  // namespace idx
