// Paged MQA logits of the lightning indexer on gfx950 (block-scaled MFMA).
//
//   logits[r, s] = sum_h w[r,h] * max(0, deq(q[r,h]) . deq(k[s]))       for s < n_r
//
// with K read where it lies in its physical page, so no gather pass precedes the
// scorer (page "Dense MXFP4 indexer for DeepSeek-V4 on ROCm", Purpose; the isolated
// decode and prefill scorer of page "[ROCm][Perf] Add AITER paged MXFP4 sparse indexing
// on gfx950", Performance and accuracy).
//
// The contraction runs on v_mfma_scale_f32_16x16x128_f8f6f4: A = 16 head rows of one
// query (lane l: head l%16, 32-element block l/16, with its E8M0 scale byte), B = 16
// cached tokens (lane l: token l%16, block l/16 — 16 bytes at token*64 + 16*(l/16), so
// one wave-wide load covers 16 consecutive tokens = 1 KB contiguous).  Output lane l
// holds heads 4*(l/16)..+3 of token l%16; the epilogue applies ReLU and the weights
// per lane and finishes the head sum with a 4x16 transpose-reduce (three lane swaps).
// FP8 uses the same instruction with e4m3 operands, unit block scales, and the fp32
// per-token K scale applied to the weighted partial sums.
//
// Page ids are looked up once per wave (decode) or once per 64 pages (prefill, one id
// per lane, read back with readlane), always before the K loads they address, so the
// only dependent memory round trip is page id -> K bytes.
#include <algorithm>

#include "scorer.hpp"

namespace idx {
namespace {

// ------------------------------------------------------------------------------------
// Decode kernel: 4 waves per block; grid = (ceil(max_ctx / (256*G)), B).
// ------------------------------------------------------------------------------------
constexpr int kDecodeWaves = 4;

template <int FMT, int NT, int G>
__global__ __launch_bounds__(256) void logits_decode_kernel(LogitsArgs a) {
  const int wave = uniform(threadIdx.x >> 6);
  const int tok0 = (blockIdx.x * kDecodeWaves + wave) * (64 * G);
  NoPatch none;
  decode_wave<FMT, NT, G>(a, blockIdx.y, tok0, threadIdx.x & 63, none);
}

// Calls this large run many rounds of one-pass waves; the streaming form keeps the memory
// system busy across them instead (and its waves stop at their sequence's end).
constexpr int64_t kStreamTokens = int64_t(1) << 21;

// Row-split decode kernel for several query rows with many heads (e.g. 3 speculative
// tokens x 64 heads): each wave holds one query row's head tiles instead of all rows', so
// registers stay low enough for several waves per SIMD.  The waves of a block take rows
// 4i..4i+3 of one token range, so K is fetched from memory once per CU and the other
// rows read it from the cache (rows past n_q leave at once).  Waves past their sequence
// leave early too (these shapes come with mixed lengths).
// Grid = (ceil(max_ctx / (64*G)) * ceil(n_q / 4), B).
template <int FMT, int HT, int G>
__global__ __launch_bounds__(256) void logits_decode_rows_kernel(LogitsArgs a) {
  const int wave = uniform(threadIdx.x >> 6);
  const int rb = (a.n_q + 3) >> 2;
  const int chunk = blockIdx.x / rb, j = (blockIdx.x - chunk * rb) * 4 + wave;
  if (j >= a.n_q) return;
  const int tok0 = chunk * (64 * G);
  NoPatch none;
  decode_wave<FMT, HT, G, NoPatch, true, false>(a, blockIdx.y, tok0, threadIdx.x & 63, none, j);
}

// ------------------------------------------------------------------------------------
// Prefill / long query sets: each wave owns 4 query rows (one per lane group after the
// transpose-reduce) and walks 16-token K tiles; a block is 4 waves = 16 rows.  Work
// units are (16-row block, token chunk) pairs enumerated chunk-major from a host-built
// table so that no unit is empty and all units have similar cost.  The waves keep the
// physical ids of the unit's (at most 64) logical pages one per lane.
// ------------------------------------------------------------------------------------
constexpr int kPrefillRowsPerWave = 4;
constexpr int kPrefillRowsPerBlock = 16;
constexpr int kMaxChunks = 256;

struct PrefillPlan {
  int32_t chunk;                      // tokens per chunk (multiple of 16)
  int32_t n_chunks;
  int32_t n_qb;                       // 16-row blocks per sequence
  int32_t unit_start[kMaxChunks + 1]; // first unit of each chunk (prefix counts)
  int32_t qb_min[kMaxChunks];         // first row block that reaches each chunk
};


// Prefill form with the K tiles shared through LDS: the four waves of a block score the
// same tokens for different rows, so each group of eight 16-token tiles is fetched once
// per block (wave w fetches tiles 2w and 2w + 1 into registers, then LDS; lane l of every
// wave reads back the operand lane l fetched, which is its own MFMA operand for that
// tile).  Two LDS buffers alternate, with one barrier per group; the next group's fetch is
// in flight while the current one is scored.  Block-uniform token range (the block's last
// row), so every wave runs the same number of groups.  The occupancy targets hold the
// MXFP4 forms with one and two head tiles at their register budgets (six and four waves
// per SIMD).
constexpr int kStageTiles = 8;  // tiles per group: kStageTiles / 4 per wave

template <int FMT>
struct alignas(16) PrefillStage {
  uint4 data[2][kStageTiles][64][FMT == 0 ? 1 : 2];
  uint32_t scale[2][kStageTiles][64];
  float out[4][kPrefillRowsPerWave][64];  // per wave: four tiles' logits, re-read per row
};

template <int FMT, int HT>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(FMT != 0 ? 1 : HT == 1 ? 6 : HT == 2 ? 4 : 1)))
void logits_prefill_kernel(LogitsArgs a, PrefillPlan plan) {
  __shared__ PrefillStage<FMT> st;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int b = blockIdx.y;
  const int u = blockIdx.x;
  int lo = 0, hi = plan.n_chunks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (plan.unit_start[mid] <= u) lo = mid; else hi = mid - 1;
  }
  const int c = lo;
  const int qb = plan.n_qb - 1 - (u - plan.unit_start[c]);
  const int jb = qb * kPrefillRowsPerBlock;  // first row of the block
  const int j0 = jb + wave * kPrefillRowsPerWave;
  const int n_b = uniform(std::min(std::max(a.ctx[b], 0), a.max_ctx));
  const int jb_last = std::min(jb + kPrefillRowsPerBlock, a.n_q) - 1;
  const int t_end = std::min(valid_len(n_b, a.n_q, jb_last), (c + 1) * plan.chunk);  // block-uniform
  const int t_begin = c * plan.chunk;
  if (t_begin >= t_end) return;  // the whole block
  const int P = a.pool.page_size, lgP = a.pool.page_shift;
  const int32_t* __restrict__ ptb = a.page_table + (int64_t)b * a.max_pages;
  const int last_page = (t_end - 1) >> lgP;
  const int page0 = t_begin >> lgP;
  const int32_t win = ptb[std::min(page0 + lane, last_page)];
  // page ids are int32, so the bound fits one (a 32-bit compare stays on the scalar unit)
  const int32_t np32 = (int32_t)std::min<int64_t>(a.pool.num_pages, INT32_MAX);
  auto tile_ok = [&](int s0) {  // uniform
    const int32_t pid = __builtin_amdgcn_readlane(win, (std::min(s0, t_end - 1) >> lgP) - page0);
    return s0 < t_end && pid >= 0 && pid < np32;
  };

  v8i qa[kPrefillRowsPerWave][HT];
  uint32_t qs[kPrefillRowsPerWave][HT];
  v4f qw[kPrefillRowsPerWave][HT];
#pragma unroll
  for (int g = 0; g < kPrefillRowsPerWave; ++g) {
    const int j = std::min(j0 + g, a.n_q - 1);
    const int64_t r = (int64_t)b * a.n_q + j;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      load_q_tile<FMT>(a, r, ht, lane, qa[g][ht], qs[g][ht]);
      qw[g][ht] = load_w_tile(a, r, ht, lane);
    }
  }
  // One store descriptor per row of the wave, its range the row's valid cells inside this
  // unit's chunk: a store past it is dropped by the hardware, so no store is conditional.
  __amdgpu_buffer_rsrc_t orow_rsrc[kPrefillRowsPerWave];
#pragma unroll
  for (int g = 0; g < kPrefillRowsPerWave; ++g) {
    const int jr = j0 + g;  // uniform
    const int n_g = jr < a.n_q ? std::min(valid_len(n_b, a.n_q, jr), t_end) : 0;
    float* row = a.logits + ((int64_t)b * a.n_q + std::min(jr, a.n_q - 1)) * a.lstride;
    orow_rsrc[g] = __builtin_amdgcn_make_buffer_rsrc(row, 0, n_g * 4, kBufferRsrcFlags);
  }
  const float qnan = __builtin_nanf("");

  constexpr int TPW = kStageTiles / 4;  // tiles each wave fetches per group
  // tile w*TPW + i of group gg (tokens t_begin + 16*kStageTiles*gg + 16*(w*TPW + i))
  auto fetch = [&](int gg, int i) {
    const int s0 = t_begin + 16 * kStageTiles * gg + 16 * (wave * TPW + i);
    const bool okk = tile_ok(s0);
    const int32_t pid = __builtin_amdgcn_readlane(win, (std::min(s0, t_end - 1) >> lgP) - page0);
    const uint8_t* page = a.pool.base + (okk ? (int64_t)pid : 0) * a.pool.stride;
    return load_k_tile_w<FMT, false>(page, P, okk ? (s0 & (P - 1)) : 0, lane);
  };
  auto stash = [&](int buf, int i, const KTile<FMT>& k) {
    const int t = wave * TPW + i;
    st.data[buf][t][lane][0] = make_uint4((uint32_t)k.v[0], (uint32_t)k.v[1], (uint32_t)k.v[2], (uint32_t)k.v[3]);
    if (FMT == 1)
      st.data[buf][t][lane][FMT] = make_uint4((uint32_t)k.v[4], (uint32_t)k.v[5], (uint32_t)k.v[6], (uint32_t)k.v[7]);
    st.scale[buf][t][lane] = lane_scale<FMT>(k.scale, lane);
  };
  auto unstash = [&](int buf, int t) {
    KTile<FMT> k;
    const uint4 x = st.data[buf][t][lane][0];
    if (FMT == 0) {
      k.v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
    } else {
      const uint4 y = st.data[buf][t][lane][FMT];
      k.v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
    }
    k.scale = st.scale[buf][t][lane];
    return k;
  };

  const int n_groups = (t_end - t_begin + 16 * kStageTiles - 1) / (16 * kStageTiles);
  // Group gg + 1's tiles are staged at the end of group gg (into the other buffer, whose last
  // readers passed this group's barrier), so the only loads younger than the ones waited for
  // there are that group's stores; staged at the loop head, the path from the first fetch
  // made the compiler wait for every memory operation in flight on each iteration.
  KTile<FMT> nxt[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) nxt[i] = fetch(0, i);
#pragma unroll
  for (int i = 0; i < TPW; ++i) stash(0, i, nxt[i]);
  for (int gg = 0; gg < n_groups; ++gg) {
    const int buf = gg & 1;
#pragma unroll
    for (int i = 0; i < TPW; ++i) nxt[i] = fetch(gg + 1, i);  // past the end: page 0 row 0, never stashed
    __syncthreads();
    // Tiles go in fours: after the transpose lane l holds row l/16, token l%16 of a tile, and
    // the four tiles' logits pass through the wave's LDS rows, so each store writes 64
    // consecutive logits of one row (whole 128-byte lines) instead of a half line of four.
    // The stores are unconditional buffer stores (cells past a row's valid length fall
    // outside its descriptor): with stores under a branch, the compiler waited at the next
    // group's head for every memory operation in flight, these stores included.
#pragma unroll
    for (int t = 0; t < kStageTiles; t += 4) {
      const int s0 = t_begin + 16 * kStageTiles * gg + 16 * t;
      if (s0 < t_end) {  // uniform; tiles of the four past t_end score stale data, never stored
        float* orow = st.out[wave][lane >> 4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const KTile<FMT> kt = unstash(buf, t + h);
          float p[kPrefillRowsPerWave];
#pragma unroll
          for (int g = 0; g < kPrefillRowsPerWave; ++g) {
            float acc = 0.0f;
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
              acc = relu_dot_acc(mfma<FMT>(qa[g][ht], qs[g][ht], kt), qw[g][ht], acc, ht == 0);
            p[g] = acc;
          }
          float logit = reduce4_transpose(p[0], p[1], p[2], p[3]);
          if (FMT == 1) logit *= __uint_as_float(kt.scale);
          if (!tile_ok(s0 + 16 * h)) logit = qnan;
          orow[16 * h + (lane & 15)] = logit;
        }
      }
      __builtin_amdgcn_wave_barrier();  // the reads below take other lanes' writes
#pragma unroll
      for (int g = 0; g < kPrefillRowsPerWave; ++g)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(st.out[wave][g][lane]), orow_rsrc[g],
                                              (uint32_t)(s0 + lane) * 4u, 0, 0);
      __builtin_amdgcn_wave_barrier();  // and the next writes come after them
    }
    if (gg + 1 < n_groups) {  // uniform
#pragma unroll
      for (int i = 0; i < TPW; ++i) stash(buf ^ 1, i, nxt[i]);
    }
  }
}

template <int FMT, int G>
hipError_t launch_decode_g(const LogitsArgs& a, int nt, hipStream_t s) {
  const int tok_per_block = kDecodeWaves * 64 * G;
  const dim3 grid((unsigned)((a.max_ctx + tok_per_block - 1) / tok_per_block), (unsigned)a.B);
  switch (nt) {
#define IDX_DECODE_CASE(N) \
  case N: hipLaunchKernelGGL((logits_decode_kernel<FMT, N, G>), grid, dim3(256), 0, s, a); break;
    IDX_DECODE_CASE(1) IDX_DECODE_CASE(2) IDX_DECODE_CASE(3) IDX_DECODE_CASE(4)
    IDX_DECODE_CASE(5) IDX_DECODE_CASE(6) IDX_DECODE_CASE(7) IDX_DECODE_CASE(8)
    IDX_DECODE_CASE(9) IDX_DECODE_CASE(10) IDX_DECODE_CASE(11) IDX_DECODE_CASE(12)
    IDX_DECODE_CASE(13) IDX_DECODE_CASE(14) IDX_DECODE_CASE(15) IDX_DECODE_CASE(16)
#undef IDX_DECODE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT, int G>
hipError_t launch_decode_rows_g(const LogitsArgs& a, int ht, hipStream_t s) {
  const int tok_per_block = 64 * G;
  const dim3 grid((unsigned)((a.max_ctx + tok_per_block - 1) / tok_per_block * ((a.n_q + 3) / 4)), (unsigned)a.B);
  switch (ht) {
#define IDX_ROWS_CASE(N) \
  case N: hipLaunchKernelGGL((logits_decode_rows_kernel<FMT, N, G>), grid, dim3(256), 0, s, a); break;
    IDX_ROWS_CASE(1) IDX_ROWS_CASE(2) IDX_ROWS_CASE(3) IDX_ROWS_CASE(4)
    IDX_ROWS_CASE(5) IDX_ROWS_CASE(6) IDX_ROWS_CASE(7) IDX_ROWS_CASE(8)
#undef IDX_ROWS_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Two 64-token groups per wave while the query tiles leave room in registers: each wave
// then carries twice the K bytes per page-table and Q round trip.  Several query rows
// with more than four head tiles in all are split one row per wave.
template <int FMT>
hipError_t launch_decode(const LogitsArgs& a, int nt, hipStream_t s) {
  const int ht = (a.H + kHeadTile - 1) / kHeadTile;
  if (a.n_q > 1 && nt > 4)
    return ht <= 4 ? launch_decode_rows_g<FMT, 2>(a, ht, s) : launch_decode_rows_g<FMT, 1>(a, ht, s);
  return nt <= 4 ? launch_decode_g<FMT, 2>(a, nt, s) : launch_decode_g<FMT, 1>(a, nt, s);
}

// Host-side plan of the prefill units (assumes every sequence has max_ctx tokens;
// shorter sequences make some units return early).
bool build_prefill_plan(const LogitsArgs& a, PrefillPlan& plan) {
  plan.n_qb = (a.n_q + kPrefillRowsPerBlock - 1) / kPrefillRowsPerBlock;
  int chunk = 1024;
  while ((a.max_ctx + chunk - 1) / chunk > kMaxChunks) chunk *= 2;
  if (chunk > 64 * a.pool.page_size) return false;  // rejected by the API layer first
  plan.chunk = chunk;
  plan.n_chunks = (a.max_ctx + chunk - 1) / chunk;
  if (plan.n_chunks == 0) return false;
  auto reach = [&](int qb) {  // largest valid length among the block's rows
    const int j_last = std::min((qb + 1) * kPrefillRowsPerBlock, a.n_q) - 1;
    int n = a.max_ctx - a.n_q + 1 + j_last;
    return n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
  };
  int32_t units = 0;
  for (int c = 0; c < plan.n_chunks; ++c) {
    int qmin = plan.n_qb;
    for (int lo = 0, hi = plan.n_qb; lo < hi;) {  // first block whose reach exceeds c*chunk
      const int mid = (lo + hi) / 2;
      if (reach(mid) > c * chunk) { hi = mid; qmin = mid; } else { lo = mid + 1; }
    }
    plan.qb_min[c] = qmin;
    plan.unit_start[c] = units;
    units += plan.n_qb - qmin;
  }
  plan.unit_start[plan.n_chunks] = units;
  return units > 0;
}

template <int FMT>
hipError_t launch_prefill(const LogitsArgs& a, int ht, hipStream_t s) {
  PrefillPlan plan;
  if (!build_prefill_plan(a, plan)) return hipSuccess;
  const dim3 grid((unsigned)plan.unit_start[plan.n_chunks], (unsigned)a.B);
  switch (ht) {
#define IDX_PREFILL_CASE(N) \
  case N: hipLaunchKernelGGL((logits_prefill_kernel<FMT, N>), grid, dim3(256), 0, s, a, plan); break;
    IDX_PREFILL_CASE(1) IDX_PREFILL_CASE(2) IDX_PREFILL_CASE(3) IDX_PREFILL_CASE(4)
    IDX_PREFILL_CASE(5) IDX_PREFILL_CASE(6) IDX_PREFILL_CASE(7) IDX_PREFILL_CASE(8)
#undef IDX_PREFILL_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool logits_uses_decode_kernel(int n_q, int H) {
  return n_q * ((H + kHeadTile - 1) / kHeadTile) <= kDecodeMaxTiles;
}

int64_t logits_max_ctx(int n_q, int H, int page_size) {
  if (logits_uses_decode_kernel(n_q, H)) return INT32_MAX;
  // prefill units span one chunk of at most 64 pages, with at most kMaxChunks chunks
  return (int64_t)kMaxChunks * std::min(64 * page_size, 1 << 30);
}

hipError_t launch_logits(const LogitsArgs& args, hipStream_t s, int num_cus) {
  if (args.max_ctx == 0) return hipSuccess;
  const LogitsArgs& a = args;
  const int ht = (a.H + kHeadTile - 1) / kHeadTile;
  // several query rows with many heads: the streaming form with balanced runs
  const bool stream_ok = logits_stream_takes(a.B, a.n_q, a.max_ctx);
  if (stream_ok && a.n_q > 1 && a.n_q * ht > 4) return launch_logits_stream(a, num_cus, s);
  // one row per sequence over many tokens (mixed lengths likely): the streaming form too,
  // with non-temporal K loads (on B64/8K the one-pass kernel stays faster)
  if (stream_ok && a.n_q == 1 && (int64_t)a.B * a.max_ctx >= kStreamTokens) return launch_logits_stream(a, num_cus, s);
  if (logits_uses_decode_kernel(a.n_q, a.H))
    return a.pool.kv_format == 0 ? launch_decode<0>(a, a.n_q * ht, s) : launch_decode<1>(a, a.n_q * ht, s);
  return a.pool.kv_format == 0 ? launch_prefill<0>(a, ht, s) : launch_prefill<1>(a, ht, s);
}

}  // namespace idx
