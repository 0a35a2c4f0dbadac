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
#include "device_common.hpp"
#include "launch.hpp"

namespace idx {
namespace {

constexpr int kHeadTile = 16;

struct Page {
  const uint8_t* base;  // start of the physical page, or null for an invalid page id
};

__device__ __forceinline__ Page page_of(const LogitsArgs& a, int b, int64_t s) {
  const int32_t pid = a.page_table[(int64_t)b * a.max_pages + s / a.pool.page_size];
  Page p;
  p.base = (pid >= 0 && pid < a.pool.num_pages) ? a.pool.base + (int64_t)pid * a.pool.stride : nullptr;
  return p;
}

// Valid length of query j of a sequence with n_b cached tokens.
__device__ __forceinline__ int valid_len(int n_b, int n_q, int j) {
  int n = n_b - n_q + 1 + j;
  return n < 0 ? 0 : (n > n_b ? n_b : n);
}

// B operand (16 tokens starting at page row `row0`) and the lane's scale byte / fp32
// token scale.  FMT 0: 16 B nibbles + E8M0 byte; FMT 1: 32 B e4m3 + fp32 scale.
template <int FMT>
struct KTile {
  v8i v;
  uint32_t scale;  // E8M0 byte in bits 0..7 (MXFP4) or fp32 bits of the token scale (FP8)
};

template <int FMT>
__device__ __forceinline__ KTile<FMT> load_k_tile(const uint8_t* page, int P, int row0, int lane) {
  KTile<FMT> t;
  const int tok = row0 + (lane & 15), g = lane >> 4;
  if (FMT == 0) {
    const uint4 x = *(const uint4*)(page + (int64_t)tok * 64 + 16 * g);
    t.v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
    t.scale = page[(int64_t)P * 64 + tok * 4 + g];
  } else {
    const uint4* src = (const uint4*)(page + (int64_t)tok * 128 + 32 * g);
    const uint4 x = src[0], y = src[1];
    t.v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
    t.scale = *(const uint32_t*)(page + (int64_t)P * 128 + tok * 4);
  }
  return t;
}

// A operand for head tile `ht` of query row r: lane l -> head ht*16 + l%16, block l/16.
template <int FMT>
__device__ __forceinline__ void load_q_tile(const LogitsArgs& a, int64_t r, int ht, int lane, v8i& v,
                                            uint32_t& sc) {
  const int h = ht * kHeadTile + (lane & 15), g = lane >> 4;
  v = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  sc = 0;
  if (h >= a.H) return;
  const int64_t vec = r * a.H + h;
  if (FMT == 0) {
    const uint4 x = *(const uint4*)(a.q + vec * 64 + 16 * g);
    v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
    sc = a.q_scale[vec * 4 + g];
  } else {
    const uint4* src = (const uint4*)(a.q + vec * 128 + 32 * g);
    const uint4 x = src[0], y = src[1];
    v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
    sc = kE8m0One;
  }
}

// Weights of the four accumulator rows lane l holds for head tile ht of row r.
__device__ __forceinline__ v4f load_w_tile(const LogitsArgs& a, int64_t r, int ht, int lane) {
  v4f w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = ht * kHeadTile + 4 * (lane >> 4) + i;
    w[i] = (h < a.H) ? a.w[r * a.H + h] : 0.0f;
  }
  return w;
}

template <int FMT>
__device__ __forceinline__ v4f mfma(const v8i& A, uint32_t sa, const KTile<FMT>& K) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  if (FMT == 0)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, K.v, zero, kMfmaFmtFp4, kMfmaFmtFp4, 0, (int)sa, 0,
                                                             (int)K.scale);
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, K.v, zero, kMfmaFmtFp8, kMfmaFmtFp8, 0, (int)sa, 0,
                                                           (int)kE8m0One);
}

__device__ __forceinline__ float relu_dot(const v4f& d, const v4f& w) {
  float s = w[0] * fmaxf(d[0], 0.0f);
  s += w[1] * fmaxf(d[1], 0.0f);
  s += w[2] * fmaxf(d[2], 0.0f);
  s += w[3] * fmaxf(d[3], 0.0f);
  return s;
}

// ------------------------------------------------------------------------------------
// Decode: every query row of a sequence in registers (n_q * ceil(H/16) <= 8 head tiles),
// one wave per 64 consecutive cached tokens (four 16-token tiles), 4 waves per block.
// grid = (ceil(max_ctx / 256), B).
// ------------------------------------------------------------------------------------
constexpr int kDecodeMaxTiles = 8;
constexpr int kDecodeTokPerWave = 64;
constexpr int kDecodeWaves = 4;

template <int FMT, int NT>
__global__ __launch_bounds__(256) void logits_decode_kernel(LogitsArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int n_b = min(max(a.ctx[b], 0), a.max_ctx);
  const int tok0 = (blockIdx.x * kDecodeWaves + wave) * kDecodeTokPerWave;
  if (tok0 >= n_b) return;
  const int HT = (a.H + kHeadTile - 1) / kHeadTile;
  const int P = a.pool.page_size;

  // Issue the K loads of all four tiles first (the whole 64-token span in flight).
  KTile<FMT> kt[4];
  bool ok[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int s0 = tok0 + 16 * t;
    ok[t] = false;
    if (s0 < n_b) {
      const Page pg = page_of(a, b, s0);
      if (pg.base) {
        kt[t] = load_k_tile<FMT>(pg.base, P, s0 % P, lane);
        ok[t] = true;
      }
    }
  }

  v8i qa[NT];
  uint32_t qs[NT];
  v4f qw[NT];
#pragma unroll
  for (int m = 0; m < NT; ++m) {
    const int j = m / HT, ht = m % HT;
    const int64_t r = (int64_t)b * a.n_q + j;
    load_q_tile<FMT>(a, r, ht, lane, qa[m], qs[m]);
    qw[m] = load_w_tile(a, r, ht, lane);
  }

  const float qnan = __builtin_nanf("");
  for (int j = 0; j < a.n_q; ++j) {
    float p[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float acc = 0.0f;
      if (ok[t]) {
#pragma unroll
        for (int m = 0; m < NT; ++m)
          if (m / HT == j) acc += relu_dot(mfma<FMT>(qa[m], qs[m], kt[t]), qw[m]);
        if (FMT == 1) acc *= __uint_as_float(kt[t].scale);
      } else {
        acc = qnan;
      }
      p[t] = acc;
    }
    const float logit = reduce4_transpose(p[0], p[1], p[2], p[3]);
    const int s = tok0 + lane;
    if (s < valid_len(n_b, a.n_q, j)) a.logits[((int64_t)b * a.n_q + j) * a.lstride + s] = logit;
  }
}

// ------------------------------------------------------------------------------------
// Prefill / long query sets: each wave owns 4 query rows (one per lane group after the
// transpose-reduce) and walks 16-token K tiles; a block is 4 waves = 16 rows.  Work
// units are (16-row block, token chunk) pairs enumerated chunk-major from a host-built
// table so that no unit is empty and all units have similar cost.
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

template <int FMT, int HT>
__global__ __launch_bounds__(256) void logits_prefill_kernel(LogitsArgs a, PrefillPlan plan) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  // unit -> (chunk c, row block qb): binary search of the prefix table (scalar).
  const int u = blockIdx.x;
  int lo = 0, hi = plan.n_chunks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (plan.unit_start[mid] <= u) lo = mid; else hi = mid - 1;
  }
  const int c = lo;
  const int qb = plan.n_qb - 1 - (u - plan.unit_start[c]);  // heaviest row blocks first
  const int n_b = min(max(a.ctx[b], 0), a.max_ctx);
  const int j0 = qb * kPrefillRowsPerBlock + wave * kPrefillRowsPerWave;
  if (j0 >= a.n_q) return;
  const int j_last = min(j0 + kPrefillRowsPerWave, a.n_q) - 1;
  const int t_end = min(valid_len(n_b, a.n_q, j_last), (c + 1) * plan.chunk);
  const int t_begin = c * plan.chunk;
  if (t_begin >= t_end) return;
  const int P = a.pool.page_size;

  v8i qa[kPrefillRowsPerWave][HT];
  uint32_t qs[kPrefillRowsPerWave][HT];
  v4f qw[kPrefillRowsPerWave][HT];
  int nv[kPrefillRowsPerWave];
#pragma unroll
  for (int g = 0; g < kPrefillRowsPerWave; ++g) {
    const int j = min(j0 + g, a.n_q - 1);
    const int64_t r = (int64_t)b * a.n_q + j;
    nv[g] = (j0 + g < a.n_q) ? valid_len(n_b, a.n_q, j0 + g) : 0;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      load_q_tile<FMT>(a, r, ht, lane, qa[g][ht], qs[g][ht]);
      qw[g][ht] = load_w_tile(a, r, ht, lane);
    }
  }
  // the valid length this lane's output column belongs to after the transpose
  const int my_n = nv[lane >> 4];
  float* out_row = a.logits + ((int64_t)b * a.n_q + min(j0 + (lane >> 4), a.n_q - 1)) * a.lstride;

  const float qnan = __builtin_nanf("");
  // Software pipeline: the next tile's operands load while this tile computes.
  int s0 = t_begin;
  Page pg = page_of(a, b, s0);
  KTile<FMT> cur;
  if (pg.base) cur = load_k_tile<FMT>(pg.base, P, s0 % P, lane);
  bool cur_ok = pg.base != nullptr;
  for (; s0 < t_end; s0 += 16) {
    KTile<FMT> nxt;
    bool nxt_ok = false;
    const int s1 = s0 + 16;
    if (s1 < t_end) {
      const Page pn = page_of(a, b, s1);
      if (pn.base) {
        nxt = load_k_tile<FMT>(pn.base, P, s1 % P, lane);
        nxt_ok = true;
      }
    }
    float p[kPrefillRowsPerWave];
#pragma unroll
    for (int g = 0; g < kPrefillRowsPerWave; ++g) {
      float acc = 0.0f;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) acc += relu_dot(mfma<FMT>(qa[g][ht], qs[g][ht], cur), qw[g][ht]);
      if (FMT == 1) acc *= __uint_as_float(cur.scale);
      p[g] = cur_ok ? acc : qnan;
    }
    const float logit = reduce4_transpose(p[0], p[1], p[2], p[3]);
    const int s = s0 + (lane & 15);
    if (s < my_n) out_row[s] = logit;
    cur = nxt;
    cur_ok = nxt_ok;
  }
}

template <int FMT>
hipError_t launch_decode(const LogitsArgs& a, int nt, hipStream_t s) {
  const dim3 grid((unsigned)((a.max_ctx + kDecodeWaves * kDecodeTokPerWave - 1) / (kDecodeWaves * kDecodeTokPerWave)),
                  (unsigned)a.B);
  switch (nt) {
#define IDX_DECODE_CASE(N) \
  case N: hipLaunchKernelGGL((logits_decode_kernel<FMT, N>), grid, dim3(256), 0, s, a); break;
    IDX_DECODE_CASE(1) IDX_DECODE_CASE(2) IDX_DECODE_CASE(3) IDX_DECODE_CASE(4)
    IDX_DECODE_CASE(5) IDX_DECODE_CASE(6) IDX_DECODE_CASE(7) IDX_DECODE_CASE(8)
#undef IDX_DECODE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Host-side plan of the prefill units (assumes every sequence has max_ctx tokens;
// shorter sequences make some units return early).
bool build_prefill_plan(const LogitsArgs& a, PrefillPlan& plan) {
  plan.n_qb = (a.n_q + kPrefillRowsPerBlock - 1) / kPrefillRowsPerBlock;
  int chunk = 1024;
  while ((a.max_ctx + chunk - 1) / chunk > kMaxChunks) chunk *= 2;
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

hipError_t launch_logits(const LogitsArgs& a, hipStream_t s) {
  if (a.max_ctx == 0) return hipSuccess;
  const int ht = (a.H + kHeadTile - 1) / kHeadTile;
  const int nt = a.n_q * ht;
  if (nt <= kDecodeMaxTiles)
    return a.pool.kv_format == 0 ? launch_decode<0>(a, nt, s) : launch_decode<1>(a, nt, s);
  return a.pool.kv_format == 0 ? launch_prefill<0>(a, ht, s) : launch_prefill<1>(a, ht, s);
}

}  // namespace idx
