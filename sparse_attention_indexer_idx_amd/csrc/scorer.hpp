// Scorer building blocks shared by the standalone scorer kernels and the fused decode
// step (gfx950): operand tile loads for v_mfma_scale_f32_16x16x128_f8f6f4, the ReLU /
// weight epilogue, and the decode form's per-wave body.
//
// Operand layout: A = 16 head rows of one query, B = 16 cached tokens; lane l holds row
// (head or token) l%16.  Which of the 128 dims a lane's registers hold depends on the
// element width: with 4-bit elements lane group g = l/16 holds dims [32g, 32g+32) in four
// registers; with 8-bit elements it holds dims [16g, 16g+16) in registers 0-3 and
// [64+16g, 64+16g+16) in registers 4-7.  The scale byte a lane supplies applies to dims
// [32g, 32g+32) in both cases.  Every operand here is loaded so that dim = the
// instruction's k index (so the scale blocks are the dims' own 32-blocks, and an 8-bit
// operand may meet a 4-bit one).  MXFP4 K: 16 bytes at token*64 + 16*(l/16), so one
// wave-wide load covers 16 consecutive tokens = 1 KB contiguous.  Output lane l holds
// heads 4*(l/16)..+3 of token l%16.
#pragma once

#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace idx {

constexpr int kHeadTile = 16;

// Valid length of query j of a sequence with n_b cached tokens.
__device__ __forceinline__ int valid_len(int n_b, int n_q, int j) {
  int n = n_b - n_q + 1 + j;
  return n < 0 ? 0 : (n > n_b ? n_b : n);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// B operand (16 tokens starting at page row `row0` of `page`) and the lane's scale.
// FMT 0: 16 B nibbles + E8M0 byte; FMT 1: 32 B e4m3 + fp32 token scale bits.
template <int FMT>
struct KTile {
  v8i v;
  uint32_t scale;
};

// A load that is either plain or marked non-temporal (STREAM: K bytes read once per
// call, as in decode — the hint keeps them from displacing reused lines in the caches;
// prefill re-reads its K tiles from L2 and loads them plainly).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <bool STREAM, typename T>
__device__ __forceinline__ T ld(const T* p) {
  if (STREAM) return __builtin_nontemporal_load(p);
  return *p;
}

template <int FMT, bool STREAM>
__device__ __forceinline__ KTile<FMT> load_k_tile(const uint8_t* __restrict__ page, int P, int row0, int lane) {
  KTile<FMT> t;
  const uint32_t tok = (uint32_t)(row0 + (lane & 15)), g = (uint32_t)(lane >> 4);
  if (FMT == 0) {
    const u32x4 x = ld<STREAM>((const u32x4*)(page + (tok * 64u + 16u * g)));
    t.v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
    t.scale = ld<STREAM>(page + ((uint32_t)P * 64u + tok * 4u + g));
  } else {
    const u32x4* src = (const u32x4*)(page + (tok * 128u + 16u * g));
    const u32x4 x = ld<STREAM>(src), y = ld<STREAM>(src + 4);  // dims 16g.., 64+16g..
    t.v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
    t.scale = ld<STREAM>((const uint32_t*)(page + ((uint32_t)P * 128u + tok * 4u)));
  }
  return t;
}

// As load_k_tile, but an MXFP4 tile's E8M0 scales come as each token's four bytes in one
// word, which lane_scale shifts to the lane's byte (the MFMA reads the low byte): in a loop, a
// byte load made the compiler wait for every memory operation in flight at the loop head.
template <int FMT, bool STREAM>
__device__ __forceinline__ KTile<FMT> load_k_tile_w(const uint8_t* __restrict__ page, int P, int row0, int lane) {
  if (FMT == 1) return load_k_tile<FMT, STREAM>(page, P, row0, lane);
  KTile<FMT> t;
  const uint32_t tok = (uint32_t)(row0 + (lane & 15)), g = (uint32_t)(lane >> 4);
  const u32x4 x = ld<STREAM>((const u32x4*)(page + (tok * 64u + 16u * g)));
  t.v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  t.scale = ld<STREAM>((const uint32_t*)(page + ((uint32_t)P * 64u + tok * 4u)));
  return t;
}
template <int FMT>
__device__ __forceinline__ uint32_t lane_scale(uint32_t w, int lane) {
  return FMT == 0 ? w >> (8 * (lane >> 4)) : w;
}

// A operand for head tile `ht` of query row r: lane l -> head ht*16 + l%16, block l/16.
// Branch-free: a head past H loads head H-1 and is zeroed by a select after the load, so
// the loads of every tile go out together and nothing waits for them before first use.
template <int FMT>
__device__ __forceinline__ void load_q_tile(const LogitsArgs& a, int64_t r, int ht, int lane, v8i& v,
                                            uint32_t& sc) {
  const int h = ht * kHeadTile + (lane & 15), g = lane >> 4;
  const bool hv = h < a.H;
  const int64_t vec = r * a.H + (hv ? h : a.H - 1);
  if (FMT == 0) {
    const uint4 x = *(const uint4*)(a.q + vec * 64 + 16 * g);
    v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
    sc = a.q_scale[vec * 4 + g];
  } else {
    const uint4* src = (const uint4*)(a.q + vec * 128 + 16 * g);
    const uint4 x = src[0], y = src[4];  // dims 16g.., 64+16g..
    v = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
    sc = kE8m0One;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = hv ? v[i] : 0;
}

// Weights of the four accumulator rows lane l holds for head tile ht of row r (heads
// ht*16 + 4*(l/16) + i); a head past H gets weight 0.
__device__ __forceinline__ v4f load_w_tile(const LogitsArgs& a, int64_t r, int ht, int lane) {
  const int h0 = ht * kHeadTile + 4 * (lane >> 4);
  v4f w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = h0 + i;
    const float x = a.w[r * a.H + (h < a.H ? h : a.H - 1)];
    w[i] = h < a.H ? x : 0.0f;
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

// ReLU on the fp32 bit pattern: every negative value (and -0.0) has a negative int32
// pattern, so an integer max with 0 is ReLU in one instruction, with none of the NaN
// canonicalisation a floating-point max carries.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// acc + sum_i w_i * ReLU(d_i) as one multiply-add chain (first: start from w_0 * ReLU(d_0)).
__device__ __forceinline__ float relu_dot_acc(const v4f& d, const v4f& w, float acc, bool first) {
  float s = first ? w[0] * relu(d[0]) : fmaf(w[0], relu(d[0]), acc);
  s = fmaf(w[1], relu(d[1]), s);
  s = fmaf(w[2], relu(d[2]), s);
  s = fmaf(w[3], relu(d[3]), s);
  return s;
}

__device__ __forceinline__ float relu_dot(const v4f& d, const v4f& w) {
  float s = w[0] * relu(d[0]);
  s += w[1] * relu(d[1]);
  s += w[2] * relu(d[2]);
  s += w[3] * relu(d[3]);
  return s;
}

// ------------------------------------------------------------------------------------
// Decode: every query row of a sequence in registers (n_q * ceil(H/16) <= 16 head
// tiles), one wave per G*64 consecutive cached tokens (G groups of four 16-token tiles).
// Per wave: Q and w loads, then the page ids of its tiles and the sequence length
// together, then all K loads, before the first use.  Patch::kCoherentStores makes the
// logits stores device-coherent; Patch::kNewRows rescores new tokens at the end.
// ------------------------------------------------------------------------------------
constexpr int kDecodeMaxTiles = 16;

// Hooks of the decode wave body: the plain scorer has none; the fused decode step stores
// its logits device-coherently and rescoring its new tokens (see NewRows).
struct NoPatch {
  static constexpr bool kCoherentStores = false;
  static constexpr bool kNewRows = false;
  __device__ __forceinline__ void prepare(int) {}
  __device__ __forceinline__ bool skip(int) const { return false; }
  __device__ __forceinline__ bool rescorer() const { return false; }
  template <int FMT>
  __device__ __forceinline__ bool new_row(int, int, KTile<FMT>&, int&, int&) const {
    return false;
  }
};

// The wave scores query rows j_base .. j_base + NT/HT - 1 of sequence b (all n_q rows when
// j_base = 0 and NT = n_q * HT; one row when NT = HT).  EXIT_DEAD: a wave wholly past its
// sequence leaves before its K loads (worth it where many waves are: many heads and mixed
// lengths); the price is that the compiler then issues the Q loads after the page-table
// round trip instead of before it, so the single-row decode kernel does without.
// STREAM_K: K loads are non-temporal (read once per call).  By default on for MXFP4 only: an
// FP8 token row is two 64-byte halves of a line fetched by separate loads, and cacheable
// loads let the second find the line the first brought in (fused decode step, B64/H32/8K
// FP8: 23.8 -> 22.3 us); off too where several waves read the same tiles from the cache.
template <int FMT, int NT, int G, class Patch, bool EXIT_DEAD = false, bool STREAM_K = (FMT == 0)>
__device__ __forceinline__ void decode_wave(const LogitsArgs& a, int b, int tok0, int lane, Patch& patch,
                                            int j_base = 0) {
  constexpr int T = 4 * G;  // K tiles per wave
  const int P = a.pool.page_size, lgP = a.pool.page_shift;
  const int last_page = (a.max_ctx - 1) >> lgP;
  const int32_t* __restrict__ ptb = a.page_table + (int64_t)b * a.max_pages;

  // Q and w first: they do not depend on the page table and come from L2, so they are
  // in registers by the time the K bytes arrive.  Without EXIT_DEAD there is no early
  // exit: a wave past the end of the context reads page 0 row 0 for every tile (an L2
  // hit shared by all such waves) and stores nothing, so no branch stands between these
  // loads and the page-table round trip.
  const int HT = (a.H + kHeadTile - 1) / kHeadTile;
  v8i qa[NT];
  uint32_t qs[NT];
  v4f qw[NT];
#pragma unroll
  for (int m = 0; m < NT; ++m) {
    const int j = j_base + m / HT, ht = m % HT;
    const int64_t r = (int64_t)b * a.n_q + j;
    load_q_tile<FMT>(a, r, ht, lane, qa[m], qs[m]);
    qw[m] = load_w_tile(a, r, ht, lane);
  }

  // The tile page ids (clamped into the sequence's table row) and the length, together.
  int32_t pid[T];
#pragma unroll
  for (int t = 0; t < T; ++t) pid[t] = uniform(ptb[std::min((tok0 + 16 * t) >> lgP, last_page)]);
  const int n_b = uniform(std::min(std::max(a.ctx[b], 0), a.max_ctx));
  const bool live = tok0 < n_b;  // n_b <= max_ctx, so this also covers waves past max_ctx
  patch.prepare(n_b);
  if (EXIT_DEAD && !live) return;  // nothing to store

  // K tiles: a tile of a dead wave or on an invalid page reads page 0 row 0 (always
  // inside the pool); invalid pages score NaN below, dead waves store nothing.
  KTile<FMT> kt[T];
  bool ok[T];
  const int32_t np32 = (int32_t)std::min<int64_t>(a.pool.num_pages, INT32_MAX);  // page ids are int32
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int s0 = tok0 + 16 * t;
    const bool valid_page = pid[t] >= 0 && pid[t] < np32;
    const bool use = live && valid_page;
    const uint8_t* page = a.pool.base + (use ? (int64_t)pid[t] : 0) * a.pool.stride;
    kt[t] = load_k_tile<FMT, STREAM_K>(page, P, use ? (s0 & (P - 1)) : 0, lane);
    ok[t] = valid_page;  // tiles past n_b are computed but never stored
  }

  const float qnan = __builtin_nanf("");
  auto store = [&](int j, int s, float logit) {
    float* dst = a.logits + ((int64_t)b * a.n_q + j) * a.lstride + s;
    if (Patch::kCoherentStores)  // device-coherent: visible to other XCDs once complete
      __hip_atomic_store(dst, logit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *dst = logit;
  };
  // One group of four 16-token tiles: head tiles m = j*HT .. j*HT+HT-1 belong to query
  // row j; every MFMA runs unconditionally (so nothing sinks the Q loads behind a branch),
  // and a row is finished — head reduction, transpose, emit — once its last tile is in.
  // Lane l of the result holds token s0 + l.
  auto score_group = [&](const KTile<FMT>* k4, const bool* ok4, auto&& emit) {
    float acc[4];
#pragma unroll
    for (int m = 0; m < NT; ++m) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float v = relu_dot(mfma<FMT>(qa[m], qs[m], k4[t]), qw[m]);
        acc[t] = (m % HT == 0) ? v : acc[t] + v;
      }
      if ((m + 1) % HT == 0) {  // uniform
        float p[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float v = FMT == 1 ? acc[t] * __uint_as_float(k4[t].scale) : acc[t];
          p[t] = ok4[t] ? v : qnan;
        }
        emit(j_base + m / HT, reduce4_transpose(p[0], p[1], p[2], p[3]));
      }
    }
  };
  // A dead wave (tok0 >= n_b) stores nothing: s >= tok0 >= n_b >= every valid length.
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int s = tok0 + 64 * g + lane;
    score_group(&kt[4 * g], &ok[4 * g], [&](int j, float logit) {
      if (s < valid_len(n_b, a.n_q, j) && !patch.skip(s)) store(j, s, logit);
    });
  }

  if constexpr (Patch::kNewRows) {
    // The fused decode step's new tokens: the wave that holds one skips its logit above,
    // and one early-finishing wave of the block computes the token's K row (stored to
    // the pool for later steps) and scores the token from the fresh row, in the tile slot
    // and lane the token occupies in its own wave, so the logit is bit-identical to
    // scoring a pool that already held the row.  Only column (token % 16) of the new
    // tile matters.
    if (patch.rescorer()) {
      for (int jn = 0; jn < a.n_q; ++jn) {  // uniform
        KTile<FMT> nk;
        int s_new, slot4;
        if (!patch.template new_row<FMT>(jn, lane, nk, s_new, slot4)) continue;
        // page validity of the token's tile, as its own wave sees it
        const int32_t pid_new = uniform(ptb[std::min(s_new >> lgP, last_page)]);
        const bool okt = pid_new >= 0 && pid_new < np32;
        const KTile<FMT> k4[4] = {nk, nk, nk, nk};
        const bool ok4[4] = {okt, okt, okt, okt};
        const bool mine = lane == 16 * slot4 + (s_new & 15);
        score_group(k4, ok4, [&](int j, float logit) {
          if (mine && s_new < valid_len(n_b, a.n_q, j)) store(j, s_new, logit);
        });
      }
    }
  }
}

}  // namespace idx
