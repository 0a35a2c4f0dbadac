// Streaming form of the decode scorer (gfx950) for shapes where one pass of short-lived
// waves leaves the memory system idle while they compute: several query rows with many
// heads (e.g. 3 speculative tokens x 64 heads) and long, mixed context lengths.
//
// Work is balanced across workers from the device-side lengths, with no host read: a
// sequence of n_b tokens has ceil(n_b / 64) chunks of 64 tokens; with U chunks in all and
// W workers, every worker takes a contiguous run of at most q = ceil(U / (W - B)) chunks of
// one sequence (sequence b gets ceil(chunks_b / q) workers), so long and short sequences
// finish together and a worker's query tiles stay the same throughout its run.  Each wave
// computes U, q and its own run from the lengths (a wave-wide prefix over the sequences);
// the runs are laid out in order over the XCDs, so a sequence's runs mostly share one L2.
// A worker is a wave when n_q = 1; for n_q = 2..4 it is a block whose four waves stage a
// chunk's K tiles in LDS and whose wave j scores query row j from them, so a chunk's K
// leaves HBM once per block.  A run's page ids are loaded once (RunPages), and the launch
// caps the run length so that they fit its 64-entry window.  Within a run, the next chunks'
// K tiles are in flight while the current one is scored (register buffers used
// alternately); loads are issued on every step, past the run too (page 0 row 0), so the
// outstanding-load count is the same on every path and the compiler's waits stay partial.
#include <algorithm>

#include "scorer.hpp"

namespace idx {
namespace {

constexpr int kStreamMaxSeqs = 64 * 16;  // sequences a wave's prefix covers (16 per lane)

// The worker's run: sequence b and chunks [c0, c1) (c0 >= c1: no work).  Every lane of
// the wave gets the same values.  Lane l holds sequences [l*m, l*m + m).  Worker w is wave
// w % WPB of block w / WPB.  When the block count is a multiple of kXcds, XCD x takes the
// runs [x*per, (x+1)*per) in order (per: the busy runs over kXcds, in whole blocks), so the
// runs of one sequence mostly share one L2 and its query tiles are fetched there once.
template <int M, int WPB>
__device__ __forceinline__ void worker_run(const LogitsArgs& a, int worker, int n_workers, int lane, int& b, int& c0,
                                           int& c1) {
  int ch[M];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const int s = lane * M + i;
    const int n = s < a.B ? std::min(std::max(a.ctx[s], 0), a.max_ctx) : 0;
    ch[i] = (n + 63) >> 6;
    sum += ch[i];
  }
  const int total = __builtin_amdgcn_readlane(wave_incl_scan(sum), 63);  // U (< 2^31: checked on the host)
  const int spare = std::max(n_workers - a.B, 1);
  const int q = std::max(1, (total + spare - 1) / spare);  // chunks per worker
  int wsum = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) wsum += (ch[i] + q - 1) / q;
  const int wincl = wave_incl_scan(wsum);
  const int wexcl = wincl - wsum;
  if ((n_workers / WPB) % kXcds == 0) {
    const int busy = __builtin_amdgcn_readlane(wincl, 63);  // runs with work
    const int per = WPB * ((busy + WPB * kXcds - 1) / (WPB * kXcds));
    const int blk = worker / WPB, slot = blk / kXcds;
    worker = slot * WPB < per ? (blk % kXcds) * per + slot * WPB + worker % WPB : busy;  // busy: no run
  }
  const uint64_t hit = __ballot(wexcl <= worker && worker < wincl);
  b = -1;
  c0 = c1 = 0;
  if (hit == 0) return;  // past the last run (uniform)
  const int L = __builtin_ctzll(hit);
  int bb = 0, cc0 = 0, cc1 = 0;
  if (lane == L) {
    int before = wexcl;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int wi = (ch[i] + q - 1) / q;
      if (before <= worker && worker < before + wi) {
        bb = lane * M + i;
        cc0 = (worker - before) * q;
        cc1 = std::min(cc0 + q, ch[i]);
      }
      before += wi;
    }
  }
  b = __builtin_amdgcn_readlane(bb, L);
  c0 = __builtin_amdgcn_readlane(cc0, L);
  c1 = __builtin_amdgcn_readlane(cc1, L);
}

// Page ids of a worker's run, lane l holding the table entry `first + l` (clamped to the
// row), loaded once beside the query tiles: a chunk's K address then needs no page-table
// round trip inside the loop.  The launch sizes the runs so that every run's pages fit
// this 64-entry window; pages past it (only the loads issued beyond a run's end ask for
// them, and those never use the id) read as an invalid id.
struct RunPages {
  int first, last;
  int32_t ids;
  __device__ __forceinline__ RunPages(const int32_t* row, int first_pg, int last_pg, int lane)
      : first(first_pg), last(last_pg), ids(row[std::min(first_pg + lane, last_pg)]) {}
  __device__ __forceinline__ int32_t at(int pg) const {  // pg uniform and >= first
    const int rel = std::min(pg, last) - first;
    return rel < 64 ? __builtin_amdgcn_readlane(ids, rel) : -1;
  }
};

template <int FMT, int HT, bool NT_LOADS, int M>
__global__ __launch_bounds__(256) void logits_stream_kernel(LogitsArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  int b, c, c_end;
  worker_run<M, 4>(a, blockIdx.x * 4 + wave, gridDim.x * 4, lane, b, c, c_end);
  if (b < 0 || c >= c_end) return;  // uniform: no run for this worker
  const int64_t r = b;  // one query row per sequence
  const int P = a.pool.page_size, lgP = a.pool.page_shift;
  const int last_page = (a.max_ctx - 1) >> lgP;
  const RunPages pages(a.page_table + (int64_t)b * a.max_pages, (64 * c) >> lgP, last_page, lane);

  v8i qa[HT];
  uint32_t qs[HT];
  v4f qw[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    load_q_tile<FMT>(a, r, ht, lane, qa[ht], qs[ht]);
    qw[ht] = load_w_tile(a, r, ht, lane);
  }
  const int n_b = uniform(std::min(std::max(a.ctx[b], 0), a.max_ctx));
  const int n_ch = std::min((n_b + 63) >> 6, c_end);  // the row's chunks inside the run

  const int32_t np32 = (int32_t)std::min<int64_t>(a.pool.num_pages, INT32_MAX);  // page ids are int32
  // Issue the four K tiles of chunk cc (any cc: past the row they read page 0 row 0).
  auto issue = [&](int cc, KTile<FMT>* K, bool* ok) {
    const bool live = cc < n_ch;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int s0 = 64 * cc + 16 * t;
      const int32_t pid = pages.at(s0 >> lgP);
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
    if (s < n_b) out_row[s] = logit;
  };

  KTile<FMT> A[4], B[4];
  bool okA[4], okB[4];
  issue(c, A, okA);
  for (;;) {
    const int c2 = c + 1;
    issue(c2, B, okB);
    consume(c, A, okA);
    if (c2 >= n_ch) break;  // uniform
    const int c3 = c2 + 1;
    issue(c3, A, okA);
    consume(c2, B, okB);
    if (c3 >= n_ch) break;
    c = c3;
  }
}

// Several query rows (n_q = 2..4): a block is one worker; its four waves each fetch one of
// a chunk's four K tiles into registers and then LDS, and wave j < n_q scores query row j
// from all four tiles in LDS, so a chunk's K leaves HBM once per block.  Lane l of every
// wave reads back the operand lane l fetched, which is its own MFMA operand for that tile.
// Two LDS buffers alternate with one barrier per chunk; the fetches of the next two
// chunks are in flight while the current one is scored.  The chunk loop runs over the longest row of
// the sequence (row n_q - 1), the same for every wave; each row stores only its own cells.
template <int FMT>
struct alignas(16) StreamStage {
  uint4 data[2][4][64][FMT == 0 ? 1 : 2];
  uint32_t scale[2][4][64];
};

template <int FMT, int HT, int M>
__global__ __launch_bounds__(256) void logits_stream_rows_kernel(LogitsArgs a) {
  __shared__ StreamStage<FMT> st;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  int b, c0, c_end;
  worker_run<M, 1>(a, blockIdx.x, gridDim.x, lane, b, c0, c_end);
  if (b < 0 || c0 >= c_end) return;  // block-uniform: no run for this worker
  const int j = std::min(wave, a.n_q - 1);  // waves past n_q fetch but do not score
  const bool scorer = wave < a.n_q;
  const int64_t r = (int64_t)b * a.n_q + j;
  const int P = a.pool.page_size, lgP = a.pool.page_shift;
  const int last_page = (a.max_ctx - 1) >> lgP;
  const RunPages pages(a.page_table + (int64_t)b * a.max_pages, (64 * c0) >> lgP, last_page, lane);
  const int32_t np32 = (int32_t)std::min<int64_t>(a.pool.num_pages, INT32_MAX);  // page ids are int32

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
  const int n_end = std::min((n_b + 63) >> 6, c_end);  // the longest row's chunks in the run

  auto page_of = [&](int cc, int t, bool& ok) {  // uniform
    const int32_t pid = pages.at((64 * cc + 16 * t) >> lgP);
    ok = pid >= 0 && pid < np32;
    return pid;
  };
  // this wave's tile (t = wave) of chunk cc; past the run it reads page 0 row 0
  auto fetch = [&](int cc) {
    bool okk;
    const int32_t pid = page_of(cc, wave, okk);
    const bool use = okk && cc < n_end;
    const uint8_t* page = a.pool.base + (use ? (int64_t)pid : 0) * a.pool.stride;
    return load_k_tile_w<FMT, false>(page, P, use ? ((64 * cc + 16 * wave) & (P - 1)) : 0, lane);
  };
  auto stash = [&](int buf, const KTile<FMT>& k) {
    st.data[buf][wave][lane][0] = make_uint4((uint32_t)k.v[0], (uint32_t)k.v[1], (uint32_t)k.v[2], (uint32_t)k.v[3]);
    if (FMT == 1)
      st.data[buf][wave][lane][FMT] = make_uint4((uint32_t)k.v[4], (uint32_t)k.v[5], (uint32_t)k.v[6], (uint32_t)k.v[7]);
    st.scale[buf][wave][lane] = lane_scale<FMT>(k.scale, lane);
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
  const float qnan = __builtin_nanf("");
  float* __restrict__ out_row = a.logits + r * a.lstride;

  // Chunk cc: stage its tile (fetched two chunks earlier into register slot R, the LDS
  // buffer of the same parity), refill R with chunk cc + 2, and score it from LDS.  The
  // two slots alternate, so no register copy waits on a load in flight.
  auto step = [&](int cc, KTile<FMT>& R) {
    const int buf = (cc - c0) & 1;
    stash(buf, R);
    R = fetch(cc + 2);
    __syncthreads();
    if (scorer && cc < n_end && 64 * cc < n_r) {  // uniform per wave
      float p[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const KTile<FMT> kt = unstash(buf, t);
        bool okt;
        (void)page_of(cc, t, okt);
        float acc = 0.0f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc = relu_dot_acc(mfma<FMT>(qa[ht], qs[ht], kt), qw[ht], acc, ht == 0);
        const float v = FMT == 1 ? acc * __uint_as_float(kt.scale) : acc;
        p[t] = okt ? v : qnan;
      }
      const float logit = reduce4_transpose(p[0], p[1], p[2], p[3]);
      const int s = 64 * cc + lane;
      if (s < n_r) out_row[s] = logit;
    }
  };
  // Chunks go in pairs with one exit test per pair (an odd run stages one chunk past its
  // end and scores nothing from it): an exit between the two steps gave the compiler a path
  // on which it waited for every load in flight at the loop head.
  KTile<FMT> A = fetch(c0), B = fetch(c0 + 1);
  for (int cc = c0; cc < n_end; cc += 2) {  // block-uniform trip count
    step(cc, A);
    step(cc + 1, B);
  }
}

// The one-row form loads MXFP4 K non-temporally (read once per call).  An FP8 token row spans
// two 64-byte halves of a line, fetched by separate loads, and cacheable loads let the second
// half find the line the first brought in: large pool 81.5 -> 78 us, while MXFP4 measured 11 %
// slower with cacheable loads.
template <int FMT, int M>
hipError_t launch_stream_m(const LogitsArgs& a, dim3 grid, int ht, hipStream_t s) {
  switch (ht) {
#define IDX_STREAM_CASE(N) \
  case N: \
    if (a.n_q == 1) hipLaunchKernelGGL((logits_stream_kernel<FMT, N, FMT == 0, M>), grid, dim3(256), 0, s, a); \
    else hipLaunchKernelGGL((logits_stream_rows_kernel<FMT, N, M>), grid, dim3(256), 0, s, a); \
    break;
    IDX_STREAM_CASE(1) IDX_STREAM_CASE(2) IDX_STREAM_CASE(3) IDX_STREAM_CASE(4)
    IDX_STREAM_CASE(5) IDX_STREAM_CASE(6) IDX_STREAM_CASE(7) IDX_STREAM_CASE(8)
#undef IDX_STREAM_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_stream_fmt(const LogitsArgs& a, dim3 grid, int ht, hipStream_t s) {
  const int m = (a.B + 63) / 64;
  if (m <= 1) return launch_stream_m<FMT, 1>(a, grid, ht, s);
  if (m <= 2) return launch_stream_m<FMT, 2>(a, grid, ht, s);
  if (m <= 4) return launch_stream_m<FMT, 4>(a, grid, ht, s);
  if (m <= 8) return launch_stream_m<FMT, 8>(a, grid, ht, s);
  return launch_stream_m<FMT, 16>(a, grid, ht, s);
}

}  // namespace

bool logits_stream_takes(int B, int n_q, int max_ctx) {
  // the wave-wide prefix covers up to 1024 sequences; chunk counts stay inside int32
  return n_q >= 1 && n_q <= 4 && B >= 1 && B <= kStreamMaxSeqs && max_ctx <= (1 << 30) &&
         (int64_t)B * ((max_ctx + 63) / 64) < ((int64_t)1 << 31);
}

hipError_t launch_logits_stream(const LogitsArgs& a, int num_cus, hipStream_t s) {
  if (a.max_ctx == 0) return hipSuccess;
  if (!logits_stream_takes(a.B, a.n_q, a.max_ctx)) return hipErrorInvalidValue;
  const int ht = (a.H + kHeadTile - 1) / kHeadTile;
  // Two waves per SIMD of one-row MXFP4 workers, four of FP8 ones (whose 132-byte rows
  // take two loads each: large pool 77.4-78.1 -> 76.4 us, while MXFP4 measured slower with
  // more), or six blocks per CU of several-row workers (fewer, longer runs measured faster
  // than a fuller device: the page ids and query tiles are loaded once per run); at least
  // two workers per sequence (so the balanced runs have room), and no more workers than
  // chunks.  Runs are at most q_cap chunks, so that a run's pages fit the 64-entry page-id
  // window: with spare >= max_units / q_cap workers past one per sequence, the device's
  // q = ceil(U / spare) <= q_cap.
  const int64_t max_units = (int64_t)a.B * ((a.max_ctx + 63) / 64);
  const int64_t q_cap = std::max<int64_t>(1, (int64_t)63 * a.pool.page_size / 64);
  int64_t workers = a.n_q == 1 ? (int64_t)num_cus * (a.pool.kv_format == 0 ? 8 : 16) : (int64_t)num_cus * 6;
  workers = std::max<int64_t>(workers, 2 * (int64_t)a.B);
  workers = std::max<int64_t>(workers, (max_units + q_cap - 1) / q_cap + a.B);
  workers = std::min<int64_t>(workers, max_units + a.B);
  const int64_t blocks = a.n_q == 1 ? (workers + 3) / 4 : workers;
  return a.pool.kv_format == 0 ? launch_stream_fmt<0>(a, dim3((unsigned)blocks), ht, s)
                               : launch_stream_fmt<1>(a, dim3((unsigned)blocks), ht, s);
}

}  // namespace idx
