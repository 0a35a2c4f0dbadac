// Per-row top-k on gfx950, shared by the top-k kernel and the fused decode step (page
// "Dense MXFP4 indexer for DeepSeek-V4 on ROCm", Purpose: 1024 tokens kept per query).
//
// One workgroup per row.  The row's valid cells are held in registers as order-
// preserving 32-bit keys (thread t holds cells t, t+NT, t+2NT, ...: every load is a
// contiguous 256-byte wave access, and all of a row's loads are in flight together); a row
// of more than 32 cells per thread is re-read for each pass instead (topk_row_stream).
//   pass 1 — an LDS histogram of the top D1 key bits (13 for 1024-thread rows, 12 for
//            smaller blocks, which share a CU several at a time) picks the digit d1
//            holding the k-th key: cells above d1 are selected, cells below are not;
//   one block scan of two per-thread counts (cells above the bucket, cells in it) gives
//   every thread the output slots of its selected cells and the list slots of its
//   bucket cells;
//   the bucket (tens to a few hundred keys) is resolved by ranking: it is counting-sorted
//   by the next 8 key bits, and each candidate counts the candidates ordered before it by
//   (key desc, index asc) in higher digits and in its own digit's run; rank < the number
//   still needed is selected, and the rank is its output slot.
// A row whose bucket is larger than the ranking list (long runs of equal values) takes a
// slower exact path: two more histogram passes over the keys fix K*, and ranks in index
// order come from wave ballots and per-(round, wave) counts.  Either way equal logits
// resolve toward the smaller index and the output order is deterministic.
#pragma once

#include "device_common.hpp"

namespace idx {


// Order-preserving 32-bit key of an fp32 logit, by arithmetic only (no compare, so no
// lane mask stays live across a row's unrolled rounds): adding +0.0 turns -0.0 into
// +0.0 (denormals are kept: the kernels run with fp32 denormals on), then non-negative
// values get the sign bit set and negative ones are complemented.  Key 0 is reserved
// for a cell that is not a candidate (past the row's valid length), which then ranks
// below every valid one; the one fp32 pattern that would map to 0 (a negative NaN with
// every payload bit set) takes key 1 in dense rows.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// All ones when rel < 0 (a cell index below the row's length), else 0.  The empty asm
// keeps the mask an opaque register value: as a plain shift the compiler rewrites the
// masking as a compare and select, and then keeps one 64-bit lane mask per unrolled round
// live in scalar registers, which spill.
__device__ __forceinline__ uint32_t below_mask(int rel) {
  uint32_t m = (uint32_t)(rel >> 31);
  asm volatile("" : "+v"(m));
  return m;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }

constexpr int kRankCap = 1024;  // largest bucket resolved by ranking
constexpr int kFbBins = 1024;   // histogram size of the two fallback passes

template <int NT>
struct Cfg {
  static constexpr int D1 = NT >= 1024 ? 13 : 12;  // key bits resolved by pass 1
  static constexpr int Shift = 32 - D1;
  static constexpr int Bins = 1 << D1;
  static constexpr int FbBitsA = 10;                // fallback pass A: next 10 bits
  static constexpr int FbBitsB = Shift - FbBitsA;   // fallback pass B: the rest (9 or 10)
};

template <int NT, int EPT>
struct alignas(16) TopkShared {
  uint32_t hist[Cfg<NT>::Bins + 256];  // pass 1's digits, then a large bucket's second digits
  uint64_t cand[kRankCap];  // (key << 32) | ~index: one unsigned compare orders the bucket
  int32_t wave_tot[2 * (NT / 64)];
  int32_t cnt_gt[EPT * (NT / 64)];
  int32_t cnt_eq[EPT * (NT / 64)];
  int32_t sel_digit;
  int32_t sel_above;
};

// Exclusive prefix sum of v over the block in thread order (and the block total): a DPP
// wave scan, one LDS slot per wave, one barrier.  The caller keeps a barrier between two
// calls (wave_tot is reused).
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int32_t* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = wave_tot[w];
    tot += t;
    if (w < wave) before += t;
  }
  total = tot;
  return before + incl - v;
}

// Two exclusive prefix sums at once (one barrier): outputs the prefixes and the totals.
template <int NT>
__device__ __forceinline__ void block_excl_scan2(int v0, int v1, int32_t* wave_tot, int& pre0, int& pre1, int& tot0,
                                                 int& tot1) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i0 = wave_incl_scan(v0), i1 = wave_incl_scan(v1);
  if (lane == 63) {
    wave_tot[2 * wave] = i0;
    wave_tot[2 * wave + 1] = i1;
  }
  __syncthreads();
  int b0 = 0, b1 = 0, t0 = 0, t1 = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int x0 = wave_tot[2 * w], x1 = wave_tot[2 * w + 1];
    t0 += x0;
    t1 += x1;
    if (w < wave) {
      b0 += x0;
      b1 += x1;
    }
  }
  pre0 = b0 + i0 - v0;
  pre1 = b1 + i1 - v1;
  tot0 = t0;
  tot1 = t1;
}

// Given a histogram of BINS digits (BINS >= NT), find the digit d holding the kk-th
// largest item (kk >= 1): count(digits > d) < kk <= count(digits >= d), with the whole
// block (the form for 1024-thread rows, where it measured faster).  Thread t covers
// BINS/NT consecutive digits, the highest to thread 0, read as 16-byte words and kept in
// registers; only the thread whose range holds the answer walks its bins.  Leaves d and
// count(> d) in shared memory (two barriers).
template <int NT, int BINS, class SH>
__device__ __forceinline__ void select_digit_block(SH& sh, int kk) {
  constexpr int PER = BINS / NT;
  const int lo = BINS - PER * ((int)threadIdx.x + 1);  // digits [lo, lo + PER)
  uint32_t c[PER];
  if constexpr (PER % 4 == 0) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const uint4 v = reinterpret_cast<const uint4*>(sh.hist + lo)[q];
      c[4 * q] = v.x;
      c[4 * q + 1] = v.y;
      c[4 * q + 2] = v.z;
      c[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < PER; ++q) c[q] = sh.hist[lo + q];
  }
  int local = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) local += (int)c[q];
  int total;
  int before = block_excl_scan<NT>(local, sh.wave_tot, total);
  if (before < kk && kk <= before + local) {
#pragma unroll
    for (int q = PER - 1; q >= 0; --q) {
      const int cq = (int)c[q];
      if (before < kk && kk <= before + cq) {
        sh.sel_digit = lo + q;
        sh.sel_above = before;
      }
      before += cq;
    }
  }
  __syncthreads();
}

// The same with wave 0 alone, the form for the smaller blocks, which share a CU several at
// a time (prefill top-k 49 -> 47 us; 1024-thread rows measured slower with it).  Lane l
// sums the BINS/64 consecutive digits [lo, lo + BINS/64) with lo = BINS - (l + 1) *
// BINS/64 (the highest digits to lane 0), reading its 16-byte words in an order rotated by
// the lane so that one read instruction spreads over the LDS banks (in digit order every
// lane would hit the same banks); a wave scan finds the lane whose range holds the kk-th
// item, and a second scan over that range's digits, at most two per lane, finds the digit.
// Requires kk <= the histogram's total.  Leaves d and count(> d) in shared memory; one
// barrier.
template <int NT, int BINS, class SH>
__device__ __forceinline__ void select_digit_wave(SH& sh, int kk) {
  static_assert(BINS == 1024 || BINS == 4096 || BINS == 8192, "16, 64 or 128 digits per lane");
  constexpr int PER = BINS / 64;               // digits per lane
  constexpr int Q = PER / 4;                   // 16-byte words per lane
  constexpr int P2 = PER >= 64 ? PER / 64 : 1;  // digits per lane in the second scan
  constexpr int N2 = PER / P2;                 // lanes in the second scan
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int lo = BINS - PER * (lane + 1);
    int local = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const uint4 v = reinterpret_cast<const uint4*>(sh.hist + lo)[(q + lane) & (Q - 1)];
      local += (int)(v.x + v.y + v.z + v.w);
    }
    const int incl = wave_incl_scan(local);
    const int before = incl - local;
    const uint64_t own = __ballot(before < kk && kk <= incl);  // exactly one lane
    const int L = own ? __builtin_ctzll(own) : 0;
    const int base = __builtin_amdgcn_readlane(before, L);
    const int lo2 = BINS - PER * (L + 1) + PER - P2 * (lane + 1);  // lane's digits in L's range
    int cnt[P2], c2 = 0;
#pragma unroll
    for (int q = 0; q < P2; ++q) {
      cnt[q] = lane < N2 ? (int)sh.hist[lo2 + q] : 0;
      c2 += cnt[q];
    }
    const int incl2 = wave_incl_scan(c2);
    int b = base + incl2 - c2;
    if (b < kk && kk <= b + c2) {  // one lane: walk its digits from the highest
#pragma unroll
      for (int q = P2 - 1; q >= 0; --q) {
        if (b < kk && kk <= b + cnt[q]) {
          sh.sel_digit = lo2 + q;
          sh.sel_above = b;
        }
        b += cnt[q];
      }
    }
  }
  __syncthreads();
}

template <int NT, int BINS, class SH>
__device__ __forceinline__ void select_digit(SH& sh, int kk) {
  if constexpr (NT >= 1024) select_digit_block<NT, BINS>(sh, kk);
  else select_digit_wave<NT, BINS>(sh, kk);
}

// Runs f(e) for every round e < EPT whose group of 8 rounds holds a valid cell: a group
// wholly past ne (the rounds holding valid cells) is skipped by one uniform branch, and
// inside a group every round runs (a round past ne holds only key 0, which no phase
// selects), so no per-round condition has to stay live across the unrolled loops.
template <int EPT, class F>
__device__ __forceinline__ void for_rounds(int ne, F&& f) {
#pragma unroll
  for (int g = 0; g < EPT; g += 8) {
    if (g == 0 || g < ne) {
#pragma unroll
      for (int e = g; e < (g + 8 < EPT ? g + 8 : EPT); ++e) f(e);
    }
  }
}

// Runs f(e, load(e)) for every round e < EPT, in groups of 8 rounds with the next group's
// loads in flight while the current one is used: two register sets used alternately, in a
// loop kept rolled (unrolled, the compiler hoisted every load and spilled), so no register
// copy waits on a load.  No branch on the row's length: a load past the row reads 0 (buffer
// range check), which the callers mask to key 0.
template <int EPT, class L, class F>
__device__ __forceinline__ void stream_rounds(L&& load, F&& f) {
  constexpr int G = 8;  // groups of 16 measured slower (65536-cell rows: 27.1 against 25.1 us)
  static_assert(EPT % (2 * G) == 0, "whole pairs of groups");
  float A[G], B[G];
#pragma unroll
  for (int i = 0; i < G; ++i) A[i] = load(i);
#pragma unroll 1
  for (int g = 0; g < EPT; g += 2 * G) {
#pragma unroll
    for (int i = 0; i < G; ++i) B[i] = load(g + G + i);
#pragma unroll
    for (int i = 0; i < G; ++i) f(g + i, A[i]);
#pragma unroll
    for (int i = 0; i < G; ++i) A[i] = load(g + 2 * G + i);  // past EPT on the last pair: reads 0, unused
#pragma unroll
    for (int i = 0; i < G; ++i) f(g + G + i, B[i]);
  }
}

// How a row's cells become keys and output indices.  DenseRow: every cell below n is
// valid and is its own token index.  CandidateRow: cell c*P + i is token
// cand[c]*P + i, and a cell holding -inf is not a candidate (the candidate scorer writes
// -inf there), so the number of valid cells is only known once the keys are formed.
// key(f, rel): the key of cell value f, where rel = cell - n (negative inside the row).
struct DenseRow {
  static constexpr bool kCountValid = false;
  __device__ __forceinline__ uint32_t key_full(float f) const { return max(order_key(f), 1u); }
  __device__ __forceinline__ uint32_t key(float f, int rel) const { return key_full(f) & below_mask(rel); }
  __device__ __forceinline__ int32_t token(int cell) const { return cell; }
};

struct CandidateRow {
  static constexpr bool kCountValid = true;
  const int32_t* cand;
  int32_t page_shift;
  // -inf (key 0x007FFFFF) and the negative NaNs below it (keys < 2^23) are not
  // candidates: key 0.  ((k >> 23) - 1 is negative exactly for those keys.)
  __device__ __forceinline__ uint32_t key_full(float f) const {
    const uint32_t k = order_key(f);
    return k & ~(uint32_t)((int32_t)((k >> 23) - 1u) >> 31);
  }
  __device__ __forceinline__ uint32_t key(float f, int rel) const { return key_full(f) & below_mask(rel); }
  __device__ __forceinline__ int32_t token(int cell) const {
    return (cand[cell >> page_shift] << page_shift) + (cell & ((1 << page_shift) - 1));
  }
};

// Ranking the bucket by a second digit, the 8 key bits below pass 1's digit.  The bucket is
// counting-sorted by that digit into LDS (digits descending; the order inside a digit's run
// is whatever the atomics give), and each candidate's rank is the number of candidates in
// higher digits plus those of its own run ordered before it by (key desc, index asc): the
// exact rank, and so the output slot, at a cost of the run length per candidate instead of
// the bucket size.  (Measured against ranking over the whole bucket with lane groups sharing
// a candidate: as fast or faster at every bucket size of the benchmark rows.)  The 256
// counters follow pass 1's bins (cleared with them); the run starts and the sorted list
// reuse pass 1's words, dead by then.  Three barriers.  Out of line: inlined, it pushed the
// 256-thread form past its 96-register budget.
template <int NT, class SH, class Map>
__device__ __attribute__((noinline)) void rank_bucket(SH& sh, int nc, int kk, int tot_gt, int32_t* __restrict__ out,
                                                      const Map map) {
  using C = Cfg<NT>;
  static_assert(C::Bins >= 256 + 2 * kRankCap, "second-level ranking needs pass 1's histogram words");
  constexpr int S2 = C::Shift - 8;
  const int tid = threadIdx.x;
  uint32_t* cnt = sh.hist + C::Bins;  // per second digit: candidates
  uint32_t* start = sh.hist;          // per second digit: start of its run in the sorted list
  uint64_t* sorted = reinterpret_cast<uint64_t*>(sh.hist + 256);
  auto digit2 = [](uint64_t c) { return (uint32_t)(c >> (32 + S2)) & 255u; };
  // Each candidate's place within its digit's run comes back from its counter's atomic.
  constexpr int PER = (kRankCap + NT - 1) / NT;
  uint32_t place[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = tid + q * NT;
    if (i < nc) place[q] = atomicAdd(&cnt[digit2(sh.cand[i])], 1u);
  }
  __syncthreads();
  // Start of each digit's run: the candidates of higher digits.  Wave 0 alone: lane l
  // holds digits 255 - 4l - 3 .. 255 - 4l, read as one 16-byte word.
  if (tid < 64) {
    const uint4 c4 = reinterpret_cast<const uint4*>(cnt)[63 - tid];  // digits 252 - 4l .. 255 - 4l
    const int local = (int)(c4.x + c4.y + c4.z + c4.w);
    const int before = wave_incl_scan(local) - local;
    reinterpret_cast<uint4*>(start)[63 - tid] =
        make_uint4((uint32_t)before + c4.w + c4.z + c4.y, (uint32_t)before + c4.w + c4.z, (uint32_t)before + c4.w,
                   (uint32_t)before);
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = tid + q * NT;
    if (i < nc) {
      const uint64_t c = sh.cand[i];
      sorted[start[digit2(c)] + place[q]] = c;
    }
  }
  __syncthreads();
  for (int j = tid; j < nc; j += NT) {
    const uint64_t me = sorted[j];
    const uint32_t d = digit2(me);
    const int lo = (int)start[d], hi = lo + (int)cnt[d];
    int rank = lo;
    for (int i = lo; i < hi; ++i) rank += sorted[i] > me ? 1 : 0;
    if (rank < kk) out[tot_gt + rank] = map.token((int)~(uint32_t)me);
  }
}

// The exact path for a row whose boundary bucket holds more keys than the ranking list
// (long runs of equal values).  It re-reads the row's cells (from cache) in rolled loops
// instead of taking the caller's register keys, so it holds no per-round state and the
// common path's register allocation does not carry it.  Two more histogram passes over the keys inside digit d1 fix K*, the
// k-th largest key; then cells > K* and the first need_eq cells == K* in index order are
// output, their slots from per-(round, wave) ballot counts: cell i = e*NT + wave*64 + lane,
// so (e, wave) pairs in row-major order are index order.
template <int NT, int EPT, class Map>
__device__ __forceinline__ void topk_row_exact(const float* __restrict__ row, int n, int k,
                                                         int32_t* __restrict__ out, TopkShared<NT, EPT>* shp,
                                                         const Map map, uint32_t d1, int kk, int ne) {
  using C = Cfg<NT>;
  constexpr int NW = NT / 64;
  TopkShared<NT, EPT>& sh = *shp;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto key_at = [&](int e) { return map.key(row[min(e * NT + tid, n - 1)], e * NT + tid - n); };
  uint32_t prefix = d1 << C::Shift, pmask = ~0u << C::Shift;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? C::Shift - C::FbBitsA : 0;
    const uint32_t dmask = pass == 0 ? (1u << C::FbBitsA) - 1u : (1u << C::FbBitsB) - 1u;
    for (int i = tid; i < kFbBins; i += NT) sh.hist[i] = 0;
    __syncthreads();
#pragma unroll 1
    for (int e = 0; e < ne; ++e) {
      const uint32_t kv = key_at(e);
      if (kv != 0u && (kv & pmask) == prefix) atomicAdd(&sh.hist[(kv >> shift) & dmask], 1u);
    }
    __syncthreads();
    select_digit<NT, kFbBins>(sh, kk);
    prefix |= (uint32_t)sh.sel_digit << shift;
    pmask |= dmask << shift;
    kk -= sh.sel_above;
    __syncthreads();
  }
  const uint32_t kstar = prefix;
  const int need_eq = kk;  // how many cells equal to K* are taken (>= 1)
  constexpr int NE = EPT * NW;
#pragma unroll 1
  for (int e = 0; e < EPT; ++e) {  // kstar >= 1, so cells past n (key 0) never count
    const uint32_t kv = e < ne ? key_at(e) : 0u;
    const uint64_t bg = __ballot(kv > kstar);
    const uint64_t be = __ballot(kv == kstar);
    if (lane == 0) {
      sh.cnt_gt[e * NW + wave] = __popcll(bg);
      sh.cnt_eq[e * NW + wave] = __popcll(be);
    }
  }
  __syncthreads();
  if (wave == 0) {  // exclusive scan of both count arrays by one wave
    constexpr int PER = (NE + 63) / 64;
    int g[PER], q[PER], sg = 0, se = 0;
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const int f = lane * PER + t;
      g[t] = f < NE ? sh.cnt_gt[f] : 0;
      q[t] = f < NE ? sh.cnt_eq[f] : 0;
      sg += g[t];
      se += q[t];
    }
    int ig = wave_incl_scan(sg) - sg, ie = wave_incl_scan(se) - se;
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const int f = lane * PER + t;
      if (f < NE) {
        sh.cnt_gt[f] = ig;
        sh.cnt_eq[f] = ie;
      }
      ig += g[t];
      ie += q[t];
    }
  }
  __syncthreads();
  const uint64_t lt = lanemask_lt(lane);
#pragma unroll 1
  for (int e = 0; e < ne; ++e) {
    const uint32_t kv = key_at(e);
    const bool is_gt = kv > kstar;
    const bool is_eq = kv == kstar;
    const uint64_t bg = __ballot(is_gt);
    const uint64_t be = __ballot(is_eq);
    const int gt_before = sh.cnt_gt[e * NW + wave] + __popcll(bg & lt);
    const int eq_before = sh.cnt_eq[e * NW + wave] + __popcll(be & lt);
    const int pos = gt_before + min(eq_before, need_eq);
    if ((is_gt || (is_eq && eq_before < need_eq)) && pos < k) out[pos] = map.token(e * NT + tid);
  }
}

// Top-k of one row by one workgroup of NT threads: `row` holds n cells (n <= NT*EPT), the
// k selected token indices go to out[0..k); when the row has at most k valid cells, all
// of them are output, then -1 (DenseRow: 0..n-1).  Ties go to the earlier cell.  Every
// thread of the block calls it with the same arguments.
template <int NT, int EPT, class Map = DenseRow>
__device__ __forceinline__ void topk_row(const float* __restrict__ row, int n, int k, int32_t* __restrict__ out,
                                         TopkShared<NT, EPT>& sh, const Map map = Map()) {
  using C = Cfg<NT>;
  const int tid = threadIdx.x;
  if (n <= (Map::kCountValid ? 0 : k)) {  // uniform
    for (int i = tid; i < k; i += NT) out[i] = (i < n) ? map.token(i) : -1;
    return;
  }
  const int ne = __builtin_amdgcn_readfirstlane((n + NT - 1) / NT);  // rounds holding valid cells; <= EPT
  // Branch-free loads, all in flight together, through a buffer descriptor covering the
  // row's n valid cells: the row base and the round's offset are scalar (so a load costs
  // no vector address arithmetic), and a cell past n reads 0 (the descriptor's range
  // check) and is masked to key 0.  The histogram is cleared while the loads are in flight.
  // The phases after this skip every group of 8 rounds wholly past n (for_rounds), which
  // is most of a short row's rounds.
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), 0, n * 4, kBufferRsrcFlags);
  float raw[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    raw[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc, tid * 4, e * NT * 4, 0));
  for (int i = tid; i < C::Bins / 4 + 64; i += NT) reinterpret_cast<uint4*>(sh.hist)[i] = make_uint4(0, 0, 0, 0);
  // Keys: only the group of rounds that holds the row's end needs the per-cell length mask;
  // groups wholly inside the row take the unmasked key (a uniform branch per group keeps
  // the masks from being computed ahead for every round and held in registers).
  // Groups wholly past the row are not computed: no phase reads their keys (for_rounds
  // skips them, and the exact path re-reads the row).
  uint32_t key[EPT];
  constexpr int kGroup = EPT < 8 ? EPT : 8;
#pragma unroll
  for (int g = 0; g < EPT; g += kGroup) {
    if ((g + kGroup) * NT <= n) {
#pragma unroll
      for (int e = g; e < g + kGroup; ++e) key[e] = map.key_full(raw[e]);
    } else if (g == 0 || g * NT < n) {
#pragma unroll
      for (int e = g; e < g + kGroup; ++e) key[e] = map.key(raw[e], e * NT + tid - n);
    } else {
#pragma unroll
      for (int e = g; e < g + kGroup; ++e) key[e] = 0u;
    }
  }
  if constexpr (Map::kCountValid) {
    // At most k valid cells: all of them, in cell order, then -1.  (The scan's barrier
    // also orders the histogram clear; wave_tot is next written after pass 1's barrier.)
    int cnt = 0;
    for_rounds<EPT>(ne, [&](int e) { cnt += key[e] != 0u ? 1 : 0; });
    int total;
    int pos = block_excl_scan<NT>(cnt, sh.wave_tot, total);
    if (total <= k) {  // uniform
      for_rounds<EPT>(ne, [&](int e) {
        if (key[e] != 0u) out[pos++] = map.token(e * NT + tid);
      });
      for (int i = total + tid; i < k; i += NT) out[i] = -1;
      return;
    }
  }
  __syncthreads();

  // ---- pass 1: the top D1 bits of every valid cell ----
  // A group of rounds wholly inside a dense row holds only valid keys and adds every one
  // (no per-cell branch); other groups skip key 0.
#pragma unroll
  for (int g = 0; g < EPT; g += kGroup) {
    if (!Map::kCountValid && (g + kGroup) * NT <= n) {
#pragma unroll
      for (int e = g; e < g + kGroup; ++e) atomicAdd(&sh.hist[key[e] >> C::Shift], 1u);
    } else if (g == 0 || g * NT < n) {
#pragma unroll
      for (int e = g; e < g + kGroup; ++e)
        if (key[e] != 0u) atomicAdd(&sh.hist[key[e] >> C::Shift], 1u);
    }
  }
  __syncthreads();
  select_digit<NT, C::Bins>(sh, k);
  const uint32_t d1 = (uint32_t)sh.sel_digit;
  int kk = k - sh.sel_above;

  // ---- cells above the bucket, and the bucket itself (one block scan of two counts) ----
  // Cells past n (key 0) can only fall in the bucket when d1 == 0; they then rank below
  // every valid candidate, and the histogram (valid cells only) needs fewer than those.
  int n_gt = 0, n_in = 0;
  for_rounds<EPT>(ne, [&](int e) {
    const uint32_t dg = key[e] >> C::Shift;
    n_gt += dg > d1 ? 1 : 0;
    n_in += dg == d1 ? 1 : 0;
  });
  int tot_gt, nc, pos_gt, pos_in;
  block_excl_scan2<NT>(n_gt, n_in, sh.wave_tot, pos_gt, pos_in, tot_gt, nc);
  if (nc <= kRankCap) {
    // One pass: bucket cells to the ranking list, cells above the bucket to their output
    // slots (a workgroup barrier does not wait for global stores, and the register keys
    // are dead once it is done, before the ranking).  In a dense row every lane stores
    // every round, through a descriptor covering the slots those cells can take: a lane
    // whose cell is not above the bucket stores past it, which the hardware drops (no
    // offset overflows for any k), so the loop carries no branch on the (mostly mixed)
    // per-lane selection.  Bucket cells are few, and their branch is skipped whole by
    // most rounds.
    const int obytes = min(k, n) * 4;  // the slots of cells above the bucket lie below min(k, n)
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(out, 0, obytes, kBufferRsrcFlags);
    for_rounds<EPT>(ne, [&](int e) {
      const uint32_t dg = key[e] >> C::Shift;
      if (dg == d1) sh.cand[pos_in++] = ((uint64_t)key[e] << 32) | (uint32_t)~(e * NT + tid);
      if constexpr (Map::kCountValid) {
        if (dg > d1) out[pos_gt++] = map.token(e * NT + tid);
      } else {
        const bool above = dg > d1;
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)map.token(e * NT + tid), orsrc, above ? pos_gt * 4 : obytes,
                                              0, 0);
        pos_gt += above ? 1 : 0;
      }
    });
    __syncthreads();
    // Rank of each candidate among the bucket by (key desc, index asc); composites are
    // distinct, so the ranks are a permutation of 0..nc-1.
    rank_bucket<NT>(sh, nc, kk, tot_gt, out, map);
    return;
  }

  // ---- large bucket (long runs of equal values): the exact path ----
  topk_row_exact<NT, EPT, Map>(row, n, k, out, &sh, map, d1, kk, ne);
}

// Top-k of a row too long to keep in registers (more than 32 cells per thread: at 1024
// threads, 64 keys each spilled about 110 registers and a 65536-cell row took 43.7 us;
// re-reading the cells per pass, 25.1 us).
// The same passes in the same order as topk_row, so the same output bytes, but every pass
// over the cells re-reads them (from the cache after the first) instead of holding keys.
template <int NT, int EPT, class Map = DenseRow>
__device__ __forceinline__ void topk_row_stream(const float* __restrict__ row, int n, int k, int32_t* __restrict__ out,
                                                TopkShared<NT, EPT>& sh, const Map map = Map()) {
  using C = Cfg<NT>;
  const int tid = threadIdx.x;
  if (n <= (Map::kCountValid ? 0 : k)) {  // uniform
    for (int i = tid; i < k; i += NT) out[i] = (i < n) ? map.token(i) : -1;
    return;
  }
  const int ne = __builtin_amdgcn_readfirstlane((n + NT - 1) / NT);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), 0, n * 4, kBufferRsrcFlags);
  auto load = [&](int e) {  // a cell past n reads 0, masked to key 0 below
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc, tid * 4, e * NT * 4, 0));
  };
  auto key_of = [&](int e, float f) { return map.key(f, e * NT + tid - n); };
  for (int i = tid; i < C::Bins / 4 + 64; i += NT) reinterpret_cast<uint4*>(sh.hist)[i] = make_uint4(0, 0, 0, 0);
  if constexpr (Map::kCountValid) {
    int cnt = 0;
    stream_rounds<EPT>(load, [&](int e, float f) { cnt += key_of(e, f) != 0u ? 1 : 0; });
    int total;
    int pos = block_excl_scan<NT>(cnt, sh.wave_tot, total);
    if (total <= k) {  // uniform
      stream_rounds<EPT>(load, [&](int e, float f) {
        if (key_of(e, f) != 0u) out[pos++] = map.token(e * NT + tid);
      });
      for (int i = total + tid; i < k; i += NT) out[i] = -1;
      return;
    }
  }
  __syncthreads();
  stream_rounds<EPT>(load, [&](int e, float f) {
    const uint32_t kv = key_of(e, f);
    if (kv != 0u) atomicAdd(&sh.hist[kv >> C::Shift], 1u);
  });
  __syncthreads();
  select_digit<NT, C::Bins>(sh, k);
  const uint32_t d1 = (uint32_t)sh.sel_digit;
  int kk = k - sh.sel_above;
  int n_gt = 0, n_in = 0;
  stream_rounds<EPT>(load, [&](int e, float f) {
    const uint32_t dg = key_of(e, f) >> C::Shift;
    n_gt += dg > d1 ? 1 : 0;
    n_in += dg == d1 ? 1 : 0;
  });
  int tot_gt, nc, pos_gt, pos_in;
  block_excl_scan2<NT>(n_gt, n_in, sh.wave_tot, pos_gt, pos_in, tot_gt, nc);
  if (nc <= kRankCap) {
    stream_rounds<EPT>(load, [&](int e, float f) {
      const uint32_t kv = key_of(e, f);
      const uint32_t dg = kv >> C::Shift;
      if (dg == d1) sh.cand[pos_in++] = ((uint64_t)kv << 32) | (uint32_t)~(e * NT + tid);
      else if (dg > d1) out[pos_gt++] = map.token(e * NT + tid);
    });
    __syncthreads();
    rank_bucket<NT>(sh, nc, kk, tot_gt, out, map);
    return;
  }
  topk_row_exact<NT, EPT, Map>(row, n, k, out, &sh, map, d1, kk, ne);
}

}  // namespace idx
