// Fused decode step of the indexer on gfx950: K store of the new rows, paged MQA scorer and
// per-row top-k in one launch.  The pages run these as separate launches (K write, then the
// scorer, then the top-k: page "Dense MXFP4 indexer for DeepSeek-V4 on ROCm", Changes); at
// decode sizes each of them is mostly launch and dependency latency, so here they share one.
//
// Blocks of 16 waves; each wave scores 128 consecutive tokens of one sequence with the
// decode-form wave body (scorer.hpp).  In a block whose range holds new tokens, wave 0
// first computes their K rows (kstore_row.hpp) and stores them to their slots for later
// steps; after one barrier the wave holding a new token substitutes the fresh bytes into
// its K tile in registers, so no wave reads a row back from the pool it is written to.  Each
// block then publishes its logits (device-coherent stores) and counts itself in on the
// sequence's counter; the last block of a sequence invalidates its caches once and runs
// the top-k of the sequence's rows with all 1024 threads (topk_row.hpp), then resets the
// counter.
#include "kstore_row.hpp"
#include "scorer.hpp"
#include "topk_row.hpp"

namespace idx {
namespace {

constexpr int kStepWaves = 16;  // 1024-thread blocks: the last one runs a 1024-thread top-k
constexpr int kStepG = 2;       // 128 tokens per wave
constexpr int kStepTok = kStepWaves * 64 * kStepG;
constexpr int kStepMaxTiles = 2;  // query head tiles per sequence (register budget of 1024-thread blocks)
constexpr int kStepMaxCtx = 16 * 1024;
constexpr int kRowWords = 34;   // one K row in page layout (16 or 32 data words, scale word) + flag

// The block's new K rows.  pre(): wave 0 of a block whose token range holds new tokens
// computes those rows (before its own loads, so the fp64 work never shares registers with
// K tiles in flight), stores them to their slots and leaves their bytes in LDS.
// operator(): after every wave has issued its K loads, one barrier, then the wave holding
// a new token substitutes the row into its tile in registers.
template <int FMT>
struct NewRows {
  static constexpr bool kCoherentStores = true;
  const StepArgs* a;
  int b;
  int blk0;        // first token of the block
  int n_b;         // the sequence's length (clamped to max_ctx)
  bool any;        // block-uniform: the block holds a new token
  uint32_t (*buf)[kRowWords];  // [n_q] LDS rows; words[kRowWords - 1] = 1 when row j was stored

  __device__ __forceinline__ bool holds(int s) const { return s >= blk0 && s < blk0 + kStepTok; }

  __device__ __forceinline__ void pre(int lane) const {
    if (!any || (threadIdx.x >> 6) != 0) return;
    const int n_q = a->s.n_q;
    const int64_t P = a->s.pool.page_size;
    for (int j = 0; j < n_q; ++j) {  // uniform
      const int s = n_b - n_q + j;
      bool stored = false;
      if (s >= 0 && holds(s)) {
        const int64_t i = (int64_t)b * n_q + j;
        const int64_t slot = a->slots[i];
        const int32_t pos = a->positions[i];
        if (slot >= 0 && slot < a->s.pool.num_pages * P && pos >= 0 && pos < a->max_pos) {
          kstore_row<FMT>(a->s.pool, a->k + i * a->row_stride, a->gamma, a->eps, a->cos_sin + (int64_t)pos * 64,
                          slot, lane, buf[j]);
          stored = true;
        }
      }
      if (lane == 0) buf[j][kRowWords - 1] = stored ? 1u : 0u;
    }
  }

  template <class KT>
  __device__ __forceinline__ void operator()(KT& kt, int tok0, int, int lane) const {
    if (!any) return;
    __syncthreads();  // the rows in LDS are complete
    constexpr int T = sizeof(KT) / sizeof(kt[0]);
    const int n_q = a->s.n_q;
    for (int j = 0; j < n_q; ++j) {  // uniform
      const int s = n_b - n_q + j;
      if (s < tok0 || s >= tok0 + 16 * T || buf[j][kRowWords - 1] == 0u) continue;
      const uint32_t* w = buf[j];
      const int tt = (s - tok0) >> 4, g = lane >> 4;
      const bool mine = (lane & 15) == (s & 15);
      v8i v;
      uint32_t sc;
      if (FMT == 0) {
        v = v8i{(int)w[4 * g], (int)w[4 * g + 1], (int)w[4 * g + 2], (int)w[4 * g + 3], 0, 0, 0, 0};
        sc = (w[16] >> (8 * g)) & 0xFFu;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (int)w[8 * g + e];
        sc = w[32];
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const bool hit = mine && t == tt;
#pragma unroll
        for (int e = 0; e < 8; ++e) kt[t].v[e] = hit ? v[e] : kt[t].v[e];
        kt[t].scale = hit ? sc : kt[t].scale;
      }
    }
  }
};

template <int FMT, int NT, int EPT>
__global__ __launch_bounds__(1024) void decode_step_kernel(StepArgs a) {
  __shared__ TopkShared<1024, EPT> sh;
  __shared__ uint32_t rows[kStepMaxTiles][kRowWords];
  __shared__ int last;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int b = blockIdx.y;
  const int blk0 = blockIdx.x * kStepTok;
  const int tok0 = blk0 + wave * (64 * kStepG);
  const int n_b = uniform(min(max(a.s.ctx[b], 0), a.s.max_ctx));
  // block-uniform: the newest n_q tokens [n_b - n_q, n_b) meet [blk0, blk0 + kStepTok)
  const bool any = n_b > blk0 && n_b - a.s.n_q < blk0 + kStepTok;
  decode_wave<FMT, NT, kStepG>(a.s, b, tok0, lane, NewRows<FMT>{&a, b, blk0, n_b, any, rows});

  // Publish this block's logits and count it in.  The logits stores are device-coherent
  // (they write through to the level every XCD reads), and every wave waits until its
  // stores are complete before the barrier (a workgroup barrier alone does not wait for
  // them), so once a block's count is in, its logits are visible device-wide.  This costs
  // no L2 write-back, which a release fence per block would (measured several us here).
  // The last block invalidates its CU's and XCD's caches once (thread 0) before reading.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int done = __hip_atomic_fetch_add(&a.counters[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = done == (int)gridDim.x - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (!last) return;
  for (int j = 0; j < a.s.n_q; ++j) {
    const int64_t r = (int64_t)b * a.s.n_q + j;
    topk_row<1024, EPT>(a.s.logits + r * a.s.lstride, valid_len(n_b, a.s.n_q, j), a.k_top, a.out + r * a.k_top, sh);
    __syncthreads();  // the shared state is reused by the next row
  }
  if (threadIdx.x == 0) a.counters[b] = 0;
}

template <int FMT, int NT>
hipError_t launch_ept(const StepArgs& a, dim3 grid, int ept, hipStream_t s) {
  switch (ept) {
#define IDX_STEP_CASE(E) \
  case E: hipLaunchKernelGGL((decode_step_kernel<FMT, NT, E>), grid, dim3(1024), 0, s, a); break;
    IDX_STEP_CASE(1) IDX_STEP_CASE(2) IDX_STEP_CASE(4) IDX_STEP_CASE(8) IDX_STEP_CASE(16)
#undef IDX_STEP_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const StepArgs& a, dim3 grid, int nt, int ept, hipStream_t s) {
  switch (nt) {
    case 1: return launch_ept<FMT, 1>(a, grid, ept, s);
    case 2: return launch_ept<FMT, 2>(a, grid, ept, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_step_supported(int n_q, int H, int64_t max_ctx) {
  return n_q >= 1 && n_q * ((H + kHeadTile - 1) / kHeadTile) <= kStepMaxTiles && max_ctx <= kStepMaxCtx;
}

hipError_t launch_decode_step(const StepArgs& a, hipStream_t s, int num_cus) {
  const dim3 grid((unsigned)((a.s.max_ctx + kStepTok - 1) / kStepTok), (unsigned)a.s.B);
  if (a.s.max_ctx == 0 || (int64_t)grid.x * grid.y > num_cus) {
    // More blocks than CUs: a 1024-thread block per CU leaves the scorer short of waves
    // in flight, so the three kernels run one after another instead (same bytes, same
    // bits: the same wave bodies and row routines).  With max_ctx == 0 every row is
    // empty and only the top-k (all -1) has work.
    KStoreArgs k;
    k.pool = a.s.pool;
    k.k = a.k;
    k.n_rows = (int64_t)a.s.B * a.s.n_q;
    k.row_stride = a.row_stride;
    k.gamma = a.gamma;
    k.eps = a.eps;
    k.positions = a.positions;
    k.cos_sin = a.cos_sin;
    k.max_pos = a.max_pos;
    k.slots = a.slots;
    k.step_ctx = a.s.ctx;
    k.step_n_q = a.s.n_q;
    k.step_max_ctx = a.s.max_ctx;
    hipError_t e;
    if (a.s.max_ctx > 0) {
      if ((e = launch_k_store(k, s)) != hipSuccess) return e;
      if ((e = launch_logits(a.s, s)) != hipSuccess) return e;
    }
    TopkArgs t{a.s.logits, a.s.lstride, a.s.ctx, a.s.B, a.s.n_q, a.s.max_ctx, a.k_top, a.out};
    return launch_topk(t, s);
  }
  const int nt = a.s.n_q * ((a.s.H + kHeadTile - 1) / kHeadTile);
  int ept = 1;
  while (ept * 1024 < a.s.max_ctx) ept *= 2;
  return a.s.pool.kv_format == 0 ? launch_fmt<0>(a, grid, nt, ept, s) : launch_fmt<1>(a, grid, nt, ept, s);
}

}  // namespace idx
