// Fused decode step of the indexer on gfx950: K store of the new rows, paged MQA scorer and
// per-row top-k in one launch.  The pages run these as separate launches (K write, then the
// scorer, then the top-k: page "Dense MXFP4 indexer for DeepSeek-V4 on ROCm", Changes); at
// decode sizes each of them is mostly launch and dependency latency, so here they share one.
//
// Blocks of 16 waves; each wave scores 128 consecutive tokens of one sequence with the
// decode-form wave body (scorer.hpp).  For each of the step's new tokens in a block, the
// wave holding the token leaves its logit out, and wave 0 — after its own scoring —
// computes the token's K row (kstore_row.hpp), stores it to its slot for later steps and
// scores the token from the fresh row in registers; nothing reads a row back from the
// pool it is written to, and no wave waits for the K store.  Each
// block then publishes its logits (device-coherent stores) and counts itself in on the
// sequence's counter; the last block of a sequence invalidates its caches once and runs
// the top-k of the sequence's rows with all 1024 threads (topk_row.hpp), then resets the
// counter.  When B is a multiple of the XCD count, the blocks of one sequence run on one
// XCD, so its query tiles are fetched into one L2 and its last block finds its siblings'
// logits nearer (fused step 15.9 -> 15.6 us at decode B64/H32/8K).
#include "kstore_row.hpp"
#include "scorer.hpp"
#include "topk_row.hpp"

namespace idx {
namespace {

constexpr int kStepWaves = 16;  // 1024-thread blocks: the last one runs a 1024-thread top-k
constexpr int kStepG = 2;       // 128 tokens per wave
constexpr int kStepTok = kStepWaves * 64 * kStepG;
// Query head tiles per sequence the fused kernel takes: within the register budget of
// 1024-thread blocks (128 VGPRs).  Four tiles fit MXFP4 with a few spills but ran the step
// 1.5x slower than the three kernels (64 heads, B16/8K), so wider shapes take those.
constexpr int kStepMaxTiles = 2;
constexpr int kStepMaxCtx = 16 * 1024;
constexpr int kRowWords = 33;   // one K row in page layout: 16 (or 32) data words, then the scale word

__host__ __device__ __forceinline__ int step_chunks(int max_ctx) { return (max_ctx + kStepTok - 1) / kStepTok; }

// The step's new K rows.  prepare(): every wave of the block learns which of the newest
// n_q tokens fall in the block and have a row to store (valid slot and position); the
// wave holding such a token skips its logit.  Wave 0 — the first to have its K bytes, so
// the first to finish scoring — then computes each such row after its own work (its K
// tiles are no longer live, so the fp64 work has registers to spare), stores it to its
// slot, leaves it in its LDS buffer, and rescores the token from it.
template <int FMT, int NQ>  // NQ >= n_q (the launch's head-tile count bounds it)
struct NewRows {
  static constexpr bool kCoherentStores = true;
  static constexpr bool kNewRows = true;
  const StepArgs* a;
  int b;
  int blk0;        // first token of the block
  bool wave0;
  uint32_t* buf;   // wave 0's LDS row buffer (kRowWords words)
  int s_new[NQ];  // new tokens of the block with a row to store, else -1

  __device__ __forceinline__ void prepare(int n_b) {
    const int n_q = a->s.n_q;
#pragma unroll
    for (int jn = 0; jn < NQ; ++jn) {
      s_new[jn] = -1;
      if (jn >= n_q) continue;
      const int s = n_b - n_q + jn;
      if (s < 0 || s < blk0 || s >= blk0 + kStepTok) continue;
      const int64_t i = (int64_t)b * n_q + jn;
      const int64_t slot = a->slots[i];
      const int32_t pos = a->positions[i];
      if (slot < 0 || slot >= a->s.pool.num_pages * (int64_t)a->s.pool.page_size || pos < 0 || pos >= a->max_pos)
        continue;
      s_new[jn] = s;
    }
  }

  __device__ __forceinline__ bool skip(int s) const {
    bool k = false;
#pragma unroll
    for (int jn = 0; jn < NQ; ++jn) k = k || s == s_new[jn];
    return k;
  }

  __device__ __forceinline__ bool rescorer() const { return wave0; }

  template <int F>
  __device__ __forceinline__ bool new_row(int jn, int lane, KTile<F>& nk, int& s, int& slot4) const {
    if (jn >= NQ || s_new[jn] < 0) return false;
    s = s_new[jn];
    const int64_t i = (int64_t)b * a->s.n_q + jn;
    const int32_t pos = a->positions[i];
    kstore_row<F>(a->s.pool, a->k + i * a->row_stride, a->gamma, a->eps, a->cos_sin + (int64_t)pos * 64,
                  a->slots[i], lane, buf);
    __builtin_amdgcn_wave_barrier();  // the row words are written by a few lanes, read by all
    const int g = lane >> 4;
    if (F == 0) {
      nk.v = v8i{(int)buf[4 * g], (int)buf[4 * g + 1], (int)buf[4 * g + 2], (int)buf[4 * g + 3], 0, 0, 0, 0};
      nk.scale = (buf[16] >> (8 * g)) & 0xFFu;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) nk.v[e] = (int)buf[(e < 4 ? 0 : 12) + 4 * g + e];  // dims 16g.., 64+16g..
      nk.scale = buf[32];
    }
    __builtin_amdgcn_wave_barrier();  // the buffer is reused by the next new row
    slot4 = ((s - blk0) >> 4) & 3;    // the token's tile slot within its own wave's group
    return true;
  }
};

template <int FMT, int NT, int EPT>
__global__ __launch_bounds__(1024) void decode_step_kernel(StepArgs a) {
  __shared__ TopkShared<1024, EPT> sh;
  __shared__ uint32_t row_buf[kRowWords];
  __shared__ int last;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  // Linear block ids are dispatched round-robin over the XCDs, each with its own L2.  When
  // B is a multiple of their count, sequence b takes C slots of XCD b % kXcds (its query
  // tiles fetched into one L2, its logits written and re-read in one place); otherwise the
  // blocks go in sequence order, as an uneven split would leave XCDs short of work.
  const int C = step_chunks(a.s.max_ctx);
  int b, blk0;
  if (a.s.B % kXcds == 0) {
    const int x = (int)blockIdx.x & (kXcds - 1), slot = (int)blockIdx.x / kXcds;
    b = (slot / C) * kXcds + x;
    blk0 = (slot % C) * kStepTok;
  } else {
    b = (int)blockIdx.x / C;
    blk0 = ((int)blockIdx.x % C) * kStepTok;
  }
  if (b >= a.s.B) return;
  const int tok0 = blk0 + wave * (64 * kStepG);
  NewRows<FMT, NT> nr{&a, b, blk0, wave == 0, row_buf, {}};
  decode_wave<FMT, NT, kStepG>(a.s, b, tok0, lane, nr);

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
    last = done == C - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (!last) return;
  const int n_b = min(max(a.s.ctx[b], 0), a.s.max_ctx);
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
  return n_q >= 1 && logits_uses_decode_kernel(n_q, H) && max_ctx <= kTopkMaxCtx;
}

bool decode_step_fuses(int B, int n_q, int H, int max_ctx, int num_cus) {
  const int64_t blocks = (int64_t)step_chunks(max_ctx) * B;
  const int nt = n_q * ((H + kHeadTile - 1) / kHeadTile);
  return max_ctx > 0 && blocks <= num_cus && nt <= kStepMaxTiles && max_ctx <= kStepMaxCtx;
}

hipError_t launch_decode_step(const StepArgs& a, hipStream_t s, int num_cus) {
  const dim3 grid((unsigned)((int64_t)a.s.B * step_chunks(a.s.max_ctx)));
  const int nt = a.s.n_q * ((a.s.H + kHeadTile - 1) / kHeadTile);
  if (!decode_step_fuses(a.s.B, a.s.n_q, a.s.H, a.s.max_ctx, num_cus)) {
    // More blocks than CUs (a 1024-thread block per CU leaves the scorer short of waves in
    // flight), more query head tiles than the fused kernel holds, or rows longer than its
    // top-k takes: the three kernels run one after another instead (same bytes, same
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
      if ((e = launch_logits(a.s, s, num_cus)) != hipSuccess) return e;
    }
    TopkArgs t{a.s.logits, a.s.lstride, a.s.ctx, a.s.B, a.s.n_q, a.s.max_ctx, a.k_top, a.out};
    return launch_topk(t, s);
  }
  int ept = 1;
  while (ept * 1024 < a.s.max_ctx) ept *= 2;
  return a.s.pool.kv_format == 0 ? launch_fmt<0>(a, grid, nt, ept, s) : launch_fmt<1>(a, grid, nt, ept, s);
}

}  // namespace idx
