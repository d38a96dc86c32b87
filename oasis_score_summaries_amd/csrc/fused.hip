// The overlapped decode step as two fused launches on gfx950 (a third when the
// attention reads the working set in HBM: the plan's block copies).
//
// The OasisKV pages split a decode step into a foreground half, attention of the
// current token over the blocks resident in HBM now, and a background half, the
// look-ahead that scores the block summaries with the draft queries, predicts the
// top-K blocks and plans the transfers for the next step (lode.cx summary, point
// 3; legiblepapers.com summary; xllm-io review, section three, training flow
// step 3).  The two halves share only inputs, so their work items can sit in
// the same grids:
//   launch 1: the scoring workgroups and the attention split workgroups (both
//             stream HBM: summaries on one side, K/V blocks on the other);
//   launch 2: the selection-and-plan workgroups and the attention merge
//             workgroups (both latency bound).
// One grid per phase needs no second stream and no cross-stream event, and the
// ramp-up and tail of each phase are paid once instead of twice (up to 96 query
// rows per KV head; see OASIS_FUSED_MAX_RT).  A workgroup's
// role follows from its index; the scoring and selection workgroups, which run
// longest, come first so that they start first.
#include "attention_impl.h"
#include "score_impl.h"
#include "select_impl.h"

namespace oasis {

static_assert(kScoreWaves == kAttnWaves, "one workgroup size for both roles");
// Row tiles up to which the scoring shares launch 1 with the attention gather.  From
// three row tiles on the scoring reads its query fragments step by step, so it fits
// four waves per SIMD at any row count, but its LDS grows by 8 KB per row tile and
// the whole grid gets the larger of the two roles' LDS: beyond six row tiles (96
// query rows) the attention would drop to two workgroups per CU, and the two
// kernels run back to back instead.  (Measured at 80 rows: 76.5 us per step fused
// against 81.2 us back to back.)
#ifndef OASIS_FUSED_MAX_RT
#define OASIS_FUSED_MAX_RT 6
#endif
// 16-row tiles of the query rows (group x queries) of one KV head.
static inline int fused_rt(const Dims& d) { return (d.group * d.queries + 15) / 16; }

template <int RT, int GP, bool POOL = false>
__global__ __launch_bounds__(64 * kAttnWaves, OASIS_ATTN_MIN_WAVES) void score_attn_kernel(ScoreArgs sa, AttnArgs aa,
                                                                             int n_score, int score_gx,
                                                                             int attn_gx, int by_xcd) {
  __shared__ union {
    ScoreShared<RT> s;
    AttnShared<GP> a;
  } sh;
  const int b = blockIdx.x;
  const int nh = n_score / score_gx;  // (sequence, KV head) pairs
  int x, head;
  if (b < n_score) {
    xcd_item(b, score_gx, nh, by_xcd, x, head);
    score_wg<RT>(x, head, sh.s, sa);
  } else {
    xcd_item(b - n_score, attn_gx, nh, by_xcd, x, head);
    attn_split_wg<GP, true, POOL>(x, head, sh.a, aa);
  }
}

// The overlapped step with its background half inside launch 1: the scoring
// workgroups, then the attention split workgroups with one selection-and-plan
// workgroup per (sequence, KV head) among them.  A selection workgroup takes its head's scores
// over from the scoring workgroups through the hand-off region `ho` (device-scope
// stores, per-wave flags, words that carry their own validity; see common.h), so the
// selection and plan run while the attention still streams K and V instead of after
// a kernel boundary.  The splits write plain records and the merge is a second,
// small launch (the kernel boundary makes the records visible).  Every selection
// workgroup comes after the scoring workgroups it waits for in the grid, and every
// wait is bounded.  Up to K = 256 and 2048 blocks per KV head (the selection in 256
// threads) and as many query rows as launch 1 fuses.  The selection's LDS, plan
// bitmaps included, shares the union with the other roles', so the grid keeps the
// occupancy of the scoring and attention roles.  With `by_xcd` (many query rows per KV
// head) a head's scoring workgroups share an XCD, whose L2 then fetches its queries once.
constexpr int kStepAttnBeforeSelect = 512;  // measured at Qwen3-8B 32K: 256-768 alike, 1024 late
template <int RT, int GP, int ITEMS, bool POOL>
__global__ __launch_bounds__(64 * kAttnWaves, OASIS_ATTN_MIN_WAVES) void step_kernel(
    ScoreArgs sa, TopkPlanArgs ta, AttnArgs aa, Handoff ho, int n_score, int score_gx, int attn_gx,
    int by_xcd) {
  __shared__ union {
    ScoreShared<RT> s;
    AttnShared<GP> a;
    struct {
      TopkPlanShared<kScoreThreads, ITEMS> t;
      PlanBitmaps bm;
    } sel;
  } sh;
  const int heads = n_score / score_gx;
  int b = blockIdx.x;
  if (b < n_score) {
    // (The placement is resolved at run time only where it can apply: at 20 query rows
    // the extra index arithmetic measured 0.2 us per step.)
    int x = b % score_gx, head = b / score_gx;
    if (RT >= 4) xcd_item(b, score_gx, heads, by_xcd, x, head);
    score_wg<RT, true, step_score_tiles(RT)>(x, head, sh.s, sa, &ho);
    return;
  }
  b -= n_score;
  // The selection workgroups follow the first kStepAttnBeforeSelect attention
  // workgroups, so that they are dispatched about when the scores they wait for are
  // done rather than holding slots while the scoring still streams.
  const int k_pre = min(kStepAttnBeforeSelect, attn_gx * heads) & ~7;
  if (b >= k_pre && b < k_pre + heads) {
    topk_plan_wg<kScoreThreads, ITEMS, true>(b - k_pre, sh.sel.t, sh.sel.bm, ta, &ho);
    return;
  }
  if (b >= k_pre) b -= heads;
  // The attention splits of a head share one XCD (its L2 fetches the head's queries
  // once); the role starts at a multiple of 8 when the head count is one.
  int x, head;
  xcd_item(b, attn_gx, heads, true, x, head);
  if (head < heads) attn_split_wg<GP, true, POOL>(x, head, sh.a, aa);
}

template <int THREADS, int ITEMS>
__global__ __launch_bounds__(THREADS) void select_merge_kernel(TopkPlanArgs ta, const float* part,
                                                               int group, int nsplit, float* out,
                                                               float* lse, int n_select) {
  __shared__ union {
    TopkPlanShared<THREADS, ITEMS> t;
    MergeShared<THREADS / 64> m;
  } sh;
  __shared__ PlanBitmaps bm;
  if ((int)blockIdx.x < n_select) {
    topk_plan_wg<THREADS, ITEMS>(blockIdx.x, sh.t, bm, ta);
  } else if (nsplit <= kMergeWaveSplits) {  // a query head per wave
    const int bhg = merge_wave_head((int)blockIdx.x - n_select, threadIdx.x >> 6, THREADS / 64, group,
                                    n_select * group);
    if (bhg >= 0) attn_merge_wave(bhg, part, group, nsplit, out, lse);
  } else {
    attn_merge_wg<THREADS / 64>(blockIdx.x - n_select, sh.m, part, group, nsplit, out, lse);
  }
}

// Layer-pipelined decode: the previous layer's selection and plan (its background
// half) ride as extra workgroups in this layer's launch 1, next to this layer's
// scoring and attention gathering; this layer's launch 2 is then the merge alone (its
// foreground output, which the next layer needs).  The selection workgroups come
// first, as they run longest, in 256 threads, so K <= 256 and at most 2048 blocks.
template <int RT, int GP, int ITEMS>
__global__ __launch_bounds__(64 * kAttnWaves, OASIS_ATTN_MIN_WAVES) void select_score_attn_kernel(
    TopkPlanArgs prev, ScoreArgs sa, AttnArgs aa, int n_sel, int n_score, int score_gx, int attn_gx,
    int by_xcd) {
  __shared__ union {
    ScoreShared<RT> s;
    AttnShared<GP> a;
    TopkPlanShared<kScoreThreads, ITEMS> t;
  } sh;
  __shared__ PlanBitmaps bm;
  const int b = blockIdx.x;
  if (b < n_sel) {
    topk_plan_wg<kScoreThreads, ITEMS>(b, sh.t, bm, prev);
    return;
  }
  const int c = b - n_sel;  // n_sel is 0 or the number of heads
  const int nh = n_score / score_gx;
  int x, head;
  if (c < n_score) {
    xcd_item(c, score_gx, nh, by_xcd, x, head);
    score_wg<RT>(x, head, sh.s, sa);
  } else {
    xcd_item(c - n_score, attn_gx, nh, by_xcd, x, head);
    attn_split_wg<GP, true>(x, head, sh.a, aa);
  }
}

static hipError_t launch_first_half(const Dims& d, const AttnSplit& s, const void* q, const void* summ,
                                    const void* k, const void* v, const int32_t* seq_lens,
                                    float* scores, const int32_t* resident, float scale, void* ws,
                                    hipStream_t stream, const WorkingSet* pool);
static hipError_t launch_second_half(const Dims& d, const AttnSplit& s, const TopkPlanArgs& sel,
                                     const void* ws, float* out, float* lse, hipStream_t stream);

// The shared launch also needs up to 4 query heads per KV head: the selection's LDS
// on top of larger attention partials would leave fewer than four workgroups per CU.
static bool pipelined_fits(const Dims& d) {
  const int rt = fused_rt(d);
  return rt <= 2 && d.group <= 4 && d.top_k <= kScoreThreads && d.max_blocks <= 8 * kScoreThreads;
}

hipError_t launch_pipelined_layer(const Dims& d, const LayerIO* cur, const LayerIO* prev, float scale,
                                  hipStream_t stream) {
  if (handoff_step_fits(d)) {
    // Each layer's launch 1 already holds its own selection and plan (the background
    // half runs under the layer's own streaming), so the previous layer has nothing
    // left to do.
    if (cur == nullptr) return hipSuccess;
    return launch_overlapped_step(d, cur->q, cur->summ, cur->k, cur->v, cur->seq_lens, cur->scores,
                                  cur->topk, cur->resident, cur->resident_next, cur->plan,
                                  cur->plan_count, cur->table, cur->table_count, scale, cur->out,
                                  cur->lse, cur->ws, stream);
  }
  const int heads = d.batch * d.heads;
  TopkPlanArgs ta{};
  if (prev != nullptr)
    ta = topk_plan_args(d, prev->scores, prev->seq_lens, prev->topk, prev->resident,
                        prev->resident_next, prev->plan, prev->plan_count, prev->table,
                        prev->table_count);
  if (cur == nullptr) {  // draining the last layer's background half
    return prev == nullptr ? hipSuccess
                           : launch_topk_plan(d, prev->scores, prev->seq_lens, prev->topk,
                                              prev->resident, prev->resident_next, prev->plan,
                                              prev->plan_count, prev->table, prev->table_count, stream);
  }
  const AttnSplit s = attn_split(d, d.table_stride);
  const ScoreArgs sa = score_args(d, cur->q, cur->summ, cur->seq_lens, cur->scores);
  const AttnArgs aa = attn_args(d, s, cur->q, cur->k, cur->v, cur->resident, nullptr, d.table_stride,
                                cur->seq_lens, scale, cur->ws);
  const int score_gx = score_grid_x(d);
  const int n_score = score_gx * heads;
  const int attn_gx = s.num_splits;
  const int rt = fused_rt(d);
  hipError_t err;
  if (pipelined_fits(d)) {
    const int n_sel = prev != nullptr ? heads : 0;
    const int grid = n_sel + n_score + attn_gx * heads;
    const int items = select_items(d, kScoreThreads);
    switch (rt * 100 + items) {
#define OASIS_SSA_CASE(RT, I)                                                                  \
  case RT * 100 + I:                                                                           \
    select_score_attn_kernel<RT, 4, I><<<dim3(grid), dim3(64 * kAttnWaves), 0, stream>>>(      \
        ta, sa, aa, n_sel, n_score, score_gx, attn_gx, place_by_xcd(d.group * d.queries));     \
    break;
#define OASIS_SSA_ROW(RT) \
  OASIS_SSA_CASE(RT, 1) OASIS_SSA_CASE(RT, 2) OASIS_SSA_CASE(RT, 4) OASIS_SSA_CASE(RT, 8)
      OASIS_SSA_ROW(1)
      OASIS_SSA_ROW(2)
#undef OASIS_SSA_ROW
#undef OASIS_SSA_CASE
      default:
        return hipErrorInvalidValue;
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
  } else {
    // Larger shapes: this layer's launch 1 as in the overlapped step, and the previous
    // layer's selection and plan (its scores are complete) with this layer's merge as
    // launch 2 -- two launches per layer, as in the overlapped step.
    if ((err = launch_first_half(d, s, cur->q, cur->summ, cur->k, cur->v, cur->seq_lens, cur->scores,
                                 cur->resident, scale, cur->ws, stream, nullptr)) != hipSuccess)
      return err;
    if (prev != nullptr) return launch_second_half(d, s, ta, cur->ws, cur->out, cur->lse, stream);
  }
  return launch_attention_merge(d, s, cur->out, cur->lse, cur->ws, stream);
}

// Launch 1 of a step: the scoring of every candidate block into `scores` and the
// attention's split partials over `resident` and the window into `ws`, in one grid
// up to OASIS_FUSED_MAX_RT row tiles, else back to back.
static hipError_t launch_first_half(const Dims& d, const AttnSplit& s, const void* q, const void* summ,
                                    const void* k, const void* v, const int32_t* seq_lens,
                                    float* scores, const int32_t* resident, float scale, void* ws,
                                    hipStream_t stream, const WorkingSet* pool) {
  const int heads = d.batch * d.heads;
  const ScoreArgs sa = score_args(d, q, summ, seq_lens, scores);
  AttnArgs aa = attn_args(d, s, q, pool ? pool->pool_k : k, pool ? pool->pool_v : v, resident,
                          nullptr, d.table_stride, seq_lens, scale, ws);
  if (pool) {
    aa.ring_k = (const char*)pool->ring_k;
    aa.ring_v = (const char*)pool->ring_v;
  }
  const int score_gx = score_grid_x(d);
  const int n_score = score_gx * heads;
  const int attn_gx = s.num_splits;
  const int grid1 = n_score + attn_gx * heads;
  const int rt = fused_rt(d);
  const int gp = d.group <= 4 ? 4 : (d.group <= 8 ? 8 : 16);
  const int xcd = place_by_xcd(d.group * d.queries);
  // Up to OASIS_FUSED_MAX_RT row tiles the scoring work shares the grid with the
  // attention's gathering; otherwise the two kernels run back to back.
  switch (rt <= OASIS_FUSED_MAX_RT ? rt * 100 + gp : 0) {
#define OASIS_SA_CASE(RT, GP)                                                                  \
  case RT * 100 + GP:                                                                          \
    if (pool)                                                                                  \
      score_attn_kernel<RT, GP, true><<<dim3(grid1), dim3(64 * kAttnWaves), 0, stream>>>(     \
          sa, aa, n_score, score_gx, attn_gx, xcd);                                            \
    else                                                                                       \
      score_attn_kernel<RT, GP><<<dim3(grid1), dim3(64 * kAttnWaves), 0, stream>>>(           \
          sa, aa, n_score, score_gx, attn_gx, xcd);                                            \
    break;
    OASIS_SA_CASE(1, 4)
    OASIS_SA_CASE(1, 8)
    OASIS_SA_CASE(1, 16)
    OASIS_SA_CASE(2, 4)
    OASIS_SA_CASE(2, 8)
    OASIS_SA_CASE(2, 16)
#if OASIS_FUSED_MAX_RT >= 6
    OASIS_SA_CASE(3, 4)
    OASIS_SA_CASE(3, 8)
    OASIS_SA_CASE(3, 16)
    OASIS_SA_CASE(4, 4)
    OASIS_SA_CASE(4, 8)
    OASIS_SA_CASE(4, 16)
    OASIS_SA_CASE(5, 4)
    OASIS_SA_CASE(5, 8)
    OASIS_SA_CASE(5, 16)
    OASIS_SA_CASE(6, 4)
    OASIS_SA_CASE(6, 8)
    OASIS_SA_CASE(6, 16)
#endif
#undef OASIS_SA_CASE
    default: {
      hipError_t e = launch_score(d, q, summ, seq_lens, scores, stream);
      if (e != hipSuccess) return e;
      if (pool)
        e = launch_attention_split_pool(d, s, q, pool->pool_k, pool->pool_v, pool->ring_k,
                                        pool->ring_v, resident, seq_lens, scale, ws, stream);
      else
        e = launch_attention_split(d, s, q, k, v, resident, nullptr, d.table_stride, seq_lens, scale,
                                   ws, stream, true);
      if (e != hipSuccess) return e;
    }
  }
  return hipGetLastError();
}

// Launch 2 of a step: the selection and plan of `sel` (any layer whose scores are
// complete) and the merge of the partials in `ws` into out, lse, in one grid.
static hipError_t launch_second_half(const Dims& d, const AttnSplit& s, const TopkPlanArgs& sel,
                                     const void* ws, float* out, float* lse, hipStream_t stream) {
  const int heads = d.batch * d.heads;
#define OASIS_SM_CASE(T, I)                                                                    \
  case I:                                                                                      \
    select_merge_kernel<T, I><<<dim3(heads + merge_workgroups(heads * d.group, s.num_splits, T / 64)), \
                                dim3(T), 0, stream>>>(sel, (const float*)ws,                   \
                                                                   d.group, s.num_splits, out, \
                                                                   lse, heads);                \
    break;
  OASIS_SELECT_DISPATCH(OASIS_SM_CASE);
#undef OASIS_SM_CASE
  return hipGetLastError();
}

// ---- the hand-off region of the workspace -------------------------------------------
// After the split records (the layout of attn_workspace_bytes): the flags (one per
// scoring wave), the status word and the score mailbox [B*H, NB].  Only
// step_kernel touches it.  Zero before the first such launch; every one leaves it
// zero.
struct HandoffLayout {
  size_t flag_score, status, mbox, total;
};
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static HandoffLayout handoff_layout(const Dims& d) {
  const size_t heads = (size_t)d.batch * d.heads;
  const size_t recs = attn_workspace_bytes(d, d.table_stride);
  const size_t score_waves = (size_t)score_grid_x(d, step_score_tiles(fused_rt(d))) * kScoreWaves;
  HandoffLayout L;
  L.flag_score = recs;
  L.status = L.flag_score + heads * score_waves * sizeof(uint32_t);
  L.mbox = align256(L.status + sizeof(uint32_t));
  L.total = align256(L.mbox + heads * d.max_blocks * sizeof(uint32_t));
  return L;
}
size_t step_workspace_bytes(const Dims& d) { return handoff_layout(d).total; }
size_t handoff_status_offset(const Dims& d) { return handoff_layout(d).status; }

// Zero-fills the hand-off region (a fill kernel rather than a memset node, so that the
// call can sit inside a captured graph).
__global__ void clear_words_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}
hipError_t launch_clear_handoff(const Dims& d, void* ws, hipStream_t stream) {
  const HandoffLayout L = handoff_layout(d);
  const size_t n = (L.total - L.flag_score) / sizeof(uint32_t);
  const size_t blocks = (n + 255) / 256;
  clear_words_kernel<<<dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream>>>(
      reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + L.flag_score), n);
  return hipGetLastError();
}

// The selection workgroups of launch 1 hold a workgroup slot each for most of the
// launch, so past a few hundred heads the selection is better off in launch 2.
// Measured per step at 20 query rows (Qwen3-8B layer shape): 64 heads 31.5 against
// 35.9 us, 128 heads 55.5 against 58.7, 256 heads 104.1 against 103.5, and 512 heads
// of 1024 blocks (36-layer shape) 152.9 against 143.7; at 80 query rows (Qwen3-235B,
// 128 heads) 63.0 against 64.4.
constexpr int kHandoffMaxHeads = 256;
bool handoff_step_fits(const Dims& d) {
  const int rt = fused_rt(d);
  return rt <= OASIS_FUSED_MAX_RT && d.top_k <= kScoreThreads && d.max_blocks <= 8 * kScoreThreads &&
         d.batch * d.heads <= kHandoffMaxHeads &&
         score_grid_x(d, step_score_tiles(rt)) * kScoreWaves <= 256 &&
         attn_split(d, d.table_stride).num_splits <= 256;
}

static hipError_t launch_one_step(const Dims& d, const AttnSplit& s, const void* q, const void* summ,
                                  const void* k, const void* v, const int32_t* seq_lens, float* scores,
                                  const int32_t* resident, const TopkPlanArgs& ta, float scale,
                                  float* out, float* lse, void* ws, hipStream_t stream,
                                  const WorkingSet* pool) {
  const int heads = d.batch * d.heads;
  const HandoffLayout L = handoff_layout(d);
  char* base = static_cast<char*>(ws);
  Handoff ho;
  ho.flag_score = reinterpret_cast<uint32_t*>(base + L.flag_score);
  ho.status = reinterpret_cast<uint32_t*>(base + L.status);
  ho.mbox = reinterpret_cast<uint32_t*>(base + L.mbox);
  ho.scores = scores;
  const int rt = fused_rt(d);
  const int score_gx = score_grid_x(d, step_score_tiles(rt));
  ho.score_waves = score_gx * kScoreWaves;
  const ScoreArgs sa = score_args(d, q, summ, seq_lens, scores);
  AttnArgs aa = attn_args(d, s, q, pool ? pool->pool_k : k, pool ? pool->pool_v : v, resident, nullptr,
                          d.table_stride, seq_lens, scale, static_cast<float*>(ws));
  if (pool) {
    aa.ring_k = (const char*)pool->ring_k;
    aa.ring_v = (const char*)pool->ring_v;
  }
  const int n_score = score_gx * heads;
  const int attn_gx = s.num_splits;
  const int grid = n_score + heads + attn_gx * heads;
  const int gp = d.group <= 4 ? 4 : (d.group <= 8 ? 8 : 16);
  const int xcd = place_by_xcd(d.group * d.queries);
  // Up to two row tiles and four query heads every selection width has its instance;
  // the other shapes take 8 scores per thread (any count up to 2048 blocks).
  const int items = (rt <= 2 && gp == 4) ? select_items(d, kScoreThreads) : 8;
  switch (((rt * 100 + gp) * 10 + items) * 2 + (pool ? 1 : 0)) {
#define OASIS_STEP_CASE(RT, GP, I, P)                                                           \
  case ((RT * 100 + GP) * 10 + I) * 2 + P:                                                      \
    step_kernel<RT, GP, I, P><<<dim3(grid), dim3(64 * kAttnWaves), 0, stream>>>(               \
        sa, ta, aa, ho, n_score, score_gx, attn_gx, xcd);                                       \
    break;
#define OASIS_STEP_G4(RT)                                                                       \
  OASIS_STEP_CASE(RT, 4, 1, 0) OASIS_STEP_CASE(RT, 4, 2, 0) OASIS_STEP_CASE(RT, 4, 4, 0)        \
  OASIS_STEP_CASE(RT, 4, 8, 0) OASIS_STEP_CASE(RT, 4, 1, 1) OASIS_STEP_CASE(RT, 4, 2, 1)        \
  OASIS_STEP_CASE(RT, 4, 4, 1) OASIS_STEP_CASE(RT, 4, 8, 1)
#define OASIS_STEP_G4_8(RT) OASIS_STEP_CASE(RT, 4, 8, 0) OASIS_STEP_CASE(RT, 4, 8, 1)
#define OASIS_STEP_G8_16(RT)                                                                    \
  OASIS_STEP_CASE(RT, 8, 8, 0) OASIS_STEP_CASE(RT, 8, 8, 1) OASIS_STEP_CASE(RT, 16, 8, 0)       \
  OASIS_STEP_CASE(RT, 16, 8, 1)
    OASIS_STEP_G4(1)
    OASIS_STEP_G8_16(1)
    OASIS_STEP_G4(2)
    OASIS_STEP_G8_16(2)
#if OASIS_FUSED_MAX_RT >= 6
    OASIS_STEP_G4_8(3)
    OASIS_STEP_G8_16(3)
    OASIS_STEP_G4_8(4)
    OASIS_STEP_G8_16(4)
    OASIS_STEP_G4_8(5)
    OASIS_STEP_G8_16(5)
    OASIS_STEP_G4_8(6)
    OASIS_STEP_G8_16(6)
#endif
#undef OASIS_STEP_G8_16
#undef OASIS_STEP_G4_8
#undef OASIS_STEP_G4
#undef OASIS_STEP_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---- the step with the attention after the plan, from the overlapped step ----------
// oasis_decode_step attends over the slot table that the plan produces.  Launch 1 of
// the overlapped step already attends over the slot table as it was, split by split,
// and the plan changes at most C slots per (sequence, KV head): only the splits that
// hold a changed slot differ from those over the updated table (the same split
// geometry, the same blocks elsewhere).  post_plan_redo_kernel redoes those splits
// over `resident_next`, one workgroup each, writing their records over the old ones;
// the merge then runs as in the overlapped step.  `per_head` workgroups per head, at
// least as many as the splits a plan can touch.
// (Merging in the same launch, with the head's last workgroup found by an arrival
// counter, needs a device-scope release and acquire around every record: measured at
// Qwen3-8B 32K, that launch took 24.5 us against 7.4 + 4.9 us for the two.)
constexpr int kPostPlanMaxSplits = 16;
template <int GP>
__global__ __launch_bounds__(64 * kAttnWaves) void post_plan_redo_kernel(AttnArgs aa, const int32_t* __restrict__ plan,
                                                                         const int32_t* __restrict__ plan_count,
                                                                         int cap, int per_head) {
  __shared__ AttnShared<GP> sh;
  const int bh = (int)blockIdx.x / per_head, i = (int)blockIdx.x % per_head;
  const int nsplit = aa.nsplit, units_per_split = kAttnWaves * aa.rounds;
  // The plan's rows (cap <= 64), one per lane, requested together with the count.
  const int lane = threadIdx.x & 63;
  int slot = -1;
  if (lane < cap) slot = plan[((size_t)bh * cap + lane) * 3];
  const int pc = plan_count[bh];
  const int rows = pc < 0 ? 0 : (pc > cap ? cap : pc);
  // The splits holding those slots, as a mask over at most 256 splits (wave-uniform).
  uint64_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
  for (int r = 0; r < rows; ++r) {
    const int t = __builtin_amdgcn_readlane(slot, r);
    if (t < 0 || t >= aa.K) continue;
    const int lo = ((t << aa.bshift) >> 4) / units_per_split;
    int hi = ((((t + 1) << aa.bshift) - 1) >> 4) / units_per_split;
    hi = hi < nsplit - 1 ? hi : nsplit - 1;
    for (int sp = lo; sp <= hi; ++sp) {
      const uint64_t bit = 1ull << (sp & 63);
      const int w = sp >> 6;
      m0 |= w == 0 ? bit : 0ull;
      m1 |= w == 1 ? bit : 0ull;
      m2 |= w == 2 ? bit : 0ull;
      m3 |= w == 3 ? bit : 0ull;
    }
  }
  const int c0 = __builtin_popcountll(m0), c1 = __builtin_popcountll(m1), c2 = __builtin_popcountll(m2);
  if (i >= c0 + c1 + c2 + __builtin_popcountll(m3)) return;
  // Split i of the mask, in ascending order.
  int k = i, base;
  uint64_t w;
  if (k < c0) {
    w = m0, base = 0;
  } else if ((k -= c0) < c1) {
    w = m1, base = 64;
  } else if ((k -= c1) < c2) {
    w = m2, base = 128;
  } else {
    k -= c2, w = m3, base = 192;
  }
  for (; k > 0; --k) w &= w - 1;
  attn_split_wg<GP, true>(base + __builtin_ctzll(w), bh, sh, aa);
}

// The most splits that one plan row's slot lies in: one, or a few for blocks of more
// than 16 tokens (a slot spans 1 << (bshift - 4) units).
static int post_plan_row_span(const Dims& d, const AttnSplit& s) {
  const int units_per_split = kAttnWaves * s.rounds;
  const int units_per_entry = d.bshift >= 4 ? 1 << (d.bshift - 4) : 1;
  return (units_per_entry + units_per_split - 2) / units_per_split + 1;
}

// The redo pays off while a plan touches at most half of a head's splits: at Qwen3-8B
// 32K (6 of 35 splits) the step takes 38.8 us against 42.3 us as four kernels; at
// Qwen3-235B 32K, whose 128 heads of 16 query heads run 5 splits of 8 rounds each, the
// redo is nearly the whole attention again (29.0 us against 30.7 us for all of it).
bool post_plan_reuse_fits(const Dims& d) {
  if (!handoff_step_fits(d)) return false;
  const AttnSplit s = attn_split(d, d.table_stride);
  const int touched = d.cap * post_plan_row_span(d, s);
  return touched <= kPostPlanMaxSplits && 2 * touched <= s.num_splits;
}

hipError_t launch_post_plan_step(const Dims& d, const void* q, const void* summ, const void* k,
                                 const void* v, const int32_t* seq_lens, float* scores, int32_t* topk,
                                 const int32_t* resident, int32_t* resident_next, int32_t* plan,
                                 int32_t* plan_count, int32_t* table, int32_t* table_count, float scale,
                                 float* out, float* lse, void* ws, hipStream_t stream) {
  if (!post_plan_reuse_fits(d) || resident_next == resident) return hipErrorInvalidValue;
  const AttnSplit s = attn_split(d, d.table_stride);
  const TopkPlanArgs ta = topk_plan_args(d, scores, seq_lens, topk, resident, resident_next, plan,
                                         plan_count, table, table_count);
  hipError_t err = launch_one_step(d, s, q, summ, k, v, seq_lens, scores, resident, ta, scale, out, lse,
                                   ws, stream, nullptr);
  if (err != hipSuccess) return err;
  const AttnArgs aa = attn_args(d, s, q, k, v, resident_next, nullptr, d.table_stride, seq_lens, scale, ws);
  // Workgroups per head: the splits that the C rows of a plan can touch, at most all.
  int per = d.cap * post_plan_row_span(d, s);
  if (per > s.num_splits) per = s.num_splits;
  const dim3 grid((unsigned)(d.batch * d.heads * per)), block(64 * kAttnWaves);
  if (per > 0) {  // (cap 0: the plan changes nothing)
    if (d.group <= 4)
      post_plan_redo_kernel<4><<<grid, block, 0, stream>>>(aa, plan, plan_count, d.cap, per);
    else if (d.group <= 8)
      post_plan_redo_kernel<8><<<grid, block, 0, stream>>>(aa, plan, plan_count, d.cap, per);
    else
      post_plan_redo_kernel<16><<<grid, block, 0, stream>>>(aa, plan, plan_count, d.cap, per);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return launch_attention_merge(d, s, out, lse, ws, stream);
}

hipError_t launch_overlapped_step(const Dims& d, const void* q, const void* summ, const void* k,
                                  const void* v, const int32_t* seq_lens, float* scores,
                                  int32_t* topk, const int32_t* resident, int32_t* resident_next,
                                  int32_t* plan, int32_t* plan_count, int32_t* table,
                                  int32_t* table_count, float scale, float* out, float* lse,
                                  void* ws, hipStream_t stream, hipEvent_t after_first,
                                  const WorkingSet* pool, bool execute_plan) {
  const AttnSplit s = attn_split(d, d.table_stride);
  if (handoff_step_fits(d)) {
    const TopkPlanArgs ta = topk_plan_args(d, scores, seq_lens, topk, resident, resident_next, plan,
                                           plan_count, table, table_count);
    hipError_t err = launch_one_step(d, s, q, summ, k, v, seq_lens, scores, resident, ta, scale, out, lse,
                                     ws, stream, pool);
    if (err != hipSuccess) return err;
    if (after_first != nullptr && (err = hipEventRecord(after_first, stream)) != hipSuccess) return err;
    if ((err = launch_attention_merge(d, s, out, lse, ws, stream)) != hipSuccess) return err;
    if (pool == nullptr || !execute_plan) return hipSuccess;
    return launch_execute_plan(d, plan, plan_count, k, v, pool->pool_k, pool->pool_v, stream);
  }
  hipError_t err = launch_first_half(d, s, q, summ, k, v, seq_lens, scores, resident, scale, ws, stream,
                                     pool);
  if (err != hipSuccess) return err;
  if (after_first != nullptr && (err = hipEventRecord(after_first, stream)) != hipSuccess) return err;
  const TopkPlanArgs ta = topk_plan_args(d, scores, seq_lens, topk, resident, resident_next, plan,
                                         plan_count, table, table_count);
  hipError_t err2 = launch_second_half(d, s, ta, ws, out, lse, stream);
  if (err2 != hipSuccess || pool == nullptr || !execute_plan) return err2;
  // The attention has read the pool (launch 1), so the admitted blocks can take
  // their slots now.
  return launch_execute_plan(d, plan, plan_count, k, v, pool->pool_k, pool->pool_v, stream);
}

}  // namespace oasis
