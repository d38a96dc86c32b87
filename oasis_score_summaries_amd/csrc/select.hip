// Head-wise top-K block selection and the capped-eviction transfer plan on gfx950.
//
// Selection: the K best candidate blocks of each KV head (xllm-io review of
// OasisKV, section three, component table: top-K = 128 blocks per head;
// section six: block size 16).  Order: higher fp32 score first, equal scores
// lower block index first.
//
// Plan: the selection is compared with the resident set and at most
// C = floor(fetch_ratio * K) new blocks per head are admitted (xllm-io review,
// section three, training flow step 3 and component table, Capped Eviction
// Policy; legiblepapers.com FAQ Q7).  Only the head-wise slot entries change
// (xllm-io review, section four, Head-wise Mapping).  The pages leave the
// admission order, the victim order and the slot pairing open; this library
// admits the best new blocks, frees empty slots first and then the stale
// slots with the lowest scores (equal scores: higher block index first), and
// pairs freed slots in slot order with admitted blocks in block order.
//
// One workgroup per (sequence, KV head); the work is latency bound, so the
// design minimises dependent steps and barriers:
//   * scores sit in registers, element e = i * THREADS + tid (coalesced loads);
//   * exact radix select over order-preserving 32-bit keys, starting below the
//     bits that all keys share (found with two DPP wave reductions), 8 bits per
//     pass, per-wave LDS histograms (no cross-wave atomic contention), a DPP
//     prefix sum over the 256 digits, and an early exit once the threshold
//     digit holds exactly the keys still needed;
//   * fast path: when the first pass's threshold digit holds few keys, the keys at
//     or above it are dropped into per-digit buckets and ranked inside their bucket
//     only, which yields the sorted selection at once;
//   * otherwise the ties of the threshold key are taken in index order with ballot
//     ranks and the K winners are rank-sorted in LDS;
//   * the plan uses LDS bitmaps for set membership and ballot ranks for every
//     compaction, so every output position is a pure function of the inputs.
#include "select_impl.h"

namespace oasis {

template <int THREADS, int ITEMS>
__global__ __launch_bounds__(THREADS) void topk_kernel(const float* __restrict__ scores,
                                                       const int32_t* __restrict__ seq_lens,
                                                       int32_t* __restrict__ topk, int heads, int NB,
                                                       int K, int window, int bshift) {
  __shared__ SelectShared<THREADS, ITEMS> sh;
  const int bh = blockIdx.x;
  const int len = clamp_len(seq_lens[bh / heads], NB, bshift);
  const int n_cand = first_window_block(len, window, bshift);
  const int m = topk_select<THREADS, ITEMS>(scores + (size_t)bh * NB, n_cand, K, sh, NB);
  for (int t = threadIdx.x; t < K; t += THREADS) topk[(size_t)bh * K + t] = t < m ? sh.sorted_idx[t] : -1;
}

template <int THREADS>
__global__ __launch_bounds__(THREADS) void plan_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ topk,
    const int32_t* __restrict__ seq_lens, int32_t* resident, int32_t* plan, int32_t* plan_count,
    int32_t* table, int32_t* table_count, int heads, int NB, int K, int C, int window, int T,
    int bshift) {
  __shared__ PlanShared<THREADS> sh;
  __shared__ PlanBitmaps bm;
  const int bh = blockIdx.x;
  const int len = clamp_len(seq_lens[bh / heads], NB, bshift);
  const int s_i = threadIdx.x < K ? topk[(size_t)bh * K + threadIdx.x] : -1;
  const ResidentSlot rs = load_resident_slot(resident + (size_t)bh * K, scores + (size_t)bh * NB, K, NB);
  clear_bitmaps(bm, NB);
  __syncthreads();
  plan_apply<THREADS>(s_i, rs, resident + (size_t)bh * K, plan + (size_t)bh * C * 3,
                      plan_count + bh, table + (size_t)bh * T, table_count + bh, K, C, NB,
                      first_window_block(len, window, bshift), num_blocks(len, bshift), T, bm, sh);
}

template <int THREADS, int ITEMS>
__global__ __launch_bounds__(THREADS) void topk_plan_kernel(TopkPlanArgs a) {
  __shared__ TopkPlanShared<THREADS, ITEMS> sh;
  __shared__ PlanBitmaps bm;
  topk_plan_wg<THREADS, ITEMS>(blockIdx.x, sh, bm, a);
}

hipError_t launch_topk(const Dims& d, const float* scores, const int32_t* seq_lens, int32_t* topk,
                       hipStream_t stream) {
#define OASIS_TOPK_CASE(T, I)                                                                       \
  case I:                                                                                           \
    topk_kernel<T, I><<<dim3(d.batch * d.heads), dim3(T), 0, stream>>>(scores, seq_lens, topk,      \
                                                                       d.heads, d.max_blocks,       \
                                                                       d.top_k, d.window, d.bshift); \
    break;
  OASIS_SELECT_DISPATCH(OASIS_TOPK_CASE);
#undef OASIS_TOPK_CASE
  return hipGetLastError();
}

hipError_t launch_plan(const Dims& d, const float* scores, const int32_t* topk,
                       const int32_t* seq_lens, int32_t* resident, int32_t* plan,
                       int32_t* plan_count, int32_t* table, int32_t* table_count,
                       hipStream_t stream) {
  if (d.top_k <= 256) {
    plan_kernel<256><<<dim3(d.batch * d.heads), dim3(256), 0, stream>>>(
        scores, topk, seq_lens, resident, plan, plan_count, table, table_count, d.heads,
        d.max_blocks, d.top_k, d.cap, d.window, d.table_stride, d.bshift);
  } else {
    plan_kernel<1024><<<dim3(d.batch * d.heads), dim3(1024), 0, stream>>>(
        scores, topk, seq_lens, resident, plan, plan_count, table, table_count, d.heads,
        d.max_blocks, d.top_k, d.cap, d.window, d.table_stride, d.bshift);
  }
  return hipGetLastError();
}

hipError_t launch_topk_plan(const Dims& d, const float* scores, const int32_t* seq_lens,
                            int32_t* topk, const int32_t* resident, int32_t* resident_next,
                            int32_t* plan, int32_t* plan_count, int32_t* table,
                            int32_t* table_count, hipStream_t stream) {
  const TopkPlanArgs a = topk_plan_args(d, scores, seq_lens, topk, resident, resident_next, plan,
                                        plan_count, table, table_count);
#define OASIS_TP_CASE(T, I)                                                        \
  case I:                                                                          \
    topk_plan_kernel<T, I><<<dim3(d.batch * d.heads), dim3(T), 0, stream>>>(a);    \
    break;
  OASIS_SELECT_DISPATCH(OASIS_TP_CASE);
#undef OASIS_TP_CASE
  return hipGetLastError();
}

}  // namespace oasis
