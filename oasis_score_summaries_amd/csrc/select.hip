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
// One workgroup per (sequence, KV head).  Selection is an exact radix select
// over order-preserving 32-bit keys (four 8-bit digit passes with an LDS
// histogram), then the lowest-index ties of the threshold key, then a rank
// sort of the K winners in LDS.  The plan uses LDS bitmaps for set membership
// and workgroup prefix sums for every compaction, so every output position is
// a pure function of the inputs (no atomics decide an order).
#include "common.h"
#include "launch.h"

namespace oasis {

constexpr int kSelectThreads = 1024;

struct TopkShared {
  uint32_t hist[256];
  int scan[kSelectThreads / 64 + 1];
  uint32_t cand_key[kMaxTopK];
  int cand_idx[kMaxTopK];
  int sorted_idx[kMaxTopK];
  uint32_t digit;
  int above;
};

struct PlanShared {
  uint32_t bm_sel[kMaxBlocks / 32];
  uint32_t bm_res[kMaxBlocks / 32];
  float st_score[kMaxTopK];
  int st_blk[kMaxTopK];
  int adm_list[kMaxTopK];
  int adm_sorted[kMaxTopK];
  int scan[kSelectThreads / 64 + 1];
};

// Selects the min(K, n_cand) best of row[0 .. n_cand) into sh.sorted_idx, best
// first; returns that count.  Thread t owns elements [t*ITEMS, (t+1)*ITEMS), so
// thread order is index order for the tie scans.  Every thread must call it.
template <int ITEMS>
__device__ int topk_select(const float* __restrict__ row, int n_cand, int K, TopkShared& sh) {
  const int tid = threadIdx.x;
  const int m = n_cand < K ? n_cand : K;
  if (m <= 0) return 0;  // uniform across the workgroup
  uint32_t key[ITEMS];
  const int base = tid * ITEMS;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int e = base + i;
    key[i] = (e < n_cand) ? order_key(row[e]) : 0u;
  }

  uint32_t prefix = 0u, mask = 0u;
  int krem = m;  // how many of the elements matching `prefix` are still to be taken
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += blockDim.x) sh.hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      if (base + i < n_cand && (key[i] & mask) == prefix) atomicAdd(&sh.hist[(key[i] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // Lane l owns digits 255-4l .. 252-4l, i.e. the histogram read from the top.
      int c[4];
      int local = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        c[u] = (int)sh.hist[255 - 4 * tid - u];
        local += c[u];
      }
      int run = wave_inclusive_scan(local) - local;  // elements in larger digits
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (run < krem && krem <= run + c[u]) {
          sh.digit = (uint32_t)(255 - 4 * tid - u);
          sh.above = run;
        }
        run += c[u];
      }
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    mask |= 0xffu << shift;
    krem -= sh.above;
    __syncthreads();
  }

  // Threshold key `prefix`: every larger key is taken, plus the krem lowest-
  // index elements equal to it.
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    if (base + i < n_cand) {
      n_gt += key[i] > prefix;
      n_eq += key[i] == prefix;
    }
  }
  int tot_gt, tot_eq;
  int off_gt = block_exclusive_scan(n_gt, sh.scan, &tot_gt);
  int off_eq = block_exclusive_scan(n_eq, sh.scan, &tot_eq);
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int e = base + i;
    if (e >= n_cand) continue;
    if (key[i] > prefix) {
      sh.cand_key[off_gt] = key[i];
      sh.cand_idx[off_gt] = e;
      ++off_gt;
    } else if (key[i] == prefix) {
      if (off_eq < krem) {
        sh.cand_key[tot_gt + off_eq] = key[i];
        sh.cand_idx[tot_gt + off_eq] = e;
      }
      ++off_eq;
    }
  }
  __syncthreads();
  // Rank sort of the m winners: all keys differ in (key, -index).
  for (int t = tid; t < m; t += blockDim.x) {
    const uint32_t kt = sh.cand_key[t];
    const int it = sh.cand_idx[t];
    int rank = 0;
    for (int u = 0; u < m; ++u) {
      const uint32_t ku = sh.cand_key[u];
      rank += (ku > kt) || (ku == kt && sh.cand_idx[u] < it);
    }
    sh.sorted_idx[rank] = it;
  }
  __syncthreads();
  return m;
}

// Applies the capped-eviction rule for one (sequence, KV head).  `sel` holds the
// K selection entries (-1 = none), best first.  Every thread must call it, with
// blockDim.x >= K.
__device__ void plan_apply(const float* __restrict__ srow, const int* sel, const int32_t* res,
                           int32_t* res_next, int32_t* plan_row, int32_t* plan_count,
                           int32_t* table_row, int32_t* table_count, int K, int C, int NB, int w0,
                           int nblk, int T, PlanShared& sh) {
  const int tid = threadIdx.x;
  const int nwords = (NB + 31) >> 5;
  for (int w = tid; w < nwords; w += blockDim.x) {
    sh.bm_sel[w] = 0u;
    sh.bm_res[w] = 0u;
  }
  __syncthreads();
  int s_i = -1, r_i = -1;
  if (tid < K) {
    s_i = sel[tid];
    r_i = res[tid];
  }
  const bool s_ok = s_i >= 0 && s_i < NB;
  const bool r_ok = r_i >= 0 && r_i < NB;
  if (s_ok) atomicOr(&sh.bm_sel[s_i >> 5], 1u << (s_i & 31));
  if (r_ok) atomicOr(&sh.bm_res[r_i >> 5], 1u << (r_i & 31));
  __syncthreads();

  // Admission: selected, not resident, in selection order; the first n are admitted.
  const int is_new = (s_ok && !((sh.bm_res[s_i >> 5] >> (s_i & 31)) & 1u)) ? 1 : 0;
  int n_new;
  const int pos_new = block_exclusive_scan(is_new, sh.scan, &n_new);
  const int n = C < n_new ? C : n_new;
  const bool admitted = is_new && pos_new < n;

  // Victims: empty slots by slot, then stale slots by (score asc, block desc).
  const bool empty = tid < K && r_i < 0;
  const bool stale = tid < K && r_i >= 0 && !(r_ok && ((sh.bm_sel[r_i >> 5] >> (r_i & 31)) & 1u));
  int n_empty;
  const int pos_empty = block_exclusive_scan(empty ? 1 : 0, sh.scan, &n_empty);
  const float sc = stale ? (r_ok ? srow[r_i] : -INFINITY) : 0.f;
  if (tid < K) {
    sh.st_score[tid] = sc;
    sh.st_blk[tid] = stale ? r_i : -1;
  }
  if (admitted) sh.adm_list[pos_new] = s_i;
  __syncthreads();
  bool victim = false;
  if (empty) {
    victim = pos_empty < n;
  } else if (stale) {
    const int m_stale = n - n_empty;
    if (m_stale > 0) {
      int rank = 0;
      for (int u = 0; u < K; ++u) {
        const int bu = sh.st_blk[u];
        if (bu < 0) continue;
        const float su = sh.st_score[u];
        rank += (su < sc) || (su == sc && bu > r_i);
      }
      victim = rank < m_stale;
    }
  }
  if (admitted) {
    int rank = 0;
    for (int u = 0; u < n; ++u) rank += sh.adm_list[u] < s_i;
    sh.adm_sorted[rank] = s_i;
  }
  int n_vict;
  const int pos_vict = block_exclusive_scan(victim ? 1 : 0, sh.scan, &n_vict);  // syncs
  const int n_placed = n < n_vict ? n : n_vict;

  int new_r = r_i;
  if (victim && pos_vict < n_placed) {
    new_r = sh.adm_sorted[pos_vict];
    plan_row[3 * pos_vict + 0] = tid;
    plan_row[3 * pos_vict + 1] = new_r;
    plan_row[3 * pos_vict + 2] = r_i;
  }
  // Every slot is written so that res_next may be a different buffer; when it
  // is `res` itself, each thread rewrites only the slot it read above.
  if (tid < K) res_next[tid] = new_r;
  for (int r = n_placed + tid; r < C; r += blockDim.x) {
    plan_row[3 * r + 0] = -1;
    plan_row[3 * r + 1] = -1;
    plan_row[3 * r + 2] = -1;
  }
  if (tid == 0) *plan_count = n_placed;

  // Table: updated resident entries in slot order, then the window blocks.
  const bool keep = tid < K && new_r >= 0 && new_r < NB;
  int n_res;
  const int pos_t = block_exclusive_scan(keep ? 1 : 0, sh.scan, &n_res);
  if (keep) table_row[pos_t] = new_r;
  const int nwin = nblk - w0;
  for (int i = tid; i < nwin; i += blockDim.x) table_row[n_res + i] = w0 + i;
  for (int i = n_res + nwin + tid; i < T; i += blockDim.x) table_row[i] = -1;
  if (tid == 0) *table_count = n_res + nwin;
}

template <int ITEMS>
__global__ __launch_bounds__(kSelectThreads) void topk_kernel(const float* __restrict__ scores,
                                                              const int32_t* __restrict__ seq_lens,
                                                              int32_t* __restrict__ topk, int heads,
                                                              int NB, int K, int window) {
  __shared__ TopkShared sh;
  const int bh = blockIdx.x;
  const int len = clamp_len(seq_lens[bh / heads], NB);
  const int n_cand = first_window_block(len, window);
  const int m = topk_select<ITEMS>(scores + (size_t)bh * NB, n_cand, K, sh);
  for (int t = threadIdx.x; t < K; t += blockDim.x) topk[(size_t)bh * K + t] = t < m ? sh.sorted_idx[t] : -1;
}

__global__ __launch_bounds__(kSelectThreads) void plan_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ topk,
    const int32_t* __restrict__ seq_lens, int32_t* resident, int32_t* plan, int32_t* plan_count,
    int32_t* table, int32_t* table_count, int heads, int NB, int K, int C, int window, int T) {
  __shared__ PlanShared sh;
  const int bh = blockIdx.x;
  const int len = clamp_len(seq_lens[bh / heads], NB);
  plan_apply(scores + (size_t)bh * NB, topk + (size_t)bh * K, resident + (size_t)bh * K,
             resident + (size_t)bh * K, plan + (size_t)bh * C * 3, plan_count + bh,
             table + (size_t)bh * T, table_count + bh, K, C, NB, first_window_block(len, window),
             num_blocks(len), T, sh);
}

template <int ITEMS>
__global__ __launch_bounds__(kSelectThreads) void topk_plan_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int32_t* topk,
    const int32_t* resident, int32_t* resident_next, int32_t* plan, int32_t* plan_count,
    int32_t* table, int32_t* table_count, int heads, int NB, int K, int C, int window, int T) {
  __shared__ TopkShared tsh;
  __shared__ PlanShared psh;
  const int bh = blockIdx.x;
  const int len = clamp_len(seq_lens[bh / heads], NB);
  const int n_cand = first_window_block(len, window);
  const float* srow = scores + (size_t)bh * NB;
  const int m = topk_select<ITEMS>(srow, n_cand, K, tsh);
  for (int t = threadIdx.x; t < K; t += blockDim.x) {
    const int v = t < m ? tsh.sorted_idx[t] : -1;
    tsh.sorted_idx[t] = v;
    topk[(size_t)bh * K + t] = v;
  }
  __syncthreads();
  plan_apply(srow, tsh.sorted_idx, resident + (size_t)bh * K, resident_next + (size_t)bh * K,
             plan + (size_t)bh * C * 3, plan_count + bh, table + (size_t)bh * T, table_count + bh,
             K, C, NB, n_cand, num_blocks(len), T, psh);
}

static int items_for(int NB) {
  int items = 1;
  while (items * kSelectThreads < NB) items <<= 1;
  return items;
}

hipError_t launch_topk(const Dims& d, const float* scores, const int32_t* seq_lens, int32_t* topk,
                       hipStream_t stream) {
  const dim3 grid(d.batch * d.heads), block(kSelectThreads);
  switch (items_for(d.max_blocks)) {
#define OASIS_TOPK_CASE(I)                                                                        \
  case I:                                                                                         \
    topk_kernel<I><<<grid, block, 0, stream>>>(scores, seq_lens, topk, d.heads, d.max_blocks,     \
                                               d.top_k, d.window);                                \
    break;
    OASIS_TOPK_CASE(1)
    OASIS_TOPK_CASE(2)
    OASIS_TOPK_CASE(4)
    OASIS_TOPK_CASE(8)
    OASIS_TOPK_CASE(16)
    OASIS_TOPK_CASE(32)
#undef OASIS_TOPK_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_plan(const Dims& d, const float* scores, const int32_t* topk,
                       const int32_t* seq_lens, int32_t* resident, int32_t* plan,
                       int32_t* plan_count, int32_t* table, int32_t* table_count,
                       hipStream_t stream) {
  const int threads = ((d.top_k + 63) / 64) * 64;
  plan_kernel<<<dim3(d.batch * d.heads), dim3(threads), 0, stream>>>(
      scores, topk, seq_lens, resident, plan, plan_count, table, table_count, d.heads,
      d.max_blocks, d.top_k, d.cap, d.window, d.table_stride);
  return hipGetLastError();
}

hipError_t launch_topk_plan(const Dims& d, const float* scores, const int32_t* seq_lens,
                            int32_t* topk, const int32_t* resident, int32_t* resident_next,
                            int32_t* plan, int32_t* plan_count, int32_t* table,
                            int32_t* table_count, hipStream_t stream) {
  const dim3 grid(d.batch * d.heads), block(kSelectThreads);
  switch (items_for(d.max_blocks)) {
#define OASIS_TP_CASE(I)                                                                          \
  case I:                                                                                         \
    topk_plan_kernel<I><<<grid, block, 0, stream>>>(scores, seq_lens, topk, resident,             \
                                                    resident_next, plan, plan_count, table,       \
                                                    table_count, d.heads, d.max_blocks, d.top_k,  \
                                                    d.cap, d.window, d.table_stride);             \
    break;
    OASIS_TP_CASE(1)
    OASIS_TP_CASE(2)
    OASIS_TP_CASE(4)
    OASIS_TP_CASE(8)
    OASIS_TP_CASE(16)
    OASIS_TP_CASE(32)
#undef OASIS_TP_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace oasis
