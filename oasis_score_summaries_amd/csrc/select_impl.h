// Device-side building blocks of the head-wise top-K selection and the capped
// plan (one workgroup per (sequence, KV head)), shared by the selection kernels
// and the fused kernel of the overlapped step.  Internal to liboasis; the design
// notes are in select.hip.
#pragma once

#include "common.h"
#include "launch.h"

namespace oasis {

// Bucket-placement fast path: taken when the threshold digit of the first radix
// pass holds at most this many keys.
constexpr int kBucketMax = 256;

template <int THREADS, int ITEMS>
struct SelectShared {
  static constexpr int NW = THREADS / 64;
  uint32_t hist[2][NW][256];
  int scan[2][NW];
  uint32_t rmax[NW], rmin[NW];
  int start[256];                           // keys with a larger first-pass digit
  int fill[256];                            // per-digit placement counters
  int cnt[ITEMS * NW];          // packed (> threshold) << 16 | (== threshold) counts per (item, wave)
  // The fast path uses `bucket` (+32: reads past a bucket's end stay inside), the
  // radix path `cand`: (key << 32) | ~index, larger is better, all distinct.
  union {
    alignas(16) uint64_t bucket[kMaxTopK + kBucketMax + 32];
    alignas(16) uint64_t cand[kMaxTopK + 32];
  };
  int sorted_idx[kMaxTopK];
  uint32_t sel_digit;
  int sel_above, sel_count, n_gt;
};

// Set-membership bitmaps of the plan (bit j of word j / 32: block j is selected /
// resident).  Kept outside the selection's LDS so that they can be cleared while the
// selection runs.
struct PlanBitmaps {
  uint32_t sel[kMaxBlocks / 32];
  uint32_t res[kMaxBlocks / 32];
  // Per-wave counts of the plan's compactions (up to 16 waves).  Outside the LDS the
  // plan shares with the selection, so the plan can write them before its first
  // barrier while other waves still read the selection's output.
  int w_new[16], w_empty[16], w_stale[16], w_vict[16], w_tab[16];
};
__device__ inline void clear_bitmaps(PlanBitmaps& bm, int NB) {
  for (int w = threadIdx.x; w < (NB + 31) >> 5; w += blockDim.x) {
    bm.sel[w] = 0u;
    bm.res[w] = 0u;
  }
}

template <int THREADS>
struct PlanShared {
  static constexpr int NW = THREADS / 64;
  alignas(16) uint64_t st[THREADS + 32];  // stale slots, compacted: (order_key(score) << 32) | ~block
  alignas(16) int adm_list[THREADS + 16];
  int adm_sorted[THREADS];
};

// Inclusive prefix sum over the threads of the workgroup; `scratch` holds NW ints
// and is not reused by the caller before the next barrier.  Contains one barrier.
template <int NW>
__device__ inline int block_scan_incl(int x, int* scratch, int* total) {
  const int inc = wave_scan_incl(x);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 63) scratch[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = scratch[w];
    before += (w < wave) ? c : 0;
    tot += c;
  }
  *total = tot;
  return before + inc;
}

// Sum of per-wave counts `wcount` (NW entries) over the waves before this one, and in total.
template <int NW>
__device__ inline int waves_before(const int* wcount, int* total) {
  const int wave = threadIdx.x >> 6;
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = wcount[w];
    before += (w < wave) ? c : 0;
    tot += c;
  }
  *total = tot;
  return before;
}

// Number of entries of v[0 .. n) greater (ABOVE) or smaller (!ABOVE) than x.  v is
// 16-byte aligned and holds, from n up to the next multiple of 32, entries that never
// count (0 when counting larger ones, all ones when counting smaller ones), so the
// loop needs no per-entry bound; 32 entries are read per wait.
template <bool ABOVE>
__device__ inline int count_cmp(const uint64_t* v, int n, uint64_t x) {
  int rank = 0;
  for (int u = 0; u < n; u += 32) {
    u32x4 w[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) w[j] = *(const u32x4*)(v + u + 2 * j);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint64_t a = ((uint64_t)w[j].y << 32) | w[j].x;
      const uint64_t b = ((uint64_t)w[j].w << 32) | w[j].z;
      rank += ABOVE ? (a > x) : (a < x);
      rank += ABOVE ? (b > x) : (b < x);
    }
  }
  return rank;
}

// Selects the min(K, n_cand) best of row[0 .. n_cand) into sh.sorted_idx, best
// first, and returns that count.  Every thread of the workgroup must call it.
// With `bm` (cleared before the call), the selected blocks are marked in bm->sel and
// this thread's resident block `res_block` (if in [0, NB)) in bm->res, both complete
// when the call returns a count above zero.
// Scores per workgroup that fit the bucket array, where they can wait for lookups.
template <int THREADS, int ITEMS>
constexpr bool kCanStage = ITEMS * THREADS * sizeof(float) <= sizeof(SelectShared<THREADS, ITEMS>::bucket);

// row holds NB readable scores; every thread's scores are requested before anything
// waits (the length, and with it n_cand, arrives meanwhile).  With `res_key` (only
// when kCanStage), the keys also pass through LDS and *res_key receives the order key
// of the score of `res_block` (that of -inf outside the candidates), so that no second
// global read depends on the first.
// MBOX: the keys come from the mailbox row `mrow` of a hand-off instead (the caller has
// waited for the head's arrivals): each candidate's key is read until it is non-zero
// and then cleared, leaving the row zero; the row's scores then go to `score_out`
// (-inf past the candidates), whole lines at a time.
template <int THREADS, int ITEMS, bool MBOX = false>
__device__ __attribute__((always_inline)) int topk_select(const float* __restrict__ row, int n_cand, int K,
                           SelectShared<THREADS, ITEMS>& sh, int NB, PlanBitmaps* bm = nullptr,
                           int res_block = -1, uint32_t* res_key = nullptr,
                           uint32_t* mrow = nullptr, uint32_t* status = nullptr,
                           float* score_out = nullptr) {
  constexpr int NW = THREADS / 64;
  constexpr bool kStage = kCanStage<THREADS, ITEMS>;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint32_t key[ITEMS];
  // MBOX: the row through a buffer resource (device-scope loads issued together).
  const __amdgpu_buffer_rsrc_t mr =
      __builtin_amdgcn_make_buffer_rsrc(MBOX ? (void*)mrow : (void*)row, (short)0, MBOX ? NB * 4 : 0, 0x00020000);
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int e = i * THREADS + tid;
    const int ec = e < NB ? e : NB - 1;
    key[i] = MBOX ? __builtin_amdgcn_raw_buffer_load_b32(mr, (uint32_t)ec * 4u, 0, kDevScopeAux)
                  : order_key(row[ec]);
  }
  if (res_key != nullptr) *res_key = order_key(-INFINITY);
  const int m = n_cand < K ? n_cand : K;
  if (MBOX) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {  // a key still zero has not arrived yet: read it again
      const int e = i * THREADS + tid;
      if (e < n_cand && key[i] == 0u) key[i] = ld_dev_nonzero(mrow + e, status, kStatusScoreWait);
    }
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int e = i * THREADS + tid;
      if (e < n_cand) __builtin_amdgcn_raw_buffer_store_b32(0u, mr, (uint32_t)e * 4u, 0, kDevScopeAux);
      if (e < NB) score_out[e] = e < n_cand ? key_float(key[i]) : -INFINITY;
    }
  }
  if (m <= 0) return 0;  // uniform across the workgroup

  uint32_t lmax = 0u, lmin = 0xffffffffu;
  uint32_t* staged = reinterpret_cast<uint32_t*>(sh.bucket);
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int e = i * THREADS + tid;
    if (e < n_cand) {
      lmax = max(lmax, key[i]);
      lmin = min(lmin, key[i]);
      if (kStage && res_key != nullptr) staged[e] = key[i];
    } else {
      key[i] = 0u;
    }
  }
  lmax = wave_max_u32(lmax);
  lmin = wave_min_u32(lmin);
  if (lane == 0) {
    sh.rmax[wave] = lmax;
    sh.rmin[wave] = lmin;
  }
  __syncthreads();
  if (bm != nullptr && res_block >= 0 && res_block < NB)   // after the clear, before the last barrier
    atomicOr(&bm->res[res_block >> 5], 1u << (res_block & 31));
  // The staged keys are overwritten only after the first radix pass's barriers.
  if (kCanStage<THREADS, ITEMS> && res_key != nullptr && res_block >= 0 && res_block < n_cand)
    *res_key = staged[res_block];
  uint32_t kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    kmax = max(kmax, sh.rmax[w]);
    kmin = min(kmin, sh.rmin[w]);
  }

  // Radix select below the common high bits.  Invariant: `prefix` holds the
  // threshold key's bits at positions > top (and zeros below); krem of the keys
  // that match it there are still to be taken.
  uint32_t prefix = kmax;
  int krem = m;
  int lo = 32;  // keys are compared on key >> lo
  const uint32_t diff = kmax ^ kmin;
  if (diff != 0u) {
    int top = 31 - __clz(diff);
    prefix = (uint32_t)(((uint64_t)kmax >> (top + 1)) << (top + 1));
    for (int pass = 0;; ++pass) {
      lo = top >= 7 ? top - 7 : 0;
      const uint32_t dmask = (1u << (top - lo + 1)) - 1u;
      const uint64_t hi_match = (uint64_t)prefix >> (top + 1);
      uint32_t* hist = sh.hist[pass & 1][wave];
      for (int dd = lane; dd < 256; dd += 64) hist[dd] = 0u;  // this wave's own histogram
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int e = i * THREADS + tid;
        if (e < n_cand && ((uint64_t)key[i] >> (top + 1)) == hi_match)
          atomicAdd(&hist[(key[i] >> lo) & dmask], 1u);
      }
      __syncthreads();
      // Thread t owns digit 255 - t: the prefix sum runs from the largest digit down.
      const int digit = 255 - tid;
      int cnt = 0;
      if (tid < 256) {
#pragma unroll
        for (int w = 0; w < NW; ++w) cnt += (int)sh.hist[pass & 1][w][digit];
      }
      int tot;
      const int incl = block_scan_incl<NW>(cnt, sh.scan[pass & 1], &tot);
      const int excl = incl - cnt;
      if (cnt > 0 && excl < krem && krem <= incl) {
        sh.sel_digit = (uint32_t)digit;
        sh.sel_above = excl;
        sh.sel_count = cnt;
      }
      if (pass == 0 && tid < 256) {
        sh.start[digit] = excl;
        sh.fill[digit] = 0;
      }
      __syncthreads();
      if (pass == 0 && sh.sel_count <= kBucketMax) {
        // Fast path.  Every key whose first-pass digit is at least the threshold digit
        // d0 goes to its digit's bucket; buckets are laid out from the largest digit
        // down, bucket d starting at start[d], so the placed keys occupy
        // [0, above + count(d0)).  A key's rank among the larger composites of its own
        // bucket then gives its final position; of the threshold bucket the keys with
        // rank below the number still needed are taken.
        const uint32_t d0 = sh.sel_digit;
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
          const int e = i * THREADS + tid;
          const uint32_t dg = (key[i] >> lo) & dmask;
          if (e < n_cand && dg >= d0) {
            const int slot = (int)atomicAdd((uint32_t*)&sh.fill[dg], 1u);
            sh.bucket[sh.start[dg] + slot] = ((uint64_t)key[i] << 32) | (uint32_t)(~(uint32_t)e);
          }
        }
        __syncthreads();
        const int above = sh.sel_above;
        const int need = krem - above;
        const int placed = above + sh.sel_count;
        for (int t = tid; t < placed; t += THREADS) {
          const uint64_t c = sh.bucket[t];
          const uint32_t dg = ((uint32_t)(c >> 32) >> lo) & dmask;
          const int b0 = sh.start[dg], nb = sh.fill[dg];
          int r = 0;
          for (int u = 0; u < nb; u += 16) {  // 16 reads in flight per wait
            uint64_t a[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) a[j] = sh.bucket[b0 + u + j];  // padded: stays in the array
#pragma unroll
            for (int j = 0; j < 16; ++j) r += (u + j < nb) && a[j] > c;
          }
          const int pos = dg > d0 ? b0 + r : (r < need ? above + r : -1);
          if (pos >= 0) {
            const int e = (int)(~(uint32_t)c);
            sh.sorted_idx[pos] = e;
            if (bm != nullptr) atomicOr(&bm->sel[e >> 5], 1u << (e & 31));
          }
        }
        __syncthreads();
        return m;
      }
      prefix |= sh.sel_digit << lo;
      krem -= sh.sel_above;
      const int count = sh.sel_count;
      if (lo == 0 || count == krem) break;  // every key matching the prefix is taken
      top = lo - 1;
    }
  }

  // Collect: keys above the threshold (on key >> lo) all go; of the keys equal to
  // it, the krem with the lowest indices.  Index order is (item, wave, lane).
  const uint64_t thr = (uint64_t)prefix >> lo;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int e = i * THREADS + tid;
    const uint64_t kk = (uint64_t)key[i] >> lo;
    const int cg = __popcll(__ballot(e < n_cand && kk > thr));
    const int ce = __popcll(__ballot(e < n_cand && kk == thr));
    if (lane == 0) sh.cnt[i * NW + wave] = ce | (cg << 16);
  }
  __syncthreads();
  {
    const int v = (tid < ITEMS * NW) ? sh.cnt[tid] : 0;
    int tot;
    const int incl = block_scan_incl<NW>(v, sh.scan[0], &tot);
    if (tid < ITEMS * NW) sh.cnt[tid] = incl - v;  // exclusive, packed
    if (tid == 0) sh.n_gt = (int)((uint32_t)tot >> 16);
  }
  __syncthreads();
  const int n_gt = sh.n_gt;  // == m - krem
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int e = i * THREADS + tid;
    const uint64_t kk = (uint64_t)key[i] >> lo;
    const bool gt = e < n_cand && kk > thr;
    const bool eq = e < n_cand && kk == thr;
    int unused;
    const int rg = wave_flag_rank(gt, &unused);
    const int re = wave_flag_rank(eq, &unused);
    const int base = sh.cnt[i * NW + wave];
    const uint64_t comp = ((uint64_t)key[i] << 32) | (uint32_t)(~(uint32_t)e);
    if (gt) sh.cand[(int)((uint32_t)base >> 16) + rg] = comp;
    const int r = (base & 0xffff) + re;
    if (eq && r < krem) sh.cand[n_gt + r] = comp;
  }
  if (tid >= m && tid < ((m + 31) & ~31)) sh.cand[tid] = 0ull;  // never larger than a key
  __syncthreads();
  // Rank sort of the m winners: rank = number of larger composites.  The loop reads
  // LDS 16 bytes at a time, several reads in flight.
  for (int t = tid; t < m; t += THREADS) {
    const uint64_t ct = sh.cand[t];
    const int e = (int)(~(uint32_t)ct);
    sh.sorted_idx[count_cmp<true>(sh.cand, m, ct)] = e;
    if (bm != nullptr) atomicOr(&bm->sel[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  return m;
}

// The resident slot a thread t < K owns (-1 for the other threads) and the order key
// of that block's score (that of -inf when the block is out of range or not a
// candidate).  Loaded by the caller before the selection so that the latency
// overlaps it.
struct ResidentSlot {
  int block;
  uint32_t key;
};
__device__ inline ResidentSlot load_resident_slot(const int32_t* res, const float* __restrict__ srow,
                                                  int K, int NB) {
  const int tid = threadIdx.x;
  const int r = tid < K ? res[tid] : -1;
  const bool ok = r >= 0 && r < NB;
  const float sc = srow[ok ? r : 0];
  return ResidentSlot{r, order_key(ok ? sc : -INFINITY)};
}

// Applies the capped-eviction rule for one (sequence, KV head).  Thread t < K passes
// selection entry t as `s_i` (-1 = none; the entries are best first) and resident slot
// t as `rs`; the updated slots go to `res_next`.  `bm` must have been cleared, with a
// barrier since; with MARKED it already holds both sets (the selection marked them).
// Needs K <= THREADS; every thread calls it.
template <int THREADS, bool MARKED = false>
__device__ __attribute__((always_inline)) void plan_apply(
    int s_i, ResidentSlot rs, int32_t* res_next, int32_t* plan_row, int32_t* plan_count,
    int32_t* table_row, int32_t* table_count, int K, int C, int NB, int w0, int nblk, int T,
    PlanBitmaps& bm, PlanShared<THREADS>& sh) {
  constexpr int NW = THREADS / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r_i = rs.block;
  if (tid >= K) s_i = -1;
  const bool s_ok = s_i >= 0 && s_i < NB;
  const bool r_ok = r_i >= 0 && r_i < NB;
  if (!MARKED) {
    if (s_ok) atomicOr(&bm.sel[s_i >> 5], 1u << (s_i & 31));
    if (r_ok) atomicOr(&bm.res[r_i >> 5], 1u << (r_i & 31));
    __syncthreads();
  }

  // New blocks (selection order) and empty slots (slot order): ballot ranks.
  const bool is_new = s_ok && !((bm.res[s_i >> 5] >> (s_i & 31)) & 1u);
  const bool empty = tid < K && r_i < 0;
  const bool stale = tid < K && r_i >= 0 && !(r_ok && ((bm.sel[r_i >> 5] >> (r_i & 31)) & 1u));
  int c_new, c_empty, c_stale;
  const int rk_new = wave_flag_rank(is_new, &c_new);
  const int rk_empty = wave_flag_rank(empty, &c_empty);
  const int rk_stale = wave_flag_rank(stale, &c_stale);
  if (lane == 0) {
    bm.w_new[wave] = c_new;
    bm.w_empty[wave] = c_empty;
    bm.w_stale[wave] = c_stale;
  }
  // Worst-first order of stale slots: ascending score, equal scores higher block first.
  const uint64_t st_me =
      stale ? (((uint64_t)(r_ok ? rs.key : order_key(-INFINITY)) << 32) | (uint32_t)(~(uint32_t)r_i))
            : ~0ull;
  __syncthreads();
  int n_new, n_empty, n_stale;
  const int pos_new = waves_before<NW>(bm.w_new, &n_new) + rk_new;
  const int pos_empty = waves_before<NW>(bm.w_empty, &n_empty) + rk_empty;
  const int pos_stale = waves_before<NW>(bm.w_stale, &n_stale) + rk_stale;
  const int n = C < n_new ? C : n_new;
  const bool admitted = is_new && pos_new < n;
  if (admitted) sh.adm_list[pos_new] = s_i;
  if (stale) sh.st[pos_stale] = st_me;  // only the stale slots are ranked
  if (tid >= n_stale && tid < ((n_stale + 31) & ~31)) sh.st[tid] = ~0ull;  // never smaller
  if (tid >= n && tid < ((n + 15) & ~15)) sh.adm_list[tid] = 0x7fffffff;   // never smaller
  __syncthreads();

  // Victims: the first n of (empty slots by slot, stale slots by score asc, block desc).
  bool victim = false;
  if (empty) {
    victim = pos_empty < n;
  } else if (stale && n > n_empty) {
    victim = count_cmp<false>(sh.st, n_stale, st_me) < n - n_empty;
  }
  if (admitted) {
    int rank = 0;
    for (int u = 0; u < n; u += 16) {
      u32x4 w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = *(const u32x4*)(sh.adm_list + u + 4 * j);
#pragma unroll
      for (int j = 0; j < 16; ++j) rank += (int)w[j >> 2][j & 3] < s_i;
    }
    sh.adm_sorted[rank] = s_i;
  }
  int c_vict;
  const int rk_vict = wave_flag_rank(victim, &c_vict);
  // Table entries: a victim takes an admitted block (a candidate); a kept slot is listed
  // if its block lies before the first window block.  A block the window has reached
  // stays resident but is attended once, as a window block.
  const bool tabled = tid < K && (victim || (r_i >= 0 && r_i < w0));
  int c_tab;
  const int rk_tab = wave_flag_rank(tabled, &c_tab);
  if (lane == 0) {
    bm.w_vict[wave] = c_vict;
    bm.w_tab[wave] = c_tab;
  }
  __syncthreads();
  int n_vict, n_res;
  const int pos_vict = waves_before<NW>(bm.w_vict, &n_vict) + rk_vict;
  const int pos_tab = waves_before<NW>(bm.w_tab, &n_res) + rk_tab;
  // Empty plus stale slots number K - |R and S| >= |S without R| >= n, so every one
  // of the n victims takes an admitted block.
  const int n_placed = n < n_vict ? n : n_vict;

  int new_r = r_i;
  if (victim && pos_vict < n_placed) {
    new_r = sh.adm_sorted[pos_vict];
    plan_row[3 * pos_vict + 0] = tid;
    plan_row[3 * pos_vict + 1] = new_r;
    plan_row[3 * pos_vict + 2] = r_i;
  }
  // Every slot is written so that res_next may be another buffer; when it is `res`
  // itself each thread rewrites only the slot it read above.
  if (tid < K) res_next[tid] = new_r;
  for (int r = n_placed + tid; r < C; r += THREADS) {
    plan_row[3 * r + 0] = -1;
    plan_row[3 * r + 1] = -1;
    plan_row[3 * r + 2] = -1;
  }
  if (tid == 0) *plan_count = n_placed;

  // Table: the listed resident entries in slot order, then the window blocks.  Every
  // victim takes an admitted block (there are n of each), so a victim's entry is its
  // new block.
  if (tabled) table_row[pos_tab] = new_r;
  const int nwin = nblk - w0;
  for (int i = tid; i < nwin; i += THREADS) table_row[n_res + i] = w0 + i;
  for (int i = n_res + nwin + tid; i < T; i += THREADS) table_row[i] = -1;
  if (tid == 0) *table_count = n_res + nwin;
}

// The LDS of a selection-and-plan workgroup.  The selection's part is dead once
// each thread holds its entry, so the plan reuses it (the plan's first write to it
// follows a barrier that comes after every read of the selection).
template <int THREADS, int ITEMS>
union TopkPlanShared {
  SelectShared<THREADS, ITEMS> t;
  PlanShared<THREADS> p;
};

// Arguments of the selection-and-plan work.
struct TopkPlanArgs {
  const float* scores;
  const int32_t* seq_lens;
  int32_t* topk;
  const int32_t* resident;
  int32_t* resident_next;
  int32_t* plan;
  int32_t* plan_count;
  int32_t* table;
  int32_t* table_count;
  int heads, NB, K, C, window, T, bshift;
};

// Selection and plan of (sequence, KV head) `bh` in one workgroup; the bitmaps are
// cleared while the selection runs.  Every thread of the workgroup calls it.
// MBOX: the scores are handed over by the scoring workgroups of the same launch
// through `ho` (wave 0 waits for the flags of the head's scoring waves and clears
// them, then every thread reads its keys from the mailbox), and the workgroup writes
// the head's row of the scores output from them.
template <int THREADS, int ITEMS, bool MBOX = false>
__device__ __attribute__((always_inline)) void topk_plan_wg(int bh, TopkPlanShared<THREADS, ITEMS>& sh,
                                                            PlanBitmaps& bm, const TopkPlanArgs& a,
                                                            const Handoff* ho = nullptr) {
  static_assert(!MBOX || kCanStage<THREADS, ITEMS>, "mailbox keys are staged for the resident lookup");
  const int NB = a.NB, K = a.K, C = a.C, T = a.T;
  const int len = clamp_len(a.seq_lens[bh / a.heads], NB, a.bshift);
  const int n_cand = first_window_block(len, a.window, a.bshift);
  const float* srow = a.scores + (size_t)bh * NB;
  ResidentSlot rs;
  if (kCanStage<THREADS, ITEMS>) {  // the key comes from the selection's staging
    rs.block = (int)threadIdx.x < K ? a.resident[(size_t)bh * K + threadIdx.x] : -1;
    rs.key = order_key(-INFINITY);
  } else {
    rs = load_resident_slot(a.resident + (size_t)bh * K, srow, K, NB);
  }
  clear_bitmaps(bm, NB);
  if (MBOX) {
    if (threadIdx.x < 64)
      wait_flags(ho->flag_score + (size_t)bh * ho->score_waves, ho->score_waves, ho->status, kStatusScoreWait);
    __syncthreads();
  }
  const int m = topk_select<THREADS, ITEMS, MBOX>(srow, n_cand, K, sh.t, NB, &bm, rs.block,
                                                  kCanStage<THREADS, ITEMS> ? &rs.key : nullptr,
                                                  MBOX ? ho->mbox + (size_t)bh * NB : nullptr,
                                                  MBOX ? ho->status : nullptr,
                                                  MBOX ? ho->scores + (size_t)bh * NB : nullptr);
  if (m == 0) {  // the selection returned at once: mark the resident set here
    __syncthreads();
    if (rs.block >= 0 && rs.block < NB) atomicOr(&bm.res[rs.block >> 5], 1u << (rs.block & 31));
    __syncthreads();
  }
  for (int t = threadIdx.x; t < K; t += THREADS) a.topk[(size_t)bh * K + t] = t < m ? sh.t.sorted_idx[t] : -1;
  const int s_i = (threadIdx.x < m) ? sh.t.sorted_idx[threadIdx.x] : -1;
  plan_apply<THREADS, true>(s_i, rs, a.resident_next + (size_t)bh * K,
                      a.plan == nullptr ? nullptr : a.plan + (size_t)bh * C * 3, a.plan_count + bh,
                      a.table + (size_t)bh * T, a.table_count + bh, K, C, NB, n_cand,
                      num_blocks(len, a.bshift), T, bm, sh.p);
}

// Host side: the argument block of the selection-and-plan work for `d`.
inline TopkPlanArgs topk_plan_args(const Dims& d, const float* scores, const int32_t* seq_lens,
                                   int32_t* topk, const int32_t* resident, int32_t* resident_next,
                                   int32_t* plan, int32_t* plan_count, int32_t* table,
                                   int32_t* table_count) {
  TopkPlanArgs a;
  a.scores = scores;
  a.seq_lens = seq_lens;
  a.topk = topk;
  a.resident = resident;
  a.resident_next = resident_next;
  a.plan = plan;
  a.plan_count = plan_count;
  a.table = table;
  a.table_count = table_count;
  a.heads = d.heads;
  a.NB = d.max_blocks;
  a.K = d.top_k;
  a.C = d.cap;
  a.window = d.window;
  a.T = d.table_stride;
  a.bshift = d.bshift;
  return a;
}

// Workgroup size and scores per thread for a problem: 512 threads while K <= 512
// and the scores fit 16 per thread (measured fastest for 64 heads of 2048 blocks,
// K = 128: fewer serial loads and LDS atomics per thread than 256, fewer waves per
// barrier than 1024; and for 32 heads of 8192 blocks); with 128 heads or more, 256 threads while K <= 256 and 2048
// blocks (the selection shares launch 2 with the merge, and smaller workgroups fit
// more of both per CU: 12 against 20 us at 128 heads, 13.5 against 22.5 at 512);
// else 1024 (up to 32 per thread).
#ifndef OASIS_SELECT_MID_ITEMS
#define OASIS_SELECT_MID_ITEMS 16  // 8192 blocks: 12.8 us with 512 threads, 13.5 with 1024
#endif
inline int select_threads(const Dims& d) {
  if ((int64_t)d.batch * d.heads >= 128 && d.top_k <= 256 && d.max_blocks <= 256 * 8) return 256;
  return (d.top_k <= 512 && d.max_blocks <= 512 * OASIS_SELECT_MID_ITEMS) ? 512 : 1024;
}
inline int select_items(const Dims& d, int threads) {
  int items = 1;
  while (items * threads < d.max_blocks) items <<= 1;
  return items;
}

#define OASIS_SELECT_DISPATCH(CASE)                                                  \
  do {                                                                               \
    const int threads_ = select_threads(d);                                          \
    const int items_ = select_items(d, threads_);                                    \
    if (threads_ == 256) {                                                           \
      switch (items_) {                                                              \
        CASE(256, 1) CASE(256, 2) CASE(256, 4) CASE(256, 8)                          \
        default: return hipErrorInvalidValue;                                        \
      }                                                                              \
    } else if (threads_ == 512) {                                                    \
      switch (items_) {                                                              \
        CASE(512, 1) CASE(512, 2) CASE(512, 4) CASE(512, 8) CASE(512, 16)            \
        default: return hipErrorInvalidValue;                                        \
      }                                                                              \
    } else {                                                                         \
      switch (items_) {                                                              \
        CASE(1024, 1) CASE(1024, 2) CASE(1024, 4) CASE(1024, 8) CASE(1024, 16)       \
        CASE(1024, 32)                                                               \
        default: return hipErrorInvalidValue;                                        \
      }                                                                              \
    }                                                                                \
  } while (0)


}  // namespace oasis
