// Executing the plan: the working set of every KV head in HBM, on gfx950.
//
// The full K/V cache stays where it is (host memory, or HBM when it fits) and
// keeps its layout: that is the page table, which never changes.  HBM holds, per
// (sequence, KV head), a pool of K block slots, which the head's resident slot
// table maps to logical blocks (the head-wise logical-to-logical map), and a ring
// of window blocks (xllm-io review, section three: component table, head-wise
// mapping above the paged cache, and training flow steps 2 and 3: the GPU keeps
// the selected historical blocks and the local window, and the plan is carried
// out as an asynchronous transfer; section four, innovations table: only
// head-wise mapping entries change; legiblepapers.com FAQ Q4; lode.cx points 1
// and 3).  Pool slot s holds the block of slot s; window block j sits in ring
// slot j % WB, WB = ceil(W/bs) + 1 being the most window blocks a length has (bs:
// tokens per block, 8 to 64).
//
// Kernels:
//   fill_working_set_kernel  gathers a slot table's pool and the window ring from
//                            the full cache (admission, or a rebuild);
//   execute_plan_kernel      copies each plan row's admitted block into its slot
//                            (the evicted block needs no transfer: the full tier
//                            keeps every block);
//   append_token_kernel      writes a decoded token's K and V into the full cache
//                            and the ring and updates its block's min/max summary
//                            in place (the compressed-key update, xllm-io review,
//                            section five).
// A block copy moves bs * 256 bytes of K and of V with 256 threads, one 16-byte load
// and store per thread and tensor for each 4 KB (a 16-token block: one each), so
// that copies from host memory (a mapped pinned buffer read over the host link)
// and from HBM take the same code.
#include "common.h"
#include "launch.h"

namespace oasis {

constexpr int kCopyThreads = 256;
// 16-byte chunks of one block: 16 per token.
__host__ __device__ inline int block_chunks(int bshift) { return 16 << bshift; }

__device__ inline void copy_block(const u32x4* __restrict__ sk, const u32x4* __restrict__ sv,
                                  u32x4* __restrict__ dk, u32x4* __restrict__ dv, int nch) {
  for (int t = threadIdx.x; t < nch; t += kCopyThreads) {
    const u32x4 a = sk[t], b = sv[t];
    dk[t] = a;
    dv[t] = b;
  }
}

// Workgroup (s, bh): pool slot s < K, else ring slot s - K, of (sequence, KV head) bh.
__global__ __launch_bounds__(kCopyThreads) void fill_working_set_kernel(
    const int32_t* __restrict__ resident, const int32_t* __restrict__ seq_lens,
    const u32x4* __restrict__ k, const u32x4* __restrict__ v, u32x4* __restrict__ pool_k,
    u32x4* __restrict__ pool_v, u32x4* __restrict__ ring_k, u32x4* __restrict__ ring_v,
    int heads, int NB, int K, int WB, int window, int bshift) {
  const int s = blockIdx.x, bh = blockIdx.y;
  const int nch = block_chunks(bshift);
  int j;
  size_t dst;
  u32x4 *dk, *dv;
  if (s < K) {
    j = resident[(size_t)bh * K + s];
    if (j < 0 || j >= NB) return;  // empty slot: left as it is
    dst = ((size_t)bh * K + s) * nch;
    dk = pool_k;
    dv = pool_v;
  } else {
    const int r = s - K;
    const int len = clamp_len(seq_lens[bh / heads], NB, bshift);
    const int w0 = first_window_block(len, window, bshift), nb = num_blocks(len, bshift);
    j = w0 + ((r - w0 % WB) % WB + WB) % WB;  // the window block of ring slot r, if any
    if (j >= nb) return;
    dst = ((size_t)bh * WB + r) * nch;
    dk = ring_k;
    dv = ring_v;
  }
  const size_t src = ((size_t)bh * NB + j) * nch;
  copy_block(k + src, v + src, dk + dst, dv + dst, nch);
}

// At most kCopyGrid workgroups walk all plan rows (row r = bh * C + i), kCopyRows
// rows per round with every load of the round (4 KB of each row's K and V) in flight
// before the first store: a plan of up to 1024 rows of 16-token blocks (6 per head at
// 8 x 8 heads is 384) goes out in one round from HBM, larger plans fill the host link
// in several, and the copies hold at most one workgroup's slots per CU, so that they
// can run beside another stream's kernels.
#ifndef OASIS_COPY_ROWS
#define OASIS_COPY_ROWS 4
#endif
#ifndef OASIS_COPY_GRID
#define OASIS_COPY_GRID 256
#endif
constexpr int kCopyRows = OASIS_COPY_ROWS;
constexpr int kCopyGrid = OASIS_COPY_GRID;
__global__ __launch_bounds__(kCopyThreads) void execute_plan_kernel(
    const int32_t* __restrict__ plan, const int32_t* __restrict__ plan_count,
    const u32x4* __restrict__ k, const u32x4* __restrict__ v, u32x4* __restrict__ pool_k,
    u32x4* __restrict__ pool_v, int NB, int K, int C, int rows, int bshift) {
  const int nch = block_chunks(bshift);
  for (int r0 = blockIdx.x * kCopyRows; r0 < rows; r0 += gridDim.x * kCopyRows) {
    size_t src[kCopyRows], dst[kCopyRows];
    bool ok[kCopyRows];
#pragma unroll
    for (int u = 0; u < kCopyRows; ++u) {
      const int r = r0 + u;
      ok[u] = false;
      src[u] = dst[u] = 0;
      if (r < rows) {
        const int bh = r / C, i = r % C;
        if (i < plan_count[bh]) {
          const int32_t* row = plan + (size_t)r * 3;
          const int slot = row[0], blk = row[1];
          ok[u] = slot >= 0 && slot < K && blk >= 0 && blk < NB;
          src[u] = ((size_t)bh * NB + (ok[u] ? blk : 0)) * nch;
          dst[u] = ((size_t)bh * K + (ok[u] ? slot : 0)) * nch;
        }
      }
    }
    for (int t = threadIdx.x; t < nch; t += kCopyThreads) {
      u32x4 a[kCopyRows], b[kCopyRows];
#pragma unroll
      for (int u = 0; u < kCopyRows; ++u) {
        if (ok[u]) {
          a[u] = k[src[u] + t];
          b[u] = v[src[u] + t];
        }
      }
#pragma unroll
      for (int u = 0; u < kCopyRows; ++u) {
        if (ok[u]) {
          pool_k[dst[u] + t] = a[u];
          pool_v[dst[u] + t] = b[u];
        }
      }
    }
  }
}

// Workgroup bh, one wave: lane l owns head dims 2l and 2l + 1 (one packed bf16 pair).
__global__ __launch_bounds__(64) void append_token_kernel(
    const uint32_t* __restrict__ k_new, const uint32_t* __restrict__ v_new,
    const int32_t* __restrict__ seq_lens, uint32_t* __restrict__ summ, uint32_t* __restrict__ k,
    uint32_t* __restrict__ v, uint32_t* __restrict__ ring_k, uint32_t* __restrict__ ring_v,
    int heads, int NB, int WB, int bshift) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  const int L = seq_lens[bh / heads];
  if (L < 0 || L >= (NB << bshift)) return;  // no room: the sequence is skipped
  const int j = L >> bshift, t = L & ((1 << bshift) - 1);
  const uint32_t kn = k_new[(size_t)bh * 64 + lane], vn = v_new[(size_t)bh * 64 + lane];
  const size_t tok = ((((size_t)bh * NB + j) << bshift) + t) * 64 + lane;
  if (k != nullptr) {
    k[tok] = kn;
    v[tok] = vn;
  }
  const size_t rtok = ((((size_t)bh * WB + j % WB) << bshift) + t) * 64 + lane;
  ring_k[rtok] = kn;
  ring_v[rtok] = vn;
  uint32_t* su = summ + ((size_t)bh * NB + j) * 128 + lane;  // min at [0], max at [64]
  if (t == 0) {  // the token opens its block
    su[0] = kn;
    su[64] = kn;
  } else {
    const uint32_t lo = su[0], hi = su[64];
    const float mn0 = fminf(bf16_lo(lo), bf16_lo(kn)), mn1 = fminf(bf16_hi(lo), bf16_hi(kn));
    const float mx0 = fmaxf(bf16_lo(hi), bf16_lo(kn)), mx1 = fmaxf(bf16_hi(hi), bf16_hi(kn));
    // Each result is one of two bf16 values, so keeping its top 16 bits is exact.
    su[0] = (__float_as_uint(mn0) >> 16) | (__float_as_uint(mn1) & 0xffff0000u);
    su[64] = (__float_as_uint(mx0) >> 16) | (__float_as_uint(mx1) & 0xffff0000u);
  }
}

hipError_t launch_fill_working_set(const Dims& d, const int32_t* resident, const int32_t* seq_lens,
                                   const void* k, const void* v, const WorkingSet& w,
                                   hipStream_t stream) {
  const int WB = d.table_stride - d.top_k;
  fill_working_set_kernel<<<dim3(d.top_k + WB, d.batch * d.heads), dim3(kCopyThreads), 0, stream>>>(
      resident, seq_lens, (const u32x4*)k, (const u32x4*)v, (u32x4*)w.pool_k, (u32x4*)w.pool_v,
      (u32x4*)w.ring_k, (u32x4*)w.ring_v, d.heads, d.max_blocks, d.top_k, WB, d.window, d.bshift);
  return hipGetLastError();
}

hipError_t launch_execute_plan(const Dims& d, const int32_t* plan, const int32_t* plan_count,
                               const void* k, const void* v, void* pool_k, void* pool_v,
                               hipStream_t stream) {
  if (d.cap <= 0 || plan == nullptr) return hipSuccess;  // nothing can be admitted
  const int rows = d.batch * d.heads * d.cap;
  int grid = (rows + kCopyRows - 1) / kCopyRows;
  if (grid > kCopyGrid) grid = kCopyGrid;
  execute_plan_kernel<<<dim3(grid), dim3(kCopyThreads), 0, stream>>>(
      plan, plan_count, (const u32x4*)k, (const u32x4*)v, (u32x4*)pool_k, (u32x4*)pool_v,
      d.max_blocks, d.top_k, d.cap, rows, d.bshift);
  return hipGetLastError();
}

hipError_t launch_append_token(const Dims& d, const void* k_new, const void* v_new,
                               const int32_t* seq_lens, void* summ, void* k, void* v,
                               void* ring_k, void* ring_v, hipStream_t stream) {
  append_token_kernel<<<dim3(d.batch * d.heads), dim3(64), 0, stream>>>(
      (const uint32_t*)k_new, (const uint32_t*)v_new, seq_lens, (uint32_t*)summ, (uint32_t*)k,
      (uint32_t*)v, (uint32_t*)ring_k, (uint32_t*)ring_v, d.heads, d.max_blocks,
      d.table_stride - d.top_k, d.bshift);
  return hipGetLastError();
}

}  // namespace oasis
