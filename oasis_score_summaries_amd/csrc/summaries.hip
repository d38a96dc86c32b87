// Per-block min/max key summaries ("compressed keys") for gfx950.
//
// The compressed key cache keeps, for every logical block and every head
// dimension, the min and the max of the block's keys (xllm-io review of
// OasisKV, section three, component table: Compressed Key Cache, 1/16 of the
// KV size; section two: Quest-style min/max pooling).
//
// One wave per block (8 to 64 tokens): lane l owns head dims 2l and 2l+1 and walks
// the valid tokens, so each token row (256 bytes) is one coalesced wave load.
// bf16 min/max is exact, the result is written back as bf16 bits.
#include "common.h"
#include "launch.h"

namespace oasis {

__global__ __launch_bounds__(256) void build_summaries_kernel(const uint32_t* __restrict__ k,
                                                              const int32_t* __restrict__ seq_lens,
                                                              uint32_t* __restrict__ summ, int heads,
                                                              int max_blocks, int bshift,
                                                              int64_t total_blocks) {
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= total_blocks) return;
  const int lane = threadIdx.x & 63;
  const int j = (int)(blk % max_blocks);
  const int b = (int)(blk / max_blocks / heads);
  const int len = clamp_len(seq_lens[b], max_blocks, bshift);
  const int bs = 1 << bshift;
  int n_valid = len - j * bs;
  n_valid = n_valid > bs ? bs : n_valid;

  // bs tokens x 128 dims of bf16 = bs rows of 64 packed pairs.
  const uint32_t* src = k + ((size_t)blk << bshift) * (kHeadDim / 2) + lane;
  uint32_t* dst = summ + blk * (2 * kHeadDim / 2) + lane;
  if (n_valid <= 0) {
    dst[0] = 0u;
    dst[64] = 0u;
    return;
  }
  float mn0 = INFINITY, mn1 = INFINITY, mx0 = -INFINITY, mx1 = -INFINITY;
  for (int t = 0; t < n_valid; ++t) {
    const uint32_t w = src[t * 64];
    const float lo = bf16_lo(w), hi = bf16_hi(w);
    mn0 = fminf(mn0, lo);
    mx0 = fmaxf(mx0, lo);
    mn1 = fminf(mn1, hi);
    mx1 = fmaxf(mx1, hi);
  }
  // Each value is one of the bf16 inputs, so truncating to 16 bits is exact.
  dst[0] = (__float_as_uint(mn0) >> 16) | (__float_as_uint(mn1) & 0xffff0000u);
  dst[64] = (__float_as_uint(mx0) >> 16) | (__float_as_uint(mx1) & 0xffff0000u);
}

hipError_t launch_build_summaries(const Dims& d, const void* k, const int32_t* seq_lens, void* summ,
                                  hipStream_t stream) {
  const int64_t total = (int64_t)d.batch * d.heads * d.max_blocks;
  const int64_t grid = (total + 3) / 4;
  build_summaries_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(
      (const uint32_t*)k, seq_lens, (uint32_t*)summ, d.heads, d.max_blocks, d.bshift, total);
  return hipGetLastError();
}

}  // namespace oasis
