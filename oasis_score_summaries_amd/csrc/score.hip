// Look-ahead block scoring on gfx950 matrix cores.
//
// The draft and target queries scan the per-block min/max key summaries to
// predict the blocks the next step will need (xllm-io review of OasisKV,
// section two, algorithm layer; section three, component table, Look-ahead
// Attention).  Per query row the block score is the Quest upper bound
//   sum_d max(q_d * kmin_d, q_d * kmax_d),
// and one score per (KV head, block) is the max over the GQA group and the
// target and draft queries.
//
// Because kmin <= kmax, max(q*kmin, q*kmax) = min(q,0)*kmin + max(q,0)*kmax,
// so the scores of all rows against all blocks are one dense product
//   [q-, q+] (rows x 256)  times  [kmin; kmax] (256 x blocks),
// with 20 to 80 multiply-adds per summary byte: above what the vector ALUs
// sustain at HBM speed, so it runs on bf16 MFMA (exact products, fp32 sums).
//
// Layout of one MFMA v_mfma_f32_16x16x32_bf16 step: the 16 rows of a row tile
// (A), 16 candidate blocks (B) and 32 summary features (K).  A block's summary
// is 512 contiguous bytes = 32 chunks of 16 bytes (chunks 0-15 kmin, 16-31
// kmax); lane l reads chunk 4s + l/16 of block l%16 at step s, so each load
// instruction fetches 64 contiguous bytes from each of 16 blocks and a wave's
// 8 steps consume every byte of its 16 blocks once.  The query features are
// permuted the same way, so the contraction is unchanged.
#include "common.h"
#include "launch.h"

namespace oasis {

constexpr int kScoreWaves = 4;          // waves per workgroup
constexpr int kScoreBlocksPerWave = 32; // two 16-block MFMA tiles per wave

template <int RT>
__global__ __launch_bounds__(256) void score_kernel(const u32x4* __restrict__ q,
                                                    const u32x4* __restrict__ summ,
                                                    const int32_t* __restrict__ seq_lens,
                                                    float* __restrict__ scores, int heads,
                                                    int max_blocks, int rows, int window) {
  const int bh = blockIdx.y;
  const int b = bh / heads;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int j0 = (blockIdx.x * kScoreWaves + wave) * kScoreBlocksPerWave;
  if (j0 >= max_blocks) return;
  const int len = clamp_len(seq_lens[b], max_blocks);
  const int n_cand = first_window_block(len, window);
  float* out = scores + (size_t)bh * max_blocks;
  if (j0 >= n_cand) {  // no candidate in this wave's range
    if (lane < kScoreBlocksPerWave && j0 + lane < max_blocks) out[j0 + lane] = -INFINITY;
    return;
  }

  // Summary fragments of both tiles first, so all 16 loads are in flight together.
  u32x4 bv[2][8];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int jb = j0 + 16 * t + col;
    const size_t base = ((size_t)bh * max_blocks + jb) * 32 + grp;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bv[t][s] = (jb < n_cand) ? summ[base + 4 * s] : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // Query fragments: row 16r + col, features of chunk 4s + grp, sign-split so
  // that kmin chunks meet min(q,0) and kmax chunks meet max(q,0).
  u32x4 av[RT][8];
  const u32x4* qb = q + (size_t)bh * rows * 16;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int row = 16 * r + col;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = 4 * s + grp;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < rows) {
        x = qb[row * 16 + (c & 15)];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (s < 4) ? bf16x2_neg_part(x[e]) : bf16x2_pos_part(x[e]);
      }
      av[r][s] = x;
    }
  }

#pragma unroll
  for (int t = 0; t < 2; ++t) {
    floatx4 acc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[r] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[r][s]), as_bf16x8(bv[t][s]),
                                                         acc[r], 0, 0, 0);
      }
    }
    // Lane l holds rows 16r + 4*(l/16) + i of block column l%16: max over its
    // real rows, then across the four lane groups of the column.
    float m = -INFINITY;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (16 * r + 4 * grp + i < rows) m = fmaxf(m, acc[r][i]);
      }
    }
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    const int jb = j0 + 16 * t + col;
    if (grp == 0 && jb < max_blocks) out[jb] = (jb < n_cand) ? m : -INFINITY;
  }
}

hipError_t launch_score(const Dims& d, const void* q, const void* summ, const int32_t* seq_lens,
                        float* scores, hipStream_t stream) {
  const int rows = d.group * d.queries;
  const int per_wg = kScoreWaves * kScoreBlocksPerWave;
  const dim3 grid((d.max_blocks + per_wg - 1) / per_wg, d.batch * d.heads);
  const dim3 block(64 * kScoreWaves);
  const u32x4* qq = (const u32x4*)q;
  const u32x4* ss = (const u32x4*)summ;
  switch ((rows + 15) / 16) {
#define OASIS_SCORE_CASE(RT)                                                                     \
  case RT:                                                                                       \
    score_kernel<RT><<<grid, block, 0, stream>>>(qq, ss, seq_lens, scores, d.heads, d.max_blocks, \
                                                 rows, d.window);                                \
    break;
    OASIS_SCORE_CASE(1)
    OASIS_SCORE_CASE(2)
    OASIS_SCORE_CASE(3)
    OASIS_SCORE_CASE(4)
    OASIS_SCORE_CASE(5)
    OASIS_SCORE_CASE(6)
    OASIS_SCORE_CASE(7)
    OASIS_SCORE_CASE(8)
#undef OASIS_SCORE_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace oasis
