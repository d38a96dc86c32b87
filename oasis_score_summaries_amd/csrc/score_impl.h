// Device-side building block of the look-ahead block scoring (one workgroup of
// candidate blocks), shared by the scoring kernel and the fused kernel of the
// overlapped step.  Internal to liboasis; the design notes are in score.hip.
#pragma once

#include "common.h"
#include "launch.h"

namespace oasis {

#ifndef OASIS_SCORE_TILES_PER_WAVE
#define OASIS_SCORE_TILES_PER_WAVE 2
#endif
constexpr int kScoreWaves = kWavesPerWG;                         // waves per workgroup
constexpr int kScoreThreads = 64 * kScoreWaves;
constexpr int kScoreTilesPerWave = OASIS_SCORE_TILES_PER_WAVE;   // 16-block MFMA tiles per wave
// Tiles per wave of the scoring in the overlapped step's first launch, by row tiles:
// one up to two row tiles (twice the workgroups of half the size, which retire sooner
// and let the attention workgroups in earlier), two from three on (a workgroup's query
// fragments, built once in LDS, then serve twice the summaries).
__host__ __device__ constexpr int step_score_tiles(int rt) { return rt <= 2 ? 1 : 2; }
__host__ __device__ constexpr int score_blocks_per_wg(int tiles) { return kScoreWaves * tiles * 16; }

// The query fragments do not depend on the block, so the workgroup builds them once
// in LDS (sign-split, in MFMA lane order) and every wave reads them from there.
template <int RT>
struct ScoreShared {
  u32x4 afrag[RT][8][64];
};

// Arguments of the scoring work.
struct ScoreArgs {
  const u32x4* q;
  const u32x4* summ;
  const int32_t* seq_lens;
  float* scores;
  int heads, max_blocks, rows, window, bshift;
};

// One workgroup: block range `bx` (score_blocks_per_wg(TILES) candidate blocks) of (sequence,
// KV head) `bh`.  Every thread of the workgroup calls it.  With HANDOFF, the scores
// go to the selection workgroup of the same launch instead of `a.scores`: each
// candidate's order key goes to the mailbox of `ho` (device-scope stores) and every
// wave then sets its flag; the selection writes the scores output, a head's row at a
// time (whole lines, where the scoring waves would write 64-byte pieces).
template <int RT, bool HANDOFF = false, int TILES = kScoreTilesPerWave>
__device__ __attribute__((always_inline)) void score_wg(int bx, int bh, ScoreShared<RT>& sh,
                                                        const ScoreArgs& a,
                                                        const Handoff* ho = nullptr) {
  const u32x4* __restrict__ q = a.q;
  const u32x4* __restrict__ summ = a.summ;
  const int heads = a.heads, max_blocks = a.max_blocks, rows = a.rows, window = a.window;
  auto& afrag = sh.afrag;
  const int b = bh / heads;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  constexpr int kBlocksPerWG = score_blocks_per_wg(TILES);
  const int jw = bx * kBlocksPerWG + wave * TILES * 16;  // this wave's first block
  const int len = clamp_len(a.seq_lens[b], max_blocks, a.bshift);
  const int n_cand = first_window_block(len, window, a.bshift);
  float* out = a.scores + (size_t)bh * max_blocks;
  if ((int)bx * kBlocksPerWG >= n_cand) {  // no candidate in this workgroup's range
    for (int j = threadIdx.x; !HANDOFF && j < kBlocksPerWG; j += blockDim.x) {
      const int jb = bx * kBlocksPerWG + j;
      if (jb < max_blocks) out[jb] = -INFINITY;
    }
    if (HANDOFF && (threadIdx.x & 63) == 0)
      st_dev(ho->flag_score + (size_t)bh * ho->score_waves + bx * kScoreWaves + (threadIdx.x >> 6), 1u);
    return;
  }

  // Loads are issued unconditionally (clamped to valid addresses, results masked
  // later) so that no branch or wait splits them: first this thread's query chunks,
  // then the wave's summary fragments; the query fragments can then be built while
  // the summaries are still in flight.
  constexpr int kQPerThread = RT * 8 * 64 / kScoreThreads;
  const u32x4* qb = q + (size_t)bh * rows * 16;
  u32x4 qv[kQPerThread];
#pragma unroll
  for (int u = 0; u < kQPerThread; ++u) {
    const int f = u * kScoreThreads + threadIdx.x;
    const int row = 16 * (f / 512) + (f & 15);
    const int c = 4 * ((f / 64) % 8) + ((f & 63) >> 4);
    qv[u] = qb[(row < rows ? row : rows - 1) * 16 + (c & 15)];
  }
  u32x4 bv[TILES][8];
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    int jb = jw + 16 * t + col;
    jb = jb < n_cand ? jb : n_cand - 1;  // n_cand >= 1 here; columns past it are masked below
    const size_t base = ((size_t)bh * max_blocks + jb) * 32 + grp;
#pragma unroll
    for (int s = 0; s < 8; ++s) bv[t][s] = summ[base + 4 * s];
  }

  // Query fragments: (row tile r, step s, lane) holds row 16r + lane%16, features of
  // chunk 4s + lane/16, sign-split so that kmin chunks (s < 4) meet min(q,0) and kmax
  // chunks meet max(q,0); rows past the real ones are zero.
#pragma unroll
  for (int u = 0; u < kQPerThread; ++u) {
    const int f = u * kScoreThreads + threadIdx.x;
    const int r = f / 512, st = (f / 64) % 8, l = f & 63;
    u32x4 x = qv[u];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (st < 4) ? bf16x2_neg_part(x[e]) : bf16x2_pos_part(x[e]);
    if (16 * r + (l & 15) >= rows) x = u32x4{0u, 0u, 0u, 0u};
    afrag[r][st][l] = x;
  }
  __syncthreads();

#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const int jb = jw + 16 * t + col;
    if (jw + 16 * t >= max_blocks) break;  // uniform across the wave
    floatx4 acc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[r] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(afrag[r][s][lane]),
                                                         as_bf16x8(bv[t][s]), acc[r], 0, 0, 0);
      }
      // With three or more row tiles, holding every step's query fragments at once
      // would cost more registers than the occupancy allows: read them step by step.
      if (RT >= 3) __builtin_amdgcn_sched_barrier(0);
    }
    // Lane l holds rows 16r + 4*(l/16) + i of block column l%16: max over its real
    // rows, then across the four lane groups of the column.
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
    if (!HANDOFF && grp == 0 && jb < max_blocks) out[jb] = (jb < n_cand) ? m : -INFINITY;
    if (HANDOFF && grp == 0 && jb < n_cand) {
      const uint32_t key = order_key(m);
      st_dev(ho->mbox + (size_t)bh * max_blocks + jb, key != 0u ? key : 1u);  // 0 marks "not written"
    }
  }
  if (HANDOFF && lane == 0) st_dev(ho->flag_score + (size_t)bh * ho->score_waves + bx * kScoreWaves + wave, 1u);
}

// Host side: the argument block of the scoring work for `d`.
inline ScoreArgs score_args(const Dims& d, const void* q, const void* summ, const int32_t* seq_lens,
                            float* scores) {
  ScoreArgs a;
  a.q = (const u32x4*)q;
  a.summ = (const u32x4*)summ;
  a.seq_lens = seq_lens;
  a.scores = scores;
  a.heads = d.heads;
  a.max_blocks = d.max_blocks;
  a.rows = d.group * d.queries;
  a.window = d.window;
  a.bshift = d.bshift;
  return a;
}
inline int score_grid_x(const Dims& d, int tiles = kScoreTilesPerWave) {
  return (d.max_blocks + score_blocks_per_wg(tiles) - 1) / score_blocks_per_wg(tiles);
}

}  // namespace oasis
