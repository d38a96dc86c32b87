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
#include "score_impl.h"

namespace oasis {

template <int RT>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a) {
  __shared__ ScoreShared<RT> sh;
  score_wg<RT>(blockIdx.x, blockIdx.y, sh, a);
}

hipError_t launch_score(const Dims& d, const void* q, const void* summ, const int32_t* seq_lens,
                        float* scores, hipStream_t stream) {
  const int rows = d.group * d.queries;
  const dim3 grid(score_grid_x(d), d.batch * d.heads);
  const dim3 block(64 * kScoreWaves);
  const ScoreArgs a = score_args(d, q, summ, seq_lens, scores);
  switch ((rows + 15) / 16) {
#define OASIS_SCORE_CASE(RT)                                 \
  case RT:                                                   \
    score_kernel<RT><<<grid, block, 0, stream>>>(a);         \
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
