// Sparse decode attention over the head-wise block table on gfx950.
//
// Foreground attention of the target queries over the sparse working set:
// the resident (selected) blocks plus the local window (xllm-io review of
// OasisKV, section three: training flow step 3 and the architecture figure;
// legiblepapers.com summary).  Every KV head has its own table of logical
// block ids (xllm-io review, section four, Head-wise Mapping).
//
// The work is a gather of 8 KB per 16 tokens of the table (K and V), and on this
// part a gather finishes soonest when each wave fetches as little as possible and
// the whole table is requested at once: 16 tokens per wave and round (one
// 16-token block, two 8-token blocks, or a 16-token chunk of a larger block), four
// waves per workgroup, a workgroup per 64 tokens of a head's table (more rounds
// only when a head has over 1024 units of 16 tokens).  K is requested
// before V, so the QK product and the softmax run while V is in flight; the
// waves merge in LDS and each workgroup writes one (max, sum, unnormalised
// output) partial per query head; a second kernel merges the partials of a
// head by log-sum-exp weights (the kernel boundary, not a device-scope fence,
// makes them visible: on this multi-XCD part such a fence writes back and
// invalidates the whole L2).  K and V are read with buffer loads through a
// per-head resource whose range check turns a masked load (past the table, an
// invalid id, a block past the sequence) into zeros without a memory access.
//
// Per 16-token unit, per wave (G <= 16 query heads padded to 16 MFMA columns):
//   S^T = K (16 tokens x 128) . q^T           4 x v_mfma_f32_16x16x32_bf16
//   O^T += V^T (128 x 16 tokens) . P^T        2 x 8 x v_mfma_f32_16x16x16_bf16
// bf16 K and q multiply exactly.  Each fp32 probability p enters the PV product
// as two bf16 terms, bf16(p) and bf16(p - bf16(p)), which carry p to about 2^-17
// relative at twice the (small) cost of one bf16 product.  The token order
// inside the PV contraction is chosen so that each lane feeds the probabilities
// it computed itself (no cross-lane exchange), and the head-dim order inside an
// output tile is interleaved so that each lane feeds one element of a 16-byte V
// load it already holds.  Lane l ends up owning query head l%16 and head dims
// [32*(l/16), 32*(l/16)+32), i.e. 128 contiguous output bytes.
#include "attention_impl.h"
#include "launch.h"

namespace oasis {

// Measured at 8 x 8 heads (32K), 4 x 8 (128K), 32 x 4 with 16 query heads (32K) and
// 64 x 8 (8K-16K): 2048 keeps one 16-token unit per wave for the first two (64 and 32 heads)
// and takes 4 rounds for the 64 x 8 heads, 6-7 % faster steps there.  A split's
// record grows with the group (528 bytes per query head), so with more than 8 query
// heads per KV head a quarter of the workgroups suffice and splits run up to 8 rounds:
// the 32 x 4 heads with 16 query heads each take 8 rounds instead of 2 (step 69.5 ->
// 67.1 us at 4 rounds, 66.3-66.8 -> 65.8-66.1 us at 8; the gathering alone 36.0 ->
// 33.0 us).  Half the threshold at 4 query heads made that step slower (35.7 -> 36.3 us).
#ifndef OASIS_ATTN_MIN_WGS
#define OASIS_ATTN_MIN_WGS 2048
#endif
#ifndef OASIS_ATTN_MAX_ROUNDS
#define OASIS_ATTN_MAX_ROUNDS 4
#endif

AttnSplit attn_split(const Dims& d, int table_stride) {
  const int units = attn_units(d, table_stride);
  // Rounds per workgroup: enough that no head has more than kAttnMaxSplits partials.
  const int groups = (units + kAttnWaves - 1) / kAttnWaves;
  AttnSplit s;
  s.rounds = (groups + kAttnMaxSplits - 1) / kAttnMaxSplits;
  if (s.rounds < 1) s.rounds = 1;
  // Every split writes a record per query head that the merge reads back, so with
  // many heads fewer, longer splits save bytes, while the grid keeps at least
  // OASIS_ATTN_MIN_WGS workgroups to hide the gather's latency.
  const int64_t heads = (int64_t)d.batch * d.heads;
  const bool big_group = d.group > 8;
  const int64_t min_wgs = big_group ? OASIS_ATTN_MIN_WGS / 4 : OASIS_ATTN_MIN_WGS;
  const int max_rounds = big_group ? 2 * OASIS_ATTN_MAX_ROUNDS : OASIS_ATTN_MAX_ROUNDS;
  while (s.rounds * 2 <= max_rounds) {
    const int r = s.rounds * 2;
    const int ns = (units + kAttnWaves * r - 1) / (kAttnWaves * r);
    if (heads * ns < min_wgs) break;
    s.rounds = r;
  }
  s.num_splits = (units + kAttnWaves * s.rounds - 1) / (kAttnWaves * s.rounds);
  if (s.num_splits < 1) s.num_splits = 1;
  return s;
}

// Workspace: one record per (sequence, KV head, split, query head): the unnormalised
// output (128 floats), the running max (log2 units), the sum, and padding to 16
// bytes.  Records of one (sequence, KV head) are contiguous, so a run of sequences
// owns a contiguous slice of the workspace.
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t attn_workspace_bytes(const Dims& d, int table_stride) {
  const AttnSplit s = attn_split(d, table_stride);
  return align256((size_t)d.batch * d.heads * s.num_splits * d.group * kRec * sizeof(float));
}

// Kernels: one workgroup per (split, sequence x KV head), and one per query head.
template <int GP, bool RES, bool POOL = false>
__global__ __launch_bounds__(64 * kAttnWaves, OASIS_ATTN_MIN_WAVES) void attn_split_kernel(AttnArgs a) {
  __shared__ AttnShared<GP> sh;
  attn_split_wg<GP, RES, POOL>(blockIdx.x, blockIdx.y, sh, a);
}

constexpr int kMergeWaves = 4;
__global__ __launch_bounds__(64 * kMergeWaves) void attn_merge_kernel(const float* __restrict__ part,
                                                                      int group, int nsplit,
                                                                      float* __restrict__ out,
                                                                      float* __restrict__ lse, int n_qh) {
  __shared__ MergeShared<kMergeWaves> sh;
  if (nsplit <= kMergeWaveSplits) {  // a query head per wave
    const int bhg = merge_wave_head(blockIdx.x, threadIdx.x >> 6, kMergeWaves, group, n_qh);
    if (bhg >= 0) attn_merge_wave(bhg, part, group, nsplit, out, lse);
    return;
  }
  // Query heads of KV head h on XCD h % 8, the XCD its splits ran on when they were
  // placed by XCD (a multiple of 8 heads); otherwise in order.
  int x, head;
  xcd_item(blockIdx.x, group, gridDim.x / group, true, x, head);
  attn_merge_wg<kMergeWaves>(head * group + x, sh, part, group, nsplit, out, lse);
}

hipError_t launch_attention_split(const Dims& d, const AttnSplit& s, const void* q, const void* k,
                                  const void* v, const int32_t* table, const int32_t* table_count,
                                  int table_stride, const int32_t* seq_lens, float scale, void* ws,
                                  hipStream_t stream, bool from_resident) {
  const dim3 grid(s.num_splits, d.batch * d.heads), block(64 * kAttnWaves);
  const AttnArgs a = attn_args(d, s, q, k, v, table, table_count, table_stride, seq_lens, scale, ws);
#define OASIS_ATTN_LAUNCH(GP)                                                        \
  if (from_resident) attn_split_kernel<GP, true><<<grid, block, 0, stream>>>(a);    \
  else attn_split_kernel<GP, false><<<grid, block, 0, stream>>>(a);
  if (d.group <= 4) {
    OASIS_ATTN_LAUNCH(4)
  } else if (d.group <= 8) {
    OASIS_ATTN_LAUNCH(8)
  } else {
    OASIS_ATTN_LAUNCH(16)
  }
#undef OASIS_ATTN_LAUNCH
  return hipGetLastError();
}

hipError_t launch_attention_split_pool(const Dims& d, const AttnSplit& s, const void* q,
                                       const void* pool_k, const void* pool_v, const void* ring_k,
                                       const void* ring_v, const int32_t* resident,
                                       const int32_t* seq_lens, float scale, void* ws,
                                       hipStream_t stream) {
  const dim3 grid(s.num_splits, d.batch * d.heads), block(64 * kAttnWaves);
  AttnArgs a = attn_args(d, s, q, pool_k, pool_v, resident, nullptr, d.table_stride, seq_lens, scale, ws);
  a.ring_k = (const char*)ring_k;
  a.ring_v = (const char*)ring_v;
  if (d.group <= 4) {
    attn_split_kernel<4, true, true><<<grid, block, 0, stream>>>(a);
  } else if (d.group <= 8) {
    attn_split_kernel<8, true, true><<<grid, block, 0, stream>>>(a);
  } else {
    attn_split_kernel<16, true, true><<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_attention_merge(const Dims& d, const AttnSplit& s, float* out, float* lse,
                                  const void* ws, hipStream_t stream) {
  const int n_qh = d.batch * d.heads * d.group;
  attn_merge_kernel<<<dim3(merge_workgroups(n_qh, s.num_splits, kMergeWaves)), dim3(64 * kMergeWaves), 0,
                      stream>>>((const float*)ws, d.group, s.num_splits, out, lse, n_qh);
  return hipGetLastError();
}

hipError_t launch_attention(const Dims& d, const void* q, const void* k, const void* v,
                            const int32_t* table, const int32_t* table_count, int table_stride,
                            const int32_t* seq_lens, float scale, float* out, float* lse, void* ws,
                            hipStream_t stream, bool from_resident) {
  const AttnSplit s = attn_split(d, table_stride);
  hipError_t err = launch_attention_split(d, s, q, k, v, table, table_count, table_stride, seq_lens,
                                          scale, ws, stream, from_resident);
  if (err != hipSuccess) return err;
  return launch_attention_merge(d, s, out, lse, ws, stream);
}

}  // namespace oasis
