// Internal launcher interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace oasis {

// Validated problem sizes (see oasis_dims in include/oasis.h).
struct Dims {
  int batch, heads, group, max_blocks, queries, top_k, window, cap, table_stride;
  int bshift;  // log2 of the block size in tokens
};

// Attention split geometry shared by the split kernel, the merge kernel and the
// workspace layout.  The gather works in units of 16 tokens of a head's table: one
// entry of 16-token blocks, two entries of 8-token blocks, or one 16-token chunk of
// a larger block.  Workgroup s of a head takes units [4 * rounds * s,
// 4 * rounds * (s + 1)), one per wave and round.
struct AttnSplit {
  int rounds;      // units per wave
  int num_splits;  // ceil(units / (4 * rounds))
};
// Units of a table of `table_stride` entries.
inline int attn_units(const Dims& d, int table_stride) {
  return (int)(((int64_t)table_stride << d.bshift) + 15) / 16;
}
AttnSplit attn_split(const Dims& d, int table_stride);
size_t attn_workspace_bytes(const Dims& d, int table_stride);
// Workspace of the decode steps: the split records, then the hand-off region of the
// overlapped step's launch 1 (zero before the first such step; each leaves it zero).
size_t step_workspace_bytes(const Dims& d);
// Byte offset of the hand-off status word (non-zero after a wait that timed out).
size_t handoff_status_offset(const Dims& d);
// Whether the overlapped step runs its selection and plan inside launch 1 (scores
// handed over in the launch) for these sizes.
bool handoff_step_fits(const Dims& d);
// Whether oasis_decode_step can take its attention from the overlapped step's launch 1
// (redoing only the splits that the plan touched) for these sizes.
bool post_plan_reuse_fits(const Dims& d);
// Zero-fills the hand-off region of a step workspace.
hipError_t launch_clear_handoff(const Dims& d, void* ws, hipStream_t stream);
// The library's own step workspace on the current device (a device array, no
// allocation): its size, and its device address (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_build_summaries(const Dims& d, const void* k, const int32_t* seq_lens, void* summ,
                                  hipStream_t stream);
hipError_t launch_score(const Dims& d, const void* q, const void* summ, const int32_t* seq_lens,
                        float* scores, hipStream_t stream);
hipError_t launch_topk(const Dims& d, const float* scores, const int32_t* seq_lens, int32_t* topk,
                       hipStream_t stream);
hipError_t launch_plan(const Dims& d, const float* scores, const int32_t* topk,
                       const int32_t* seq_lens, int32_t* resident, int32_t* plan,
                       int32_t* plan_count, int32_t* table, int32_t* table_count,
                       hipStream_t stream);
hipError_t launch_topk_plan(const Dims& d, const float* scores, const int32_t* seq_lens,
                            int32_t* topk, const int32_t* resident, int32_t* resident_next,
                            int32_t* plan, int32_t* plan_count, int32_t* table,
                            int32_t* table_count, hipStream_t stream);
// from_resident: `table` holds the resident slots ([B*H, top_k], -1 = empty) and the
// window blocks are appended implicitly (table_count unused, table_stride = top_k +
// the most window blocks); otherwise `table` is a compacted table of table_stride
// columns with table_count valid entries.
hipError_t launch_attention_split(const Dims& d, const AttnSplit& s, const void* q, const void* k,
                                  const void* v, const int32_t* table, const int32_t* table_count,
                                  int table_stride, const int32_t* seq_lens, float scale, void* ws,
                                  hipStream_t stream, bool from_resident = false);
// The same over the working set: resident slot e read from pool slot e, window
// block j from ring slot j % (table_stride - top_k).
hipError_t launch_attention_split_pool(const Dims& d, const AttnSplit& s, const void* q,
                                       const void* pool_k, const void* pool_v, const void* ring_k,
                                       const void* ring_v, const int32_t* resident,
                                       const int32_t* seq_lens, float scale, void* ws,
                                       hipStream_t stream);
hipError_t launch_attention_merge(const Dims& d, const AttnSplit& s, float* out, float* lse,
                                  const void* ws, hipStream_t stream);
hipError_t launch_attention(const Dims& d, const void* q, const void* k, const void* v,
                            const int32_t* table, const int32_t* table_count, int table_stride,
                            const int32_t* seq_lens, float scale, float* out, float* lse, void* ws,
                            hipStream_t stream, bool from_resident = false);

// The working set in HBM: per (sequence, KV head) a pool of top_k block slots and a
// ring of WB = table_stride - top_k window block slots, each slot one block of K
// (or V) bf16.
struct WorkingSet {
  void* pool_k;
  void* pool_v;
  void* ring_k;
  void* ring_v;
};
// Gathers the working set of the slot table `resident` from the full cache k, v.
hipError_t launch_fill_working_set(const Dims& d, const int32_t* resident, const int32_t* seq_lens,
                                   const void* k, const void* v, const WorkingSet& w,
                                   hipStream_t stream);
// Copies each plan row's admitted block from the full cache into its pool slot.
hipError_t launch_execute_plan(const Dims& d, const int32_t* plan, const int32_t* plan_count,
                               const void* k, const void* v, void* pool_k, void* pool_v,
                               hipStream_t stream);
// Appends one token per sequence at position seq_lens[b]: full cache (if k is not
// NULL), ring, and the summary of its block.
hipError_t launch_append_token(const Dims& d, const void* k_new, const void* v_new,
                               const int32_t* seq_lens, void* summ, void* k, void* v,
                               void* ring_k, void* ring_v, hipStream_t stream);

// The overlapped step (attention over `resident` and the window; scoring, selection
// and plan into `resident_next`) as two fused launches on `stream`.  With `pool`, the
// attention reads the working set and (with execute_plan) a third launch then executes
// the plan, copying the admitted blocks from k, v into the pool.
hipError_t launch_overlapped_step(const Dims& d, const void* q, const void* summ, const void* k,
                                  const void* v, const int32_t* seq_lens, float* scores,
                                  int32_t* topk, const int32_t* resident, int32_t* resident_next,
                                  int32_t* plan, int32_t* plan_count, int32_t* table,
                                  int32_t* table_count, float scale, float* out, float* lse,
                                  void* ws, hipStream_t stream, hipEvent_t after_first = nullptr,
                                  const WorkingSet* pool = nullptr, bool execute_plan = true);

// The step with the attention over the updated slot table (oasis_decode_step) as the
// overlapped step's launch 1, a launch that redoes the splits holding a changed slot
// over `resident_next`, and the merge; only where post_plan_reuse_fits(d) and
// `resident_next` is its own buffer (hipErrorInvalidValue otherwise).
hipError_t launch_post_plan_step(const Dims& d, const void* q, const void* summ, const void* k,
                                 const void* v, const int32_t* seq_lens, float* scores, int32_t* topk,
                                 const int32_t* resident, int32_t* resident_next, int32_t* plan,
                                 int32_t* plan_count, int32_t* table, int32_t* table_count, float scale,
                                 float* out, float* lse, void* ws, hipStream_t stream);

// One layer's buffers for the layer-pipelined decode.
struct LayerIO {
  const void* q;
  const void* summ;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  const int32_t* resident;
  int32_t* resident_next;
  float* scores;
  int32_t* topk;
  int32_t* plan;
  int32_t* plan_count;
  int32_t* table;
  int32_t* table_count;
  float* out;
  float* lse;
  void* ws;
};
// Layer `cur`'s scoring and attention (its merge as launch 2) with the selection and
// plan of layer `prev` in the same launch 1; either may be NULL.
hipError_t launch_pipelined_layer(const Dims& d, const LayerIO* cur, const LayerIO* prev, float scale,
                                  hipStream_t stream);

}  // namespace oasis
