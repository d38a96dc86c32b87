/*
 * oasis.h -- C ABI of liboasis: one decode step of one attention layer of
 * OasisKV's look-ahead sparse attention, on AMD Instinct MI355X (gfx950).
 *
 * The step has four parts (xllm-io paper review of OasisKV, section three,
 * training flow step 3): the draft and target queries scan per-block min/max
 * key summaries, a top-K of blocks is predicted per KV head, the prediction is
 * compared with the resident set to build a capped transfer plan, and the
 * target queries attend over the resulting head-wise block table.
 *
 * Conventions for every entry point below:
 *   - Pointers named as device pointers must point to GPU memory that stays
 *     valid until the work queued on `stream` has finished; `dims` is a host
 *     pointer read during the call only.  The library keeps no pointer after
 *     it returns, allocates no memory and holds no state apart from a
 *     thread-local error string.
 *   - Tensors are dense and row-major in the layouts stated per argument.
 *     bf16 data is IEEE bfloat16 stored in 16 bits.
 *   - Work is queued on `stream` (NULL = the default stream) and is
 *     asynchronous: a status of OASIS_OK means the launches were queued.
 *     Faults inside a kernel surface at the caller's next synchronisation.
 *   - Host-side argument checks run before anything is queued.  On an error
 *     status nothing is queued and no output is touched; the reason is in
 *     oasis_last_error().
 *   - Values that live in device memory (sequence lengths, selections,
 *     resident sets, tables) cannot be checked on the host.  Their stated
 *     ranges are preconditions; out-of-range entries are skipped or treated
 *     as empty by the kernels so that no access leaves the buffers, but the
 *     results for such entries are unspecified.
 *   - Calls that write the same buffers must not run concurrently.
 *
 * Notation: B sequences, H = num_kv_heads, G = group (query heads per KV
 * head), Q = num_queries (index 0 is the target query, 1..Q-1 the drafts),
 * d = head_dim = 128, bs = block_size (16 by default; 8, 32 and 64 also),
 * NB = max_blocks, K = top_k, W = window_tokens, C = oasis_fetch_cap(),
 * T = oasis_table_stride().
 * For sequence b with length len_b (1 <= len_b <= bs * NB):
 *   nblk_b = ceil(len_b / bs)            blocks holding a token,
 *   w0_b   = max(0, floor((len_b - W) / bs))   first local-window block.
 * Blocks [0, w0_b) are the scoring candidates; blocks [w0_b, nblk_b) form the
 * local window, which is always attended and never scored or evicted.
 */
#ifndef OASIS_H_
#define OASIS_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OASIS_ABI_VERSION 3

typedef enum {
  OASIS_OK = 0,
  OASIS_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad ratio, ... */
  OASIS_ERR_UNSUPPORTED = 2,   /* valid request outside what the kernels implement */
  OASIS_ERR_WORKSPACE = 3,     /* workspace missing or smaller than oasis_workspace_bytes() */
  OASIS_ERR_HIP = 4            /* a HIP runtime call failed; text in oasis_last_error() */
} oasis_status;

/* Problem sizes of one decode step of one layer.  Host struct, read during the
 * call only.  Supported: head_dim == 128, block_size in {8, 16, 32, 64} (the
 * pages' default is 16, xllm-io review, section six), 1 <= top_k <= 1024,
 * top_k <= max_blocks <= 32768, group * num_queries <= 128, group <= 16,
 * window_tokens >= 0, 0 <= fetch_ratio <= 1. */
typedef struct {
  int32_t batch;           /* B */
  int32_t num_kv_heads;    /* H */
  int32_t group;           /* G query heads per KV head (GQA group) */
  int32_t head_dim;        /* d, must be 128 */
  int32_t block_size;      /* bs tokens per block: 8, 16, 32 or 64 */
  int32_t max_blocks;      /* NB: block stride of every per-block tensor */
  int32_t num_queries;     /* Q = 1 + drafts per query head */
  int32_t top_k;           /* K blocks selected per KV head */
  int32_t window_tokens;   /* W local-window tokens kept resident */
  double fetch_ratio;      /* cap C = floor(fetch_ratio * K) new blocks per KV head per step */
} oasis_dims;

/* Version of this ABI (OASIS_ABI_VERSION of the header the library was built with). */
int oasis_abi_version(void);

/* Static text for a status code. */
const char* oasis_status_string(oasis_status status);

/* Text of the last error raised on the calling thread ("" if none). */
const char* oasis_last_error(void);

/* The capped-eviction cap C = floor(fetch_ratio * top_k), taken in double
 * precision with a 1e-9 guard (xllm-io review, section three component table,
 * Capped Eviction Policy: fetch ratio 0.05 by default; legiblepapers.com FAQ
 * Q7).  Returns -1 if dims is invalid. */
int32_t oasis_fetch_cap(const oasis_dims* dims);

/* Row length T of the attention table: K resident slots plus the most local-
 * window blocks any length can produce, ceil(W / bs) + 1.  -1 if invalid. */
int32_t oasis_table_stride(const oasis_dims* dims);

/* Whether oasis_decode_step_overlapped runs the selection and plan inside its
 * first launch (1: launch 1 = scoring, selection and plan, attention splits;
 * launch 2 = attention merge) or after it (0: launch 2 = selection and plan with
 * the merge); see oasis_decode_step_overlapped for the limits.  -1 if dims is
 * invalid. */
int32_t oasis_overlapped_selects_in_launch1(const oasis_dims* dims);

/* 1 if oasis_decode_step, called with its own resident_next buffer, runs for these
 * dims as the first launch of oasis_decode_step_overlapped, a launch that redoes
 * the attention splits holding a slot the plan changed over the updated slot
 * table, and the merge (see oasis_decode_step): where the selection runs in that
 * first launch and the C rows of a plan can touch at most 16 of a head's
 * attention splits and at most half of them.  0 if it runs as four kernels.
 * -1 if dims is invalid. */
int32_t oasis_decode_step_redoes_touched_splits(const oasis_dims* dims);

/* Device workspace of the decode steps (oasis_decode_step, _overlapped, _pool,
 * oasis_decode_layer_pipelined), in bytes, a multiple of 256; it also serves
 * oasis_sparse_decode_attn with table_stride == oasis_table_stride(dims).  It
 * holds the per-split attention partials and, after them, the hand-off region
 * through which the scoring workgroups of the overlapped step's first launch
 * pass the scores to the selection workgroups of the same launch.
 * The hand-off region must be zero before the workspace first serves a step:
 * allocate it zero-filled or call oasis_workspace_clear once.  Every step leaves
 * it zero again, so the workspace can serve any number of steps and layers of
 * the same dims in turn (one at a time).  Before it serves steps of other dims
 * (whose regions lie elsewhere), call oasis_workspace_clear with the new dims.
 * 0 if dims is invalid. */
size_t oasis_workspace_bytes(const oasis_dims* dims);

/* Zero-fills the hand-off region of a step workspace for `dims` on `stream` (a
 * fill kernel, so the call can be captured in a graph).  Needed once after
 * allocation unless the memory is allocated zero-filled, when the workspace
 * moves to other dims, and after a step whose status word (below) is non-zero.
 * ws_bytes >= oasis_workspace_bytes(dims), else OASIS_ERR_WORKSPACE. */
oasis_status oasis_workspace_clear(const oasis_dims* dims, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* Byte offset, inside the step workspace, of the hand-off status word (uint32).
 * It stays 0 unless a selection workgroup in the first launch of
 * oasis_decode_step_overlapped waited past its bound (about 10 ms) for the
 * scores it needs (the first launch of oasis_decode_step too, in the form that
 * redoes the touched splits); it then holds bit 1, the selection outputs of
 * that step (topk, plan, table, resident_next; in that form of oasis_decode_step
 * also out and lse) are unspecified and the workspace must be cleared.  A wait never hangs the device.  0 if dims is invalid. */
size_t oasis_workspace_status_offset(const oasis_dims* dims);

/* Device workspace that oasis_sparse_decode_attn needs for a given table
 * stride, in bytes, a multiple of 256.  0 if an argument is invalid. */
size_t oasis_attn_workspace_bytes(const oasis_dims* dims, int32_t table_stride);

/* Per-block min/max key summaries ("compressed keys"): for every block j of
 * every (b, h), summ[b,h,j,0,:] = min and summ[b,h,j,1,:] = max over the valid
 * tokens t (bs*j + t < len_b) of k[b,h,j,t,:].  Blocks without a valid token
 * get zeros.  Exact (bf16 min/max).
 * xllm-io review, section three component table (Compressed Key Cache:
 * per-dimension min/max of every logical block, 1/16 of the KV size) and
 * section two (Quest-style min/max pooling).
 *   k        device, bf16 [B, H, NB, bs, 128]
 *   seq_lens device, int32 [B]
 *   summ     device, bf16 [B, H, NB, 2, 128]   (output) */
oasis_status oasis_build_summaries(const oasis_dims* dims, const void* k, const int32_t* seq_lens,
                                   void* summ, hipStream_t stream);

/* Look-ahead block scores: for every candidate block j < w0_b,
 *   scores[b,h,j] = max over g < G, i < Q of
 *                   sum_d max(q[b,h,g,i,d] * kmin[b,h,j,d], q[b,h,g,i,d] * kmax[b,h,j,d]),
 * the Quest upper bound of q.k over the block, aggregated by max over the GQA
 * group and the target and draft queries.  Blocks j >= w0_b get -inf.
 * bf16 inputs, fp32 accumulation.
 * xllm-io review, section two (the draft queries scan the compressed key
 * summary to predict next step's important blocks) and section three
 * component table (Look-ahead Attention).
 *   q        device, bf16 [B, H, G, Q, 128]
 *   summ     device, bf16 [B, H, NB, 2, 128]  (oasis_build_summaries layout)
 *   seq_lens device, int32 [B]
 *   scores   device, fp32 [B, H, NB]          (output) */
oasis_status oasis_score_summaries(const oasis_dims* dims, const void* q, const void* summ,
                                   const int32_t* seq_lens, float* scores, hipStream_t stream);

/* Head-wise top-K block selection: topk[b,h,:] lists the min(K, w0_b) best
 * candidate blocks, best first, under the order "higher fp32 score first,
 * equal scores: lower block index first" (-0.0 counts as +0.0); remaining
 * entries are -1.  Scores must not be NaN.
 * xllm-io review, section three component table (top-K = 128 blocks per head)
 * and section six (block size 16, K = 128 blocks per KV head).
 *   scores   device, fp32 [B, H, NB]
 *   seq_lens device, int32 [B]
 *   topk     device, int32 [B, H, K]          (output) */
oasis_status oasis_topk_blocks(const oasis_dims* dims, const float* scores, const int32_t* seq_lens,
                               int32_t* topk, hipStream_t stream);

/* Capped-eviction transfer plan against the resident set, and the attention
 * table.  Per (b, h), with S = topk[b,h,:] and R = resident[b,h,:]:
 *   A = entries of S not in R, in S order; n = min(C, |A|); the first n of A
 *   are admitted.  Victim slots: empty slots (-1) by ascending slot, then
 *   slots whose block is not in S by ascending score (equal scores: higher
 *   block index first); the first n are freed.  Freed slots in ascending slot
 *   order receive the admitted blocks in ascending block order.
 *   plan[b,h,r,:] = (slot, new block, old block or -1) for r < n by ascending
 *   slot, rows r >= n are -1; plan_count[b,h] = n; resident is updated in
 *   place.  table[b,h,:] = the updated resident entries in [0, w0_b) in slot
 *   order, then the window blocks w0_b .. nblk_b - 1, then -1 up to T entries;
 *   table_count[b,h] = number of entries.
 * xllm-io review, section three training flow step 3 (compare with the
 * resident set, build the transfer plan) and component table (Capped
 * Eviction Policy; Head-wise Mapping), legiblepapers.com FAQ Q7 (the cap
 * bounds newly admitted blocks at the selection stage).  The admission,
 * victim and pairing orders are this library's readings; the pages leave
 * them open.
 *   scores      device, fp32 [B, H, NB]  (ranks stale slots)
 *   topk        device, int32 [B, H, K]  (oasis_topk_blocks output)
 *   seq_lens    device, int32 [B]
 *   resident    device, int32 [B, H, K]  in/out; entries distinct, in [0, nblk_b) or -1.
 *               A resident block at or past w0_b (one the local window has reached) is
 *               not a candidate: its score is -inf, so it is the first stale slot to be
 *               freed, and while it stays it is listed once, among the window blocks.
 *   plan        device, int32 [B, H, C, 3] (output; may be NULL when C == 0)
 *   plan_count  device, int32 [B, H]       (output)
 *   table       device, int32 [B, H, T]    (output)
 *   table_count device, int32 [B, H]       (output) */
oasis_status oasis_build_plan(const oasis_dims* dims, const float* scores, const int32_t* topk,
                              const int32_t* seq_lens, int32_t* resident, int32_t* plan,
                              int32_t* plan_count, int32_t* table, int32_t* table_count,
                              hipStream_t stream);

/* Sparse decode attention of the target queries over the head-wise table:
 *   out[b,h,g,:] = sum_t softmax_t(scale * q[b,h,g,0,:] . k_t) v_t
 * over the tokens t of the blocks table[b,h,0 .. table_count[b,h]-1] whose
 * index is below len_b; lse[b,h,g] = log(sum_t exp(scale * q.k_t)).  With no
 * token, out = 0 and lse = -inf.  bf16 inputs, fp32 softmax and accumulation.
 * xllm-io review, section three training flow step 3 (foreground attention
 * over the sparse working set) and architecture figure (sparse working set
 * in HBM: selected blocks plus the local window).
 *   q            device, bf16 [B, H, G, Q, 128] (row 0 of each query head is used)
 *   k, v         device, bf16 [B, H, NB, bs, 128]
 *   table        device, int32 [B, H, table_stride]; entries distinct, in [0, NB)
 *   table_count  device, int32 [B, H], each in [0, table_stride]
 *   table_stride host, 1 <= table_stride <= 4096
 *   seq_lens     device, int32 [B]
 *   scale        host, finite
 *   out          device, fp32 [B, H, G, 128]   (output, 16-byte aligned)
 *   lse          device, fp32 [B, H, G]        (output; may be NULL)
 *   ws, ws_bytes device workspace, at least oasis_attn_workspace_bytes(dims, table_stride) */
oasis_status oasis_sparse_decode_attn(const oasis_dims* dims, const void* q, const void* k,
                                      const void* v, const int32_t* table,
                                      const int32_t* table_count, int32_t table_stride,
                                      const int32_t* seq_lens, float scale, float* out, float* lse,
                                      void* ws, size_t ws_bytes, hipStream_t stream);

/* oasis_sparse_decode_attn over the working set held as resident slots: the
 * tokens attended are those of the blocks resident[b,h,s] (s < K, -1 = empty
 * slot) that lie before the first window block w0_b, followed by the window
 * blocks w0_b .. nblk_b - 1, i.e. the same set as the table that
 * oasis_build_plan would write for this slot table (a resident block at or
 * past w0_b is attended once, as a window block).  No compacted table is
 * needed, so the attention can start from the slot table of the previous
 * step.  Same sources as oasis_sparse_decode_attn.
 *   resident     device, int32 [B, H, K]; entries distinct, or -1
 *   ws, ws_bytes device workspace, at least oasis_workspace_bytes(dims)
 *   other arguments as for oasis_sparse_decode_attn */
oasis_status oasis_sparse_decode_attn_resident(const oasis_dims* dims, const void* q, const void* k,
                                               const void* v, const int32_t* resident,
                                               const int32_t* seq_lens, float scale, float* out,
                                               float* lse, void* ws, size_t ws_bytes,
                                               hipStream_t stream);

/* The whole step on one stream: oasis_score_summaries, then the selection and
 * the plan (one kernel doing oasis_topk_blocks and oasis_build_plan), then
 * oasis_sparse_decode_attn over the updated table (table_stride =
 * oasis_table_stride(dims)).  This is the order of the xllm-io review, section
 * three, training flow step 3, read as one stream: the look-ahead prediction
 * of the top-K blocks, the comparison with the resident set that yields the
 * capped transfer plan, and attention over the working set that results.
 * Arguments as above, except:
 *   resident_next  device, int32 [B, H, K] or NULL.  NULL: `resident` is
 *                  updated in place.  Otherwise `resident` is only read and the
 *                  updated slot table is written here (a double-buffered slot
 *                  table: step t reads one buffer and writes the other); the
 *                  two buffers must not overlap.
 * The attention is the same set as oasis_sparse_decode_attn_resident over the
 * updated slot table.  With resident_next given and
 * oasis_decode_step_redoes_touched_splits(dims) == 1, the step runs as three
 * launches: the first launch of oasis_decode_step_overlapped (its attention
 * splits over `resident`, its selection and plan writing resident_next), one
 * that redoes, over resident_next, only the splits holding a slot that a plan
 * row changed (the other splits read the same blocks either way), and the
 * merge of each head's partials.  That form uses the hand-off region of the
 * workspace (zero before the first step, left zero; see
 * oasis_workspace_bytes); the results differ from the four-kernel form's only
 * in the order of the fp32 additions. */
oasis_status oasis_decode_step(const oasis_dims* dims, const void* q, const void* summ,
                               const void* k, const void* v, const int32_t* seq_lens,
                               float* scores, int32_t* topk, int32_t* resident,
                               int32_t* resident_next, int32_t* plan, int32_t* plan_count,
                               int32_t* table, int32_t* table_count, float scale, float* out,
                               float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/* The step as a foreground and a background half: while the target queries
 * attend over the blocks resident now, the look-ahead scoring, the selection
 * and the plan produce the resident set of the next step (lode.cx summary,
 * point 3: background prefetch while the GPU computes the current attention;
 * legiblepapers.com summary: foreground attention over the entries currently
 * resident, background look-ahead for future blocks; xllm-io review, section
 * three, training flow step 3).
 *   foreground: exactly oasis_sparse_decode_attn_resident(dims, q, k, v,
 *     resident, seq_lens, scale, out, lse, ws, ws_bytes).
 *   background: oasis_score_summaries, then the selection and the plan, reading
 *     `resident` and writing the next slot table to `resident_next` (and plan,
 *     table, table_count for it), as oasis_decode_step does.
 * The halves share only inputs, so their work items sit in the same grids.  Up
 * to 96 query rows (G * Q), K = 256, 2048 blocks per KV head and 256
 * (sequence, KV head) pairs, launch 1 holds the scoring
 * workgroups, one selection-and-plan workgroup per KV head that takes its
 * head's scores over from the scoring workgroups through the hand-off region of
 * the workspace (it must be zero before the first step; see
 * oasis_workspace_bytes), and the attention split workgroups; the selection
 * then runs while the attention still streams K and V.  Launch 2 is the
 * attention merge (oasis_overlapped_selects_in_launch1 tells which form runs).  Larger shapes keep the selection out of
 * launch 1: scoring with the attention's block gathering, then the selection
 * and plan with the attention's merge.
 * resident_next is required and must not overlap `resident`; the caller swaps
 * the two between steps.  Other arguments as for oasis_decode_step. */
oasis_status oasis_decode_step_overlapped(const oasis_dims* dims, const void* q, const void* summ,
                                          const void* k, const void* v, const int32_t* seq_lens,
                                          float* scores, int32_t* topk, const int32_t* resident,
                                          int32_t* resident_next, int32_t* plan,
                                          int32_t* plan_count, int32_t* table,
                                          int32_t* table_count, float scale, float* out,
                                          float* lse, void* ws, size_t ws_bytes,
                                          hipStream_t stream);

/* oasis_decode_step_overlapped without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The workspace is a 16 MiB device
 * array of the library (one copy per GPU, held from the library's load until
 * the process ends); dims whose oasis_workspace_bytes exceeds it are rejected
 * with OASIS_ERR_WORKSPACE before anything is queued.  The call queues a fill
 * kernel that clears the array's hand-off region for `dims`, then the kernels of
 * oasis_decode_step_overlapped; it allocates nothing and calls no allocating
 * routine.  All calls on one GPU share its array: calls whose work overlaps on
 * that GPU (other streams, other threads) race and their results are undefined;
 * calls ordered on one stream are safe.  Arguments and outputs as for
 * oasis_decode_step_overlapped. */
oasis_status oasis_decode_step_overlapped_noalloc(
    const oasis_dims* dims, const void* q, const void* summ, const void* k, const void* v,
    const int32_t* seq_lens, float* scores, int32_t* topk, const int32_t* resident,
    int32_t* resident_next, int32_t* plan, int32_t* plan_count, int32_t* table,
    int32_t* table_count, float scale, float* out, float* lse, hipStream_t stream);

/* oasis_decode_step_overlapped with timing markers, for measurement:
 * events[0..2] (created by the caller with hipEventCreate) are recorded on
 * `stream` before the first launch, after it, and after the second launch (the
 * attention merge, with the selection and plan when those are not in launch 1).
 * The kernels queued are the same. */
oasis_status oasis_decode_step_overlapped_timed(
    const oasis_dims* dims, const void* q, const void* summ, const void* k, const void* v,
    const int32_t* seq_lens, float* scores, int32_t* topk, const int32_t* resident,
    int32_t* resident_next, int32_t* plan, int32_t* plan_count, int32_t* table,
    int32_t* table_count, float scale, float* out, float* lse, void* ws, size_t ws_bytes,
    hipStream_t stream, hipEvent_t* events);

/* oasis_decode_step with timing markers, for measurement: events[0..4]
 * (created by the caller with hipEventCreate) are recorded on `stream` before
 * the scoring kernel, after it, after the selection-and-plan kernel, after the
 * attention split kernel and after the attention merge kernel.  The kernels
 * queued are the same as oasis_decode_step's. */
oasis_status oasis_decode_step_timed(const oasis_dims* dims, const void* q, const void* summ,
                                     const void* k, const void* v, const int32_t* seq_lens,
                                     float* scores, int32_t* topk, int32_t* resident,
                                     int32_t* resident_next, int32_t* plan, int32_t* plan_count,
                                     int32_t* table, int32_t* table_count, float scale, float* out,
                                     float* lse, void* ws, size_t ws_bytes, hipStream_t stream,
                                     hipEvent_t* events);

/* ---- Executing the plan: the working set in HBM -----------------------------
 *
 * The full K/V cache keeps its layout and place ([B, H, max_blocks, bs, 128]
 * bf16, in HBM or in pinned host memory that the device can address): that is
 * the page table, and it never changes.  HBM holds each KV head's working set:
 * a pool of K block slots, slot s holding the block the resident slot table
 * names in slot s (the head-wise logical-to-logical map), and a ring of
 * WB = oasis_window_ring_slots(dims) window blocks, window block j in ring slot
 * j % WB.  (xllm-io review, section three: component table, head-wise mapping
 * above the paged cache; training flow steps 2 and 3: the GPU keeps the
 * selected historical blocks and the local window, the plan is carried out as
 * an asynchronous transfer; section four, innovations table: only head-wise
 * mapping entries change; section five: compressed-key update and KV
 * transfer.  legiblepapers.com FAQ Q4; lode.cx points 1 and 3.)
 *   pool_k, pool_v  device, bf16 [B, H, K, bs, 128]
 *   ring_k, ring_v  device, bf16 [B, H, WB, bs, 128]
 *   k, v            the full cache, bf16 [B, H, max_blocks, bs, 128]: device
 *                   memory, or pinned host memory given by its device address
 *                   (hipHostGetDevicePointer); read (and, by append, written)
 *                   by the kernels directly.
 * Buffers are caller-owned and must be pairwise disjoint (checked on the
 * address ranges).  Errors as for the calls above. */

/* Ring slots per KV head, ceil(W / bs) + 1 (== oasis_table_stride - top_k).
 * -1 if dims is invalid. */
int32_t oasis_window_ring_slots(const oasis_dims* dims);

/* Gathers the working set of slot table `resident` ([B, H, K], -1 = empty) from
 * the full cache: pool slot s <- block resident[b,h,s] (empty slots are left as
 * they are), ring slot j % WB <- window block j for j in [first window block,
 * number of blocks) of seq_lens[b].  For admission, or to rebuild. */
oasis_status oasis_fill_working_set(const oasis_dims* dims, const int32_t* resident,
                                    const int32_t* seq_lens, const void* k, const void* v,
                                    void* pool_k, void* pool_v, void* ring_k, void* ring_v,
                                    hipStream_t stream);

/* Executes a plan of oasis_build_plan: for every row i < plan_count[b,h] of
 * plan[b,h] (slot, new, old), copies block `new` of the full cache into pool
 * slot `slot`.  The evicted block needs no transfer (the full cache keeps every
 * block).  Rows out of range are skipped.  plan may be NULL when the cap is 0. */
oasis_status oasis_execute_plan(const oasis_dims* dims, const int32_t* plan,
                                const int32_t* plan_count, const void* k, const void* v,
                                void* pool_k, void* pool_v, hipStream_t stream);

/* Appends one decoded token per sequence at position L = seq_lens[b]:
 *   k_new, v_new  device, bf16 [B, H, 128]
 *   k, v          the full cache (both NULL: not written)
 *   ring_k/v      token L % bs of ring slot (L / bs) % WB
 *   summ          the summary of block L / bs: the new key itself when L % bs
 *                 == 0 (the token opens the block), else the elementwise min
 *                 and max with the summary so far (exact in bf16).
 * seq_lens is not changed: the caller counts the token in afterwards.  A
 * sequence with L >= bs * max_blocks has no room and is skipped. */
oasis_status oasis_append_token(const oasis_dims* dims, const void* k_new, const void* v_new,
                                const int32_t* seq_lens, void* summ, void* k, void* v,
                                void* ring_k, void* ring_v, hipStream_t stream);

/* oasis_sparse_decode_attn_resident over the working set: resident slot s is
 * read from pool slot s, window block j from ring slot j % WB.  Equal to the
 * full-cache form when the working set holds the slot table's blocks. */
oasis_status oasis_sparse_decode_attn_pool(const oasis_dims* dims, const void* q, const void* pool_k,
                                           const void* pool_v, const void* ring_k,
                                           const void* ring_v, const int32_t* resident,
                                           const int32_t* seq_lens, float scale, float* out,
                                           float* lse, void* ws, size_t ws_bytes,
                                           hipStream_t stream);

/* oasis_decode_step_overlapped with the foreground attention over the working
 * set (oasis_sparse_decode_attn_pool), followed by oasis_execute_plan of the
 * plan just built, copying the admitted blocks from the full cache k, v into
 * the pool: after the call the pool holds resident_next's blocks.  Three
 * launches on `stream`; the copies start after the attention has read the
 * pool.  Other arguments as for oasis_decode_step_overlapped. */
oasis_status oasis_decode_step_pool(const oasis_dims* dims, const void* q, const void* summ,
                                    const void* k, const void* v, void* pool_k, void* pool_v,
                                    const void* ring_k, const void* ring_v,
                                    const int32_t* seq_lens, float* scores, int32_t* topk,
                                    const int32_t* resident, int32_t* resident_next,
                                    int32_t* plan, int32_t* plan_count, int32_t* table,
                                    int32_t* table_count, float scale, float* out, float* lse,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/* oasis_decode_step_pool with the plan's copies on a background stream, for a
 * layer-pipelined decode (xllm-io review, section three: component table,
 * asynchronous pipeline of per-layer background workers on their own streams;
 * section five: stream events order the work of each layer; Eq. (4)): the two
 * launches of the step go to `stream`, `plan_ready` (a caller-created event) is
 * recorded on it after them, and `transfer_stream` waits for that event and then
 * runs the copies.  The caller must make the next reader of the pool (this
 * layer's next step) wait for `transfer_stream`, and must not overwrite `plan`
 * and `plan_count` before the copies have run (per-layer buffers).
 * transfer_stream must differ from stream.  Other arguments as for
 * oasis_decode_step_pool. */
oasis_status oasis_decode_step_pool_async(
    const oasis_dims* dims, const void* q, const void* summ, const void* k, const void* v,
    void* pool_k, void* pool_v, const void* ring_k, const void* ring_v, const int32_t* seq_lens,
    float* scores, int32_t* topk, const int32_t* resident, int32_t* resident_next, int32_t* plan,
    int32_t* plan_count, int32_t* table, int32_t* table_count, float scale, float* out, float* lse,
    void* ws, size_t ws_bytes, hipStream_t stream, hipStream_t transfer_stream,
    hipEvent_t plan_ready);

/* ---- Layer-pipelined decode ---------------------------------------------------
 *
 * The pages run each layer's background half (look-ahead scoring, selection, plan)
 * beside the foreground of the layers after it (xllm-io review, section three:
 * component table, asynchronous pipeline, parallel across layers and serial within
 * a layer; Eq. (4)).  Here a layer's scoring goes with its own foreground
 * attention (launch 1); its launch 2 is the attention merge, the output the next
 * layer needs.  Up to the one-launch limits of oasis_decode_step_overlapped the
 * layer's selection and plan run inside its own launch 1, fed by the hand-off
 * region; above them they ride in the next layer's launch 1 (or, for the
 * largest shapes, its launch 2).  One layer's buffers: */
typedef struct {
  const void* q;            /* device, bf16 [B, H, G, Q, 128] (row 0 target) */
  const void* summ;         /* device, bf16 [B, H, NB, 2, 128] */
  const void* k;            /* device, bf16 [B, H, NB, bs, 128] */
  const void* v;            /* device, bf16 [B, H, NB, bs, 128] */
  const int32_t* seq_lens;  /* device, int32 [B] */
  const int32_t* resident;  /* device, int32 [B, H, K]: the slot table attended now */
  int32_t* resident_next;   /* device, int32 [B, H, K]: the next slot table (own buffer) */
  float* scores;            /* device, fp32 [B, H, NB] */
  int32_t* topk;            /* device, int32 [B, H, K] */
  int32_t* plan;            /* device, int32 [B, H, C, 3] (NULL allowed when C = 0) */
  int32_t* plan_count;      /* device, int32 [B, H] */
  int32_t* table;           /* device, int32 [B, H, oasis_table_stride] */
  int32_t* table_count;     /* device, int32 [B, H] */
  float* out;               /* device, fp32 [B, H, G, 128] */
  float* lse;               /* device, fp32 [B, H, G] or NULL */
  void* ws;                 /* device workspace of oasis_workspace_bytes(dims) */
  size_t ws_bytes;
} oasis_layer_io;

/* Queues, on `stream`: `layer`'s foreground (attention of its target queries over
 * `resident` and the window into out, lse) and its look-ahead scoring (scores),
 * and `previous`'s selection and plan (topk, plan, plan_count, table, table_count,
 * resident_next from previous->scores, previous->seq_lens, previous->resident), as
 * oasis_decode_step_overlapped computes them for each layer.  Call it for every
 * layer in order with the layer before as `previous` (for the first layer, the
 * last layer of the step before, or NULL), and once more with layer = NULL and
 * previous = the last layer to finish the sweep.  Either argument may be NULL,
 * not both.  The two must not share scores buffers (one is written while the
 * other is read), and each resident_next must be its own buffer; a layer's
 * selection outputs are valid after the next call returns its launches to the
 * stream order (within the one-launch limits, as soon as this call's own
 * launches are done; `previous` then has nothing left to run and the final call
 * with layer = NULL queues nothing).  Calls ordered on one stream may all pass
 * the same workspace: a call reads back its split records within its own
 * launches and leaves the hand-off region zero. */
oasis_status oasis_decode_layer_pipelined(const oasis_dims* dims, const oasis_layer_io* layer,
                                          const oasis_layer_io* previous, float scale,
                                          hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* OASIS_H_ */
