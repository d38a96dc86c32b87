// C ABI of liboasis: host-side argument checks and launches (see include/oasis.h).
#include "oasis.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.h"
#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

oasis_status fail(oasis_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

oasis_status hip_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return OASIS_OK;
  return fail(OASIS_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

// Checks `in` and fills `out`.  Returns OASIS_OK or the error (text set).
oasis_status check_dims(const oasis_dims* in, oasis::Dims* out) {
  using namespace oasis;
  // Launch errors are read back with hipGetLastError; drop an error left by an
  // earlier, unrelated HIP call of the caller so that it is not reported as ours.
  (void)hipGetLastError();
  if (in == nullptr) return fail(OASIS_ERR_INVALID_ARG, "dims is NULL");
  if (in->head_dim != kHeadDim)
    return fail(OASIS_ERR_UNSUPPORTED, "head_dim %d: only %d is implemented", in->head_dim, kHeadDim);
  int bshift = -1;
  for (int sh = kMinBlockShift; sh <= kMaxBlockShift; ++sh)
    if (in->block_size == (1 << sh)) bshift = sh;
  if (bshift < 0)
    return fail(OASIS_ERR_UNSUPPORTED, "block_size %d: only 8, 16, 32 and 64 are implemented",
                in->block_size);
  if (in->batch < 1 || in->num_kv_heads < 1 || in->group < 1 || in->num_queries < 1)
    return fail(OASIS_ERR_INVALID_ARG, "batch, num_kv_heads, group and num_queries must be >= 1");
  if (in->max_blocks < 1) return fail(OASIS_ERR_INVALID_ARG, "max_blocks must be >= 1");
  if (in->top_k < 1) return fail(OASIS_ERR_INVALID_ARG, "top_k must be >= 1");
  if (in->top_k > in->max_blocks)
    return fail(OASIS_ERR_INVALID_ARG, "top_k %d exceeds max_blocks %d", in->top_k, in->max_blocks);
  if (in->window_tokens < 0) return fail(OASIS_ERR_INVALID_ARG, "window_tokens must be >= 0");
  if (!(in->fetch_ratio >= 0.0 && in->fetch_ratio <= 1.0))
    return fail(OASIS_ERR_INVALID_ARG, "fetch_ratio must lie in [0, 1]");
  if (in->max_blocks > kMaxBlocks)
    return fail(OASIS_ERR_UNSUPPORTED, "max_blocks %d exceeds %d", in->max_blocks, kMaxBlocks);
  if (in->top_k > kMaxTopK) return fail(OASIS_ERR_UNSUPPORTED, "top_k %d exceeds %d", in->top_k, kMaxTopK);
  if ((int64_t)in->group * in->num_queries > kMaxRows)
    return fail(OASIS_ERR_UNSUPPORTED, "group * num_queries exceeds %d", kMaxRows);
  if (in->group > kMaxGroup) return fail(OASIS_ERR_UNSUPPORTED, "group %d exceeds %d", in->group, kMaxGroup);
  if ((int64_t)in->batch * in->num_kv_heads > 65535)
    return fail(OASIS_ERR_UNSUPPORTED, "batch * num_kv_heads exceeds 65535");
  if (in->window_tokens > (kMaxBlocks << bshift))
    return fail(OASIS_ERR_UNSUPPORTED, "window_tokens exceeds %d", kMaxBlocks << bshift);
  out->batch = in->batch;
  out->heads = in->num_kv_heads;
  out->group = in->group;
  out->max_blocks = in->max_blocks;
  out->queries = in->num_queries;
  out->top_k = in->top_k;
  out->window = in->window_tokens;
  out->cap = (int)floor(in->fetch_ratio * (double)in->top_k + 1e-9);
  out->table_stride = in->top_k + num_blocks(in->window_tokens, bshift) + 1;
  out->bshift = bshift;
  return OASIS_OK;
}

#define OASIS_REQUIRE(ptr)                                                      \
  do {                                                                          \
    if ((ptr) == nullptr) return fail(OASIS_ERR_INVALID_ARG, "%s is NULL", #ptr); \
  } while (0)

oasis_status check_table_stride(const oasis::Dims& d, int32_t table_stride) {
  if (table_stride < 1 || table_stride > oasis::kMaxTableStride)
    return fail(OASIS_ERR_INVALID_ARG, "table_stride %d outside [1, %d]", table_stride,
                oasis::kMaxTableStride);
  (void)d;
  return OASIS_OK;
}

}  // namespace

extern "C" {

int oasis_abi_version(void) { return OASIS_ABI_VERSION; }

const char* oasis_status_string(oasis_status status) {
  switch (status) {
    case OASIS_OK: return "ok";
    case OASIS_ERR_INVALID_ARG: return "invalid argument";
    case OASIS_ERR_UNSUPPORTED: return "unsupported";
    case OASIS_ERR_WORKSPACE: return "workspace too small";
    case OASIS_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* oasis_last_error(void) { return g_last_error; }

int32_t oasis_fetch_cap(const oasis_dims* dims) {
  oasis::Dims d;
  if (check_dims(dims, &d) != OASIS_OK) return -1;
  return d.cap;
}

int32_t oasis_table_stride(const oasis_dims* dims) {
  oasis::Dims d;
  if (check_dims(dims, &d) != OASIS_OK) return -1;
  return d.table_stride;
}

int32_t oasis_overlapped_selects_in_launch1(const oasis_dims* dims) {
  oasis::Dims d;
  if (check_dims(dims, &d) != OASIS_OK) return -1;
  return oasis::handoff_step_fits(d) ? 1 : 0;
}

int32_t oasis_decode_step_redoes_touched_splits(const oasis_dims* dims) {
  oasis::Dims d;
  if (check_dims(dims, &d) != OASIS_OK) return -1;
  return oasis::post_plan_reuse_fits(d) ? 1 : 0;
}

size_t oasis_workspace_bytes(const oasis_dims* dims) {
  oasis::Dims d;
  if (check_dims(dims, &d) != OASIS_OK) return 0;
  return oasis::step_workspace_bytes(d);
}

size_t oasis_workspace_status_offset(const oasis_dims* dims) {
  oasis::Dims d;
  if (check_dims(dims, &d) != OASIS_OK) return 0;
  return oasis::handoff_status_offset(d);
}

oasis_status oasis_workspace_clear(const oasis_dims* dims, void* ws, size_t ws_bytes, hipStream_t stream) {
  oasis::Dims d;
  oasis_status st = check_dims(dims, &d);
  if (st != OASIS_OK) return st;
  const size_t need = oasis::step_workspace_bytes(d);
  if (ws == nullptr || ws_bytes < need)
    return fail(OASIS_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                ws == nullptr ? (size_t)0 : ws_bytes);
  return hip_status(oasis::launch_clear_handoff(d, ws, stream), "workspace_clear");
}

size_t oasis_attn_workspace_bytes(const oasis_dims* dims, int32_t table_stride) {
  oasis::Dims d;
  if (check_dims(dims, &d) != OASIS_OK) return 0;
  if (check_table_stride(d, table_stride) != OASIS_OK) return 0;
  return oasis::attn_workspace_bytes(d, table_stride);
}

oasis_status oasis_build_summaries(const oasis_dims* dims, const void* k, const int32_t* seq_lens,
                                   void* summ, hipStream_t stream) {
  oasis::Dims d;
  oasis_status st = check_dims(dims, &d);
  if (st != OASIS_OK) return st;
  OASIS_REQUIRE(k);
  OASIS_REQUIRE(seq_lens);
  OASIS_REQUIRE(summ);
  return hip_status(oasis::launch_build_summaries(d, k, seq_lens, summ, stream), "build_summaries");
}

oasis_status oasis_score_summaries(const oasis_dims* dims, const void* q, const void* summ,
                                   const int32_t* seq_lens, float* scores, hipStream_t stream) {
  oasis::Dims d;
  oasis_status st = check_dims(dims, &d);
  if (st != OASIS_OK) return st;
  OASIS_REQUIRE(q);
  OASIS_REQUIRE(summ);
  OASIS_REQUIRE(seq_lens);
  OASIS_REQUIRE(scores);
  return hip_status(oasis::launch_score(d, q, summ, seq_lens, scores, stream), "score_summaries");
}

oasis_status oasis_topk_blocks(const oasis_dims* dims, const float* scores, const int32_t* seq_lens,
                               int32_t* topk, hipStream_t stream) {
  oasis::Dims d;
  oasis_status st = check_dims(dims, &d);
  if (st != OASIS_OK) return st;
  OASIS_REQUIRE(scores);
  OASIS_REQUIRE(seq_lens);
  OASIS_REQUIRE(topk);
  return hip_status(oasis::launch_topk(d, scores, seq_lens, topk, stream), "topk_blocks");
}

oasis_status oasis_build_plan(const oasis_dims* dims, const float* scores, const int32_t* topk,
                              const int32_t* seq_lens, int32_t* resident, int32_t* plan,
                              int32_t* plan_count, int32_t* table, int32_t* table_count,
                              hipStream_t stream) {
  oasis::Dims d;
  oasis_status st = check_dims(dims, &d);
  if (st != OASIS_OK) return st;
  OASIS_REQUIRE(scores);
  OASIS_REQUIRE(topk);
  OASIS_REQUIRE(seq_lens);
  OASIS_REQUIRE(resident);
  if (d.cap > 0) OASIS_REQUIRE(plan);
  OASIS_REQUIRE(plan_count);
  OASIS_REQUIRE(table);
  OASIS_REQUIRE(table_count);
  return hip_status(oasis::launch_plan(d, scores, topk, seq_lens, resident, plan, plan_count, table,
                                       table_count, stream),
                    "build_plan");
}

oasis_status oasis_sparse_decode_attn(const oasis_dims* dims, const void* q, const void* k,
                                      const void* v, const int32_t* table,
                                      const int32_t* table_count, int32_t table_stride,
                                      const int32_t* seq_lens, float scale, float* out, float* lse,
                                      void* ws, size_t ws_bytes, hipStream_t stream) {
  oasis::Dims d;
  oasis_status st = check_dims(dims, &d);
  if (st != OASIS_OK) return st;
  OASIS_REQUIRE(q);
  OASIS_REQUIRE(k);
  OASIS_REQUIRE(v);
  OASIS_REQUIRE(table);
  OASIS_REQUIRE(table_count);
  OASIS_REQUIRE(seq_lens);
  OASIS_REQUIRE(out);
  st = check_table_stride(d, table_stride);
  if (st != OASIS_OK) return st;
  if (!isfinite(scale)) return fail(OASIS_ERR_INVALID_ARG, "scale must be finite");
  const size_t need = oasis::attn_workspace_bytes(d, table_stride);
  if (ws == nullptr || ws_bytes < need)
    return fail(OASIS_ERR_WORKSPACE, "attention needs %zu workspace bytes, got %zu", need,
                ws == nullptr ? (size_t)0 : ws_bytes);
  return hip_status(oasis::launch_attention(d, q, k, v, table, table_count, table_stride, seq_lens,
                                            scale, out, lse, ws, stream),
                    "sparse_decode_attn");
}

oasis_status oasis_sparse_decode_attn_resident(const oasis_dims* dims, const void* q, const void* k,
                                               const void* v, const int32_t* resident,
                                               const int32_t* seq_lens, float scale, float* out,
                                               float* lse, void* ws, size_t ws_bytes,
                                               hipStream_t stream) {
  oasis::Dims d;
  oasis_status st = check_dims(dims, &d);
  if (st != OASIS_OK) return st;
  OASIS_REQUIRE(q);
  OASIS_REQUIRE(k);
  OASIS_REQUIRE(v);
  OASIS_REQUIRE(resident);
  OASIS_REQUIRE(seq_lens);
  OASIS_REQUIRE(out);
  if (!isfinite(scale)) return fail(OASIS_ERR_INVALID_ARG, "scale must be finite");
  const size_t need = oasis::attn_workspace_bytes(d, d.table_stride);
  if (ws == nullptr || ws_bytes < need)
    return fail(OASIS_ERR_WORKSPACE, "attention needs %zu workspace bytes, got %zu", need,
                ws == nullptr ? (size_t)0 : ws_bytes);
  return hip_status(oasis::launch_attention(d, q, k, v, resident, nullptr, d.table_stride, seq_lens,
                                            scale, out, lse, ws, stream, true),
                    "sparse_decode_attn_resident");
}

// Argument checks shared by the fused-step entry points.  On success `d` is filled
// and *resident_next is resolved (NULL or equal to `resident`: in place).
static oasis_status check_step_args(const oasis_dims* dims, oasis::Dims& d, const void* q,
                                    const void* summ, const void* k, const void* v,
                                    const int32_t* seq_lens, const float* scores,
                                    const int32_t* topk, const int32_t* resident,
                                    int32_t** resident_next, const int32_t* plan,
                                    const int32_t* plan_count, const int32_t* table,
                                    const int32_t* table_count, float scale, const float* out,
                                    const void* ws, size_t ws_bytes) {
  oasis_status st = check_dims(dims, &d);
  if (st != OASIS_OK) return st;
  OASIS_REQUIRE(q);
  OASIS_REQUIRE(summ);
  OASIS_REQUIRE(k);
  OASIS_REQUIRE(v);
  OASIS_REQUIRE(seq_lens);
  OASIS_REQUIRE(scores);
  OASIS_REQUIRE(topk);
  OASIS_REQUIRE(resident);
  if (d.cap > 0) OASIS_REQUIRE(plan);
  OASIS_REQUIRE(plan_count);
  OASIS_REQUIRE(table);
  OASIS_REQUIRE(table_count);
  OASIS_REQUIRE(out);
  if (!isfinite(scale)) return fail(OASIS_ERR_INVALID_ARG, "scale must be finite");
  const size_t need = oasis::step_workspace_bytes(d);
  if (ws == nullptr || ws_bytes < need)
    return fail(OASIS_ERR_WORKSPACE, "decode step needs %zu workspace bytes, got %zu", need,
                ws == nullptr ? (size_t)0 : ws_bytes);
  if (*resident_next != nullptr && *resident_next != resident) {
    const size_t n = (size_t)d.batch * d.heads * d.top_k;
    if (*resident_next < resident + n && resident < *resident_next + n)
      return fail(OASIS_ERR_INVALID_ARG, "resident and resident_next overlap");
  } else {
    *resident_next = const_cast<int32_t*>(resident);
  }
  return OASIS_OK;
}

// The step in order: scoring, selection and plan, then the attention over the updated
// slot table.  Untimed, with a separate resident_next and sizes whose selection fits
// launch 1, it is the overlapped step's launch 1, a launch that redoes only the splits
// the plan touched, and the merge; otherwise four kernels, and with `events` non-NULL
// markers are recorded between them.
static oasis_status decode_step_impl(const oasis_dims* dims, const void* q, const void* summ,
                                     const void* k, const void* v, const int32_t* seq_lens,
                                     float* scores, int32_t* topk, int32_t* resident,
                                     int32_t* resident_next, int32_t* plan, int32_t* plan_count,
                                     int32_t* table, int32_t* table_count, float scale, float* out,
                                     float* lse, void* ws, size_t ws_bytes, hipStream_t stream,
                                     hipEvent_t* events) {
  oasis::Dims d;
  oasis_status st = check_step_args(dims, d, q, summ, k, v, seq_lens, scores, topk, resident,
                                    &resident_next, plan, plan_count, table, table_count, scale,
                                    out, ws, ws_bytes);
  if (st != OASIS_OK) return st;
  if (events == nullptr && resident_next != resident && oasis::post_plan_reuse_fits(d))
    return hip_status(oasis::launch_post_plan_step(d, q, summ, k, v, seq_lens, scores, topk, resident,
                                                   resident_next, plan, plan_count, table, table_count,
                                                   scale, out, lse, ws, stream),
                      "decode_step");
  if (events != nullptr) {
    for (int i = 0; i < 5; ++i) OASIS_REQUIRE(events[i]);
  }
  auto mark = [&](int i) -> oasis_status {
    if (events == nullptr) return OASIS_OK;
    return hip_status(hipEventRecord(events[i], stream), "decode_step/event");
  };
  if ((st = mark(0)) != OASIS_OK) return st;
  st = hip_status(oasis::launch_score(d, q, summ, seq_lens, scores, stream), "decode_step/score");
  if (st != OASIS_OK || (st = mark(1)) != OASIS_OK) return st;
  st = hip_status(oasis::launch_topk_plan(d, scores, seq_lens, topk, resident, resident_next, plan,
                                          plan_count, table, table_count, stream),
                  "decode_step/select");
  if (st != OASIS_OK || (st = mark(2)) != OASIS_OK) return st;
  const oasis::AttnSplit split = oasis::attn_split(d, d.table_stride);
  st = hip_status(oasis::launch_attention_split(d, split, q, k, v, table, table_count,
                                                d.table_stride, seq_lens, scale, ws, stream),
                  "decode_step/attention");
  if (st != OASIS_OK || (st = mark(3)) != OASIS_OK) return st;
  st = hip_status(oasis::launch_attention_merge(d, split, out, lse, ws, stream),
                  "decode_step/attention-merge");
  if (st != OASIS_OK) return st;
  return mark(4);
}

static oasis_status decode_step_overlapped_impl(
    const oasis_dims* dims, const void* q, const void* summ, const void* k, const void* v,
    const int32_t* seq_lens, float* scores, int32_t* topk, const int32_t* resident,
    int32_t* resident_next, int32_t* plan, int32_t* plan_count, int32_t* table,
    int32_t* table_count, float scale, float* out, float* lse, void* ws, size_t ws_bytes,
    hipStream_t stream, hipEvent_t* events) {
  oasis::Dims d;
  OASIS_REQUIRE(resident_next);
  oasis_status st = check_step_args(dims, d, q, summ, k, v, seq_lens, scores, topk, resident,
                                    &resident_next, plan, plan_count, table, table_count, scale,
                                    out, ws, ws_bytes);
  if (st != OASIS_OK) return st;
  if (resident_next == resident)
    return fail(OASIS_ERR_INVALID_ARG,
                "resident_next must be its own buffer: the attention reads resident meanwhile");
  if (events != nullptr) {
    for (int i = 0; i < 3; ++i) OASIS_REQUIRE(events[i]);
    if ((st = hip_status(hipEventRecord(events[0], stream), "decode_step_overlapped/event")) != OASIS_OK)
      return st;
  }
  st = hip_status(oasis::launch_overlapped_step(d, q, summ, k, v, seq_lens, scores, topk, resident,
                                                resident_next, plan, plan_count, table, table_count,
                                                scale, out, lse, ws, stream,
                                                events == nullptr ? nullptr : events[1]),
                  "decode_step_overlapped");
  if (st != OASIS_OK || events == nullptr) return st;
  return hip_status(hipEventRecord(events[2], stream), "decode_step_overlapped/event");
}

oasis_status oasis_decode_step_overlapped(const oasis_dims* dims, const void* q, const void* summ,
                                          const void* k, const void* v, const int32_t* seq_lens,
                                          float* scores, int32_t* topk, const int32_t* resident,
                                          int32_t* resident_next, int32_t* plan,
                                          int32_t* plan_count, int32_t* table,
                                          int32_t* table_count, float scale, float* out,
                                          float* lse, void* ws, size_t ws_bytes,
                                          hipStream_t stream) {
  return decode_step_overlapped_impl(dims, q, summ, k, v, seq_lens, scores, topk, resident,
                                     resident_next, plan, plan_count, table, table_count, scale,
                                     out, lse, ws, ws_bytes, stream, nullptr);
}

oasis_status oasis_decode_step_overlapped_noalloc(
    const oasis_dims* dims, const void* q, const void* summ, const void* k, const void* v,
    const int32_t* seq_lens, float* scores, int32_t* topk, const int32_t* resident,
    int32_t* resident_next, int32_t* plan, int32_t* plan_count, int32_t* table,
    int32_t* table_count, float scale, float* out, float* lse, hipStream_t stream) {
  oasis::Dims d;
  oasis_status st = check_dims(dims, &d);
  if (st != OASIS_OK) return st;
  const size_t need = oasis::step_workspace_bytes(d), have = oasis::noalloc_scratch_bytes();
  if (need > have)
    return fail(OASIS_ERR_WORKSPACE,
                "decode_step_overlapped_noalloc: these dims need %zu workspace bytes, the library's "
                "scratch array holds %zu; use oasis_decode_step_overlapped with a workspace",
                need, have);
  void* ws = nullptr;
  if ((st = hip_status(oasis::noalloc_scratch(&ws), "decode_step_overlapped_noalloc/scratch")) != OASIS_OK)
    return st;
  // Every argument checked before anything is queued.
  int32_t* rn = resident_next;
  OASIS_REQUIRE(resident_next);
  if ((st = check_step_args(dims, d, q, summ, k, v, seq_lens, scores, topk, resident, &rn, plan,
                            plan_count, table, table_count, scale, out, ws, have)) != OASIS_OK)
    return st;
  if (resident_next == resident)
    return fail(OASIS_ERR_INVALID_ARG,
                "resident_next must be its own buffer: the attention reads resident meanwhile");
  // The array keeps whatever the last call on this device left (other dims, or a step
  // whose wait timed out): its hand-off region is cleared for these dims first.
  if ((st = hip_status(oasis::launch_clear_handoff(d, ws, stream), "decode_step_overlapped_noalloc/clear")) !=
      OASIS_OK)
    return st;
  return decode_step_overlapped_impl(dims, q, summ, k, v, seq_lens, scores, topk, resident,
                                     resident_next, plan, plan_count, table, table_count, scale,
                                     out, lse, ws, have, stream, nullptr);
}

oasis_status oasis_decode_step_overlapped_timed(
    const oasis_dims* dims, const void* q, const void* summ, const void* k, const void* v,
    const int32_t* seq_lens, float* scores, int32_t* topk, const int32_t* resident,
    int32_t* resident_next, int32_t* plan, int32_t* plan_count, int32_t* table,
    int32_t* table_count, float scale, float* out, float* lse, void* ws, size_t ws_bytes,
    hipStream_t stream, hipEvent_t* events) {
  OASIS_REQUIRE(events);
  return decode_step_overlapped_impl(dims, q, summ, k, v, seq_lens, scores, topk, resident,
                                     resident_next, plan, plan_count, table, table_count, scale,
                                     out, lse, ws, ws_bytes, stream, events);
}

oasis_status oasis_decode_step(const oasis_dims* dims, const void* q, const void* summ,
                               const void* k, const void* v, const int32_t* seq_lens,
                               float* scores, int32_t* topk, int32_t* resident,
                               int32_t* resident_next, int32_t* plan, int32_t* plan_count,
                               int32_t* table, int32_t* table_count, float scale, float* out,
                               float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_step_impl(dims, q, summ, k, v, seq_lens, scores, topk, resident, resident_next, plan,
                          plan_count, table, table_count, scale, out, lse, ws, ws_bytes, stream,
                          nullptr);
}

oasis_status oasis_decode_step_timed(const oasis_dims* dims, const void* q, const void* summ,
                                     const void* k, const void* v, const int32_t* seq_lens,
                                     float* scores, int32_t* topk, int32_t* resident,
                                     int32_t* resident_next, int32_t* plan, int32_t* plan_count,
                                     int32_t* table, int32_t* table_count, float scale, float* out,
                                     float* lse, void* ws, size_t ws_bytes, hipStream_t stream,
                                     hipEvent_t* events) {
  if (events == nullptr) return fail(OASIS_ERR_INVALID_ARG, "events is NULL");
  return decode_step_impl(dims, q, summ, k, v, seq_lens, scores, topk, resident, resident_next, plan,
                          plan_count, table, table_count, scale, out, lse, ws, ws_bytes, stream,
                          events);
}

}  // extern "C"

// ---- the working set in HBM -------------------------------------------------------

namespace {

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const char* x = (const char*)a;
  const char* y = (const char*)b;
  return x < y + nb && y < x + na;
}

// Pool, ring and (if given) full-cache buffers must be pairwise disjoint.
oasis_status check_working_set(const oasis::Dims& d, const void* k, const void* v,
                               const void* pool_k, const void* pool_v, const void* ring_k,
                               const void* ring_v) {
  const size_t blk = ((size_t)oasis::kHeadDim * 2) << d.bshift;
  const size_t heads = (size_t)d.batch * d.heads;
  const size_t full = heads * d.max_blocks * blk, pool = heads * d.top_k * blk;
  const size_t ring = heads * (size_t)(d.table_stride - d.top_k) * blk;
  const struct {
    const void* p;
    size_t n;
    const char* name;
  } bufs[] = {{k, full, "k"},           {v, full, "v"},           {pool_k, pool, "pool_k"},
              {pool_v, pool, "pool_v"}, {ring_k, ring, "ring_k"}, {ring_v, ring, "ring_v"}};
  for (int i = 0; i < 6; ++i)
    for (int j = i + 1; j < 6; ++j)
      if (bufs[i].p != nullptr && bufs[j].p != nullptr &&
          ranges_overlap(bufs[i].p, bufs[i].n, bufs[j].p, bufs[j].n))
        return fail(OASIS_ERR_INVALID_ARG, "%s and %s overlap", bufs[i].name, bufs[j].name);
  return OASIS_OK;
}

}  // namespace

int32_t oasis_window_ring_slots(const oasis_dims* dims) {
  oasis::Dims d;
  if (check_dims(dims, &d) != OASIS_OK) return -1;
  return d.table_stride - d.top_k;
}

oasis_status oasis_fill_working_set(const oasis_dims* dims, const int32_t* resident,
                                    const int32_t* seq_lens, const void* k, const void* v,
                                    void* pool_k, void* pool_v, void* ring_k, void* ring_v,
                                    hipStream_t stream) {
  oasis::Dims d;
  oasis_status st = check_dims(dims, &d);
  if (st != OASIS_OK) return st;
  OASIS_REQUIRE(resident);
  OASIS_REQUIRE(seq_lens);
  OASIS_REQUIRE(k);
  OASIS_REQUIRE(v);
  OASIS_REQUIRE(pool_k);
  OASIS_REQUIRE(pool_v);
  OASIS_REQUIRE(ring_k);
  OASIS_REQUIRE(ring_v);
  if ((st = check_working_set(d, k, v, pool_k, pool_v, ring_k, ring_v)) != OASIS_OK) return st;
  const oasis::WorkingSet w{pool_k, pool_v, ring_k, ring_v};
  return hip_status(oasis::launch_fill_working_set(d, resident, seq_lens, k, v, w, stream),
                    "fill_working_set");
}

oasis_status oasis_execute_plan(const oasis_dims* dims, const int32_t* plan,
                                const int32_t* plan_count, const void* k, const void* v,
                                void* pool_k, void* pool_v, hipStream_t stream) {
  oasis::Dims d;
  oasis_status st = check_dims(dims, &d);
  if (st != OASIS_OK) return st;
  if (d.cap > 0) OASIS_REQUIRE(plan);
  OASIS_REQUIRE(plan_count);
  OASIS_REQUIRE(k);
  OASIS_REQUIRE(v);
  OASIS_REQUIRE(pool_k);
  OASIS_REQUIRE(pool_v);
  if ((st = check_working_set(d, k, v, pool_k, pool_v, nullptr, nullptr)) != OASIS_OK) return st;
  return hip_status(oasis::launch_execute_plan(d, plan, plan_count, k, v, pool_k, pool_v, stream),
                    "execute_plan");
}

oasis_status oasis_append_token(const oasis_dims* dims, const void* k_new, const void* v_new,
                                const int32_t* seq_lens, void* summ, void* k, void* v,
                                void* ring_k, void* ring_v, hipStream_t stream) {
  oasis::Dims d;
  oasis_status st = check_dims(dims, &d);
  if (st != OASIS_OK) return st;
  OASIS_REQUIRE(k_new);
  OASIS_REQUIRE(v_new);
  OASIS_REQUIRE(seq_lens);
  OASIS_REQUIRE(summ);
  OASIS_REQUIRE(ring_k);
  OASIS_REQUIRE(ring_v);
  if ((k == nullptr) != (v == nullptr))
    return fail(OASIS_ERR_INVALID_ARG, "k and v must both be given or both be NULL");
  if ((st = check_working_set(d, k, v, nullptr, nullptr, ring_k, ring_v)) != OASIS_OK) return st;
  return hip_status(oasis::launch_append_token(d, k_new, v_new, seq_lens, summ, k, v, ring_k, ring_v,
                                               stream),
                    "append_token");
}

oasis_status oasis_sparse_decode_attn_pool(const oasis_dims* dims, const void* q, const void* pool_k,
                                           const void* pool_v, const void* ring_k,
                                           const void* ring_v, const int32_t* resident,
                                           const int32_t* seq_lens, float scale, float* out,
                                           float* lse, void* ws, size_t ws_bytes,
                                           hipStream_t stream) {
  oasis::Dims d;
  oasis_status st = check_dims(dims, &d);
  if (st != OASIS_OK) return st;
  OASIS_REQUIRE(q);
  OASIS_REQUIRE(pool_k);
  OASIS_REQUIRE(pool_v);
  OASIS_REQUIRE(ring_k);
  OASIS_REQUIRE(ring_v);
  OASIS_REQUIRE(resident);
  OASIS_REQUIRE(seq_lens);
  OASIS_REQUIRE(out);
  if (!isfinite(scale)) return fail(OASIS_ERR_INVALID_ARG, "scale must be finite");
  const size_t need = oasis::attn_workspace_bytes(d, d.table_stride);
  if (ws == nullptr || ws_bytes < need)
    return fail(OASIS_ERR_WORKSPACE, "attention needs %zu workspace bytes, got %zu", need,
                ws == nullptr ? (size_t)0 : ws_bytes);
  const oasis::AttnSplit split = oasis::attn_split(d, d.table_stride);
  st = hip_status(oasis::launch_attention_split_pool(d, split, q, pool_k, pool_v, ring_k, ring_v,
                                                     resident, seq_lens, scale, ws, stream),
                  "sparse_decode_attn_pool");
  if (st != OASIS_OK) return st;
  return hip_status(oasis::launch_attention_merge(d, split, out, lse, ws, stream),
                    "sparse_decode_attn_pool/merge");
}

static oasis_status decode_step_pool_impl(
    const oasis_dims* dims, const void* q, const void* summ, const void* k, const void* v,
    void* pool_k, void* pool_v, const void* ring_k, const void* ring_v, const int32_t* seq_lens,
    float* scores, int32_t* topk, const int32_t* resident, int32_t* resident_next, int32_t* plan,
    int32_t* plan_count, int32_t* table, int32_t* table_count, float scale, float* out, float* lse,
    void* ws, size_t ws_bytes, hipStream_t stream, bool async, hipStream_t transfer_stream,
    hipEvent_t plan_ready) {
  oasis::Dims d;
  OASIS_REQUIRE(resident_next);
  oasis_status st = check_step_args(dims, d, q, summ, k, v, seq_lens, scores, topk, resident,
                                    &resident_next, plan, plan_count, table, table_count, scale,
                                    out, ws, ws_bytes);
  if (st != OASIS_OK) return st;
  if (resident_next == resident)
    return fail(OASIS_ERR_INVALID_ARG,
                "resident_next must be its own buffer: the attention reads resident meanwhile");
  OASIS_REQUIRE(pool_k);
  OASIS_REQUIRE(pool_v);
  OASIS_REQUIRE(ring_k);
  OASIS_REQUIRE(ring_v);
  if ((st = check_working_set(d, k, v, pool_k, pool_v, ring_k, ring_v)) != OASIS_OK) return st;
  if (async) {
    OASIS_REQUIRE(plan_ready);
    if (transfer_stream == stream)
      return fail(OASIS_ERR_INVALID_ARG, "transfer_stream must differ from stream");
  }
  const oasis::WorkingSet w{pool_k, pool_v, const_cast<void*>(ring_k), const_cast<void*>(ring_v)};
  st = hip_status(oasis::launch_overlapped_step(d, q, summ, k, v, seq_lens, scores, topk, resident,
                                                resident_next, plan, plan_count, table, table_count,
                                                scale, out, lse, ws, stream, nullptr, &w, !async),
                  "decode_step_pool");
  if (st != OASIS_OK || !async) return st;
  // The copies wait for the plan on the transfer stream; the caller orders the next
  // read of the pool after them.
  if ((st = hip_status(hipEventRecord(plan_ready, stream), "decode_step_pool_async/event")) != OASIS_OK)
    return st;
  if ((st = hip_status(hipStreamWaitEvent(transfer_stream, plan_ready, 0),
                       "decode_step_pool_async/wait")) != OASIS_OK)
    return st;
  return hip_status(oasis::launch_execute_plan(d, plan, plan_count, k, v, pool_k, pool_v,
                                               transfer_stream),
                    "decode_step_pool_async/execute_plan");
}

oasis_status oasis_decode_step_pool(const oasis_dims* dims, const void* q, const void* summ,
                                    const void* k, const void* v, void* pool_k, void* pool_v,
                                    const void* ring_k, const void* ring_v,
                                    const int32_t* seq_lens, float* scores, int32_t* topk,
                                    const int32_t* resident, int32_t* resident_next,
                                    int32_t* plan, int32_t* plan_count, int32_t* table,
                                    int32_t* table_count, float scale, float* out, float* lse,
                                    void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_step_pool_impl(dims, q, summ, k, v, pool_k, pool_v, ring_k, ring_v, seq_lens, scores,
                               topk, resident, resident_next, plan, plan_count, table, table_count,
                               scale, out, lse, ws, ws_bytes, stream, false, nullptr, nullptr);
}

oasis_status oasis_decode_step_pool_async(
    const oasis_dims* dims, const void* q, const void* summ, const void* k, const void* v,
    void* pool_k, void* pool_v, const void* ring_k, const void* ring_v, const int32_t* seq_lens,
    float* scores, int32_t* topk, const int32_t* resident, int32_t* resident_next, int32_t* plan,
    int32_t* plan_count, int32_t* table, int32_t* table_count, float scale, float* out, float* lse,
    void* ws, size_t ws_bytes, hipStream_t stream, hipStream_t transfer_stream,
    hipEvent_t plan_ready) {
  return decode_step_pool_impl(dims, q, summ, k, v, pool_k, pool_v, ring_k, ring_v, seq_lens, scores,
                               topk, resident, resident_next, plan, plan_count, table, table_count,
                               scale, out, lse, ws, ws_bytes, stream, true, transfer_stream,
                               plan_ready);
}

// ---- layer-pipelined decode ----------------------------------------------------------

oasis_status oasis_decode_layer_pipelined(const oasis_dims* dims, const oasis_layer_io* layer,
                                          const oasis_layer_io* previous, float scale,
                                          hipStream_t stream) {
  oasis::Dims d;
  oasis_status st = check_dims(dims, &d);
  if (st != OASIS_OK) return st;
  if (layer == nullptr && previous == nullptr)
    return fail(OASIS_ERR_INVALID_ARG, "layer and previous are both NULL");
  if (layer != nullptr) {
    OASIS_REQUIRE(layer->q);
    OASIS_REQUIRE(layer->summ);
    OASIS_REQUIRE(layer->k);
    OASIS_REQUIRE(layer->v);
    OASIS_REQUIRE(layer->seq_lens);
    OASIS_REQUIRE(layer->resident);
    OASIS_REQUIRE(layer->scores);
    OASIS_REQUIRE(layer->out);
    if (!isfinite(scale)) return fail(OASIS_ERR_INVALID_ARG, "scale must be finite");
    const size_t need = oasis::step_workspace_bytes(d);
    if (layer->ws == nullptr || layer->ws_bytes < need)
      return fail(OASIS_ERR_WORKSPACE, "layer needs %zu workspace bytes, got %zu", need,
                  layer->ws == nullptr ? (size_t)0 : layer->ws_bytes);
  }
  if (previous != nullptr) {
    OASIS_REQUIRE(previous->scores);
    OASIS_REQUIRE(previous->seq_lens);
    OASIS_REQUIRE(previous->resident);
    OASIS_REQUIRE(previous->resident_next);
    OASIS_REQUIRE(previous->topk);
    if (d.cap > 0) OASIS_REQUIRE(previous->plan);
    OASIS_REQUIRE(previous->plan_count);
    OASIS_REQUIRE(previous->table);
    OASIS_REQUIRE(previous->table_count);
    const size_t n = (size_t)d.batch * d.heads * d.top_k;
    if (previous->resident_next < previous->resident + n && previous->resident < previous->resident_next + n)
      return fail(OASIS_ERR_INVALID_ARG, "previous->resident and previous->resident_next overlap");
    if (layer != nullptr) {
      const size_t nsc = (size_t)d.batch * d.heads * d.max_blocks;
      if (previous->scores < layer->scores + nsc && layer->scores < previous->scores + nsc)
        return fail(OASIS_ERR_INVALID_ARG, "layer and previous share scores");
      if (previous->resident_next < layer->resident + n && layer->resident < previous->resident_next + n)
        return fail(OASIS_ERR_INVALID_ARG, "previous->resident_next overlaps the slot table layer attends");
    }
  }
  oasis::LayerIO cur{}, prev{};
  if (layer != nullptr)
    cur = oasis::LayerIO{layer->q, layer->summ, layer->k, layer->v, layer->seq_lens, layer->resident,
                         layer->resident_next, layer->scores, layer->topk, layer->plan,
                         layer->plan_count, layer->table, layer->table_count, layer->out,
                         layer->lse, layer->ws};
  if (previous != nullptr)
    prev = oasis::LayerIO{previous->q, previous->summ, previous->k, previous->v, previous->seq_lens,
                          previous->resident, previous->resident_next, previous->scores,
                          previous->topk, previous->plan, previous->plan_count, previous->table,
                          previous->table_count, previous->out, previous->lse, previous->ws};
  return hip_status(oasis::launch_pipelined_layer(d, layer ? &cur : nullptr, previous ? &prev : nullptr,
                                                  scale, stream),
                    "decode_layer_pipelined");
}
