"""OasisKV look-ahead sparse-attention decode step on AMD Instinct MI355X (gfx950).

One decode step of one attention layer: block scoring against min/max key
summaries, head-wise top-K, the capped-eviction transfer plan, and sparse
attention over the head-wise block table.  The work runs in the HIP kernels of
liboasis.so (C ABI in include/oasis.h); this package is its Python binding.
Every call raises if the library has not been built.
"""
from ._lib import (LIB_PATH, LayerIO, OasisDims, OasisError, PipelinedLayers,  # noqa: F401
                   PreparedPlanCopy,
                   PreparedPoolStep, PreparedStep, StageEvents,
                   StepBuffers, WorkingSet, append_token, build_plan, decode_step_pool,
                   execute_plan, fill_working_set, sparse_decode_attn_pool, window_ring_slots,
                   build_summaries, decode_step, decode_step_overlapped, dims_for,
                   exported_symbols, fetch_cap, load, make_dims, score_summaries,
                   sparse_decode_attn, sparse_decode_attn_resident, step_workspace, table_stride,
                   topk_blocks, workspace_bytes, workspace_clear, workspace_status,
                   overlapped_selects_in_launch1, decode_step_overlapped_noalloc,
                   decode_step_redoes_touched_splits)
