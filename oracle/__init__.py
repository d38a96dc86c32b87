"""fp64 CPU oracle for the OasisKV look-ahead sparse-attention decode step.

Test infrastructure only: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the HIP library or its binding.
"""
from .ref import (append_token, block_attention_mass, build_plan, build_summaries, captured_attention,  # noqa: F401
                  decode_step,
                  decode_step_overlapped, execute_plan, fetch_cap, fill_working_set,
                  first_window_block, num_blocks, pool_attention, resident_table, score_blocks,
                  sparse_attention, top_overlap, topk_blocks, window_ring_slots)
