"""fp64 CPU oracle for the OasisKV look-ahead sparse-attention decode step.

Test infrastructure only: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the HIP library or its binding.
"""
from .ref import (build_plan, build_summaries, decode_step, decode_step_overlapped,  # noqa: F401
                  fetch_cap, first_window_block, num_blocks, resident_table, score_blocks,
                  sparse_attention, topk_blocks)
