"""CPU oracle of content-routed sparse attention -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this package.
It is independent of the GPU library (no shared code, no imports either way).
"""
from .routed_attention import (NO_SPAN, Problem, attend, attended_positions, num_routable, round_to_bf16,
                               route_scores, routed_rows, select_spans, summaries, summary_update, widen,
                               widen_f32, window_start)
from .compare import output_errors, output_ok, score_abs_bound, selection_verdict
from . import cold_retrieval, kv_fp8, snapshot
