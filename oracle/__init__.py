"""CPU oracle of content-routed sparse attention -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this package.
It is independent of the GPU library (no shared code, no imports either way).

Two implementations of the same definition, written apart and pinned by the same tests:
``oracle.cpp`` (the plain C++ library liboracle.so: fp64, std::thread over rows; the one the GPU
parity tests and the CPU baseline use) and the numpy module ``oracle.routed_attention``
(re-exported here, and used for the 8-bit cache and cold-retrieval oracles).
"""
from .routed_attention import (NO_SPAN, Problem, attend, attended_positions, num_routable, round_to_bf16,
                               route_scores, routed_rows, select_spans, summaries, summary_update, widen,
                               widen_f32, window_start)
from .compare import output_errors, output_ok, score_abs_bound, selection_verdict
from . import cold_retrieval, cpp, kv_fp8, snapshot
