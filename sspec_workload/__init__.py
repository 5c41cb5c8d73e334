"""Seeded synthetic inputs for the SparseSpec attention hot path.

This package holds only input generation: random tensors, context-length
draws, the paged layout and the request-to-bucket assignment.  It contains
none of the attention, scoring or selection arithmetic, so both the CPU
oracle's tests and the HIP path's tests can take their inputs from it
without sharing any of the method.
"""

from .gen import (  # noqa: F401
    ATTN_SHAPES,
    Workload,
    assign_buckets_least_loaded,
    context_lengths,
    make_workload,
    pack_rows,
    queries_per_request,
    to_numpy_bf16,
    cycle_state,
    workload_spec,
)
