"""CPU oracle of the SparseSpec attention hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  See sspec_ref.py
for what it computes and how each function is pinned.
"""

from .sspec_ref import (  # noqa: F401
    bf16_to_f64,
    draft_token_set,
    gather_kv,
    kv_append,
    kv_rollback,
    pillar_scores,
    pillar_topk,
    select_count,
    sparse_draft_attention,
    topk_lowest_index,
    unified_rows,
    unified_step,
    verify_attention,
)
