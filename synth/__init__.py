"""Seeded synthetic inputs for the sparse-KV decode step.

This package draws data in the storage formats the step consumes (fp16 /
bf16 queries, int4 key sketches with per-token fp16 scales, int8 K/V rows
with per-row fp16 scales, mean-pooled bf16 indexer keys, int4 host records,
drifting pick schedules).  It contains no part of the step itself: no query
sketch, no scoring, no selection, no attention and no tier policy.  Both the
CPU oracle's tests and the GPU path's tests and benchmark take their inputs
from here.
"""

from .gen import (  # noqa: F401
    CHUNK,
    TokenCase,
    BlockCase,
    TierCase,
    make_token_case,
    make_block_case,
    make_tier_case,
    tier_page_rows,
    drift_picks,
    draft_picks,
    multi_queries,
    prefill_picks,
    orthonormal_basis,
    pack_int4,
    flush_bf16_domain,
)
