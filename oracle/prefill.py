"""CPU oracle of sparse prefill attention over host-resident K/V.  TEST
INFRASTRUCTURE ONLY (same rules as oracle.step: only the tests, the entry
point's smoke check and the benchmark's CPU-baseline leg may use it; the GPU
library shares no code with it).

Sources (pages, by title):
  [P4] "3.14M Context on 3x 3090: The Power of an Architecture That Puts KV
       Cache in Host RAM" -- section "What Needs to Stay in VRAM" (K and V
       live in host RAM, only the pooled keys stay in VRAM) and section "The
       Downside to Keep in Mind": during prefill every token of a chunk picks
       its own 2048 tokens, so fetching picks token by token would move
       almost the whole history per token; instead the history is cut into
       fixed-size chunks, each copied once into a small VRAM working buffer
       (32 MiB), all tokens are computed against it and their partial softmax
       results merged; the bytes crossing PCIe do not depend on the buffer
       size, only the number of chunks does.

Reading: a prefill call takes P query tokens of one sequence, each with its
own ascending list of selected positions (its pick, produced by the
selection stage -- an input here), and the sequence's K/V rows for all T
positions in host memory.  Query p's output is the exact softmax attention
over its listed rows -- the decode step's attention applied per query.  The
chunking and the merge of partial softmax results are how the GPU computes
that, not a change of the result, so the oracle computes the definition.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from .step import kv_gather_bytes, sparse_attention


def prefill_attention(q, k, v, idx_lists: Sequence[np.ndarray], sm_scale: float, group: int,
                      fmt: str) -> np.ndarray:
    """q [P][H_q][D], k / v [T][H_kv][D] (fp16 values, or bf16 bit patterns for
    fmt 'bf16'); idx_lists[p] ascending positions.  Returns float64
    [P][H_q][D] (zeros for an empty list)."""
    P, Hq, D = q.shape
    out = np.zeros((P, Hq, D), dtype=np.float64)
    for p in range(P):
        out[p] = sparse_attention(q[p], k, v, None, None, np.asarray(idx_lists[p]), sm_scale,
                                  group, fmt)
    return out


def chunked_transfer_bytes(T: int, n_kv: int, D: int, elem_bytes: int) -> int:
    """Host-to-GPU bytes of one prefill call with the chunk loop outside: every
    history row crosses once, whatever the chunk size."""
    return kv_gather_bytes(T, n_kv, D, elem_bytes)


def per_token_transfer_bytes(n_sel: Sequence[int], n_kv: int, D: int, elem_bytes: int) -> int:
    """Host-to-GPU bytes if every query fetched its own picks."""
    return sum(kv_gather_bytes(int(n), n_kv, D, elem_bytes) for n in n_sel)


PINS = {
    "prefill_attention": "torch fp64 SDPA of all P queries with a boolean mask built from the lists; "
                         "empty list -> zeros",
    "transfer bytes": "[P4] 4096-token chunk x 2048 picks x 12 layers x 2 KiB = 192 GiB naive; "
                      "about half an hour for 1M tokens at 26 GB/s; chunked bytes independent of "
                      "the buffer size",
}
