"""CPU oracle of the multi-query decode step (speculative verification: several
query tokens per sequence in one step).  TEST INFRASTRUCTURE ONLY (same rules
as oracle.step: only the tests, the entry point's smoke check and the
benchmark's CPU-baseline leg may use it; the GPU library shares no code with
it).

Sources (pages, by title):
  [P1] "8 agents x 250K context on two 3090s: sparse KV decode with a rank-64
       key sketch and a host-RAM tier", section "What shipped": the model is
       served with MTP-7 speculative decoding, so a decode step verifies the
       drafted tokens together with the current one; section "The mechanism"
       for the single-query method (sketch score, top-k, sinks and tail,
       exact attention).
  [P2] "vLLM's Hybrid HiSparse Triples Concurrent Requests on Million-Token
       Contexts", section "Where the tradeoffs bite": with MTP the hot
       buffers must hold the rows of every verification token at once, i.e.
       each verification token has its own pick.

Reading (the pages do not spell the multi-query step out):
  - a step carries M query tokens per sequence: the last M positions of its
    cache, which already holds them (ctx_len = T counts them);
  - query j (0-based) sits at position T - M + j and attends causally: its
    context is T_j = T - M + 1 + j tokens (positions 0 .. T_j - 1);
  - each query takes its own pick: the single-query method at context T_j --
    its own int8 query sketch (one scale per query), keys over the middle
    [S, T_j - L), top-k with the lower position first on ties, sinks [0, S)
    and tail [T_j - L, T_j), dense when T_j <= S + k + L, exact attention;
  so verification computes for every drafted token exactly what decoding the
  tokens one at a time would.  A context shorter than M leaves the first
  queries with T_j <= 0: they select nothing and their output is zero.
"""

from __future__ import annotations

from typing import List, Sequence

import numpy as np

from .step import query_sketch, select_tokens, sketch_keys, sparse_attention


def query_contexts(T: int, M: int) -> List[int]:
    """Context length seen by each of the M query tokens of a sequence of T tokens."""
    return [max(0, T - M + 1 + j) for j in range(M)]


def token_step_multi(q, basis, codes, sk_scale, k, v, ks, vs, lens: Sequence[int], *, M: int,
                     S: int, k_top: int, L: int, group: int, sm_scale: float, fmt: str,
                     seqs: Sequence[int] = None):
    """A1..A4 for M query tokens per sequence.

    q [B][M][H_q][D] fp16.  Returns (qs int8 [B][M][H_kv*R], qscale fp32 [B][M],
    idx: list over b of list over j of ascending positions, out float64
    [B][M][H_q][D]); sequences not in `seqs` are left zero / empty.
    """
    B = codes.shape[0]
    Hq, D = q.shape[2], q.shape[3]
    seqs = list(range(B)) if seqs is None else list(seqs)
    qs_all, qscale_all = query_sketch(np.asarray(q).reshape(B * M, Hq, D), basis, group)
    qs_all = qs_all.reshape(B, M, -1)
    qscale_all = qscale_all.reshape(B, M)
    idx: List[List[np.ndarray]] = [[np.zeros(0, np.int64)] * M for _ in range(B)]
    out = np.zeros((B, M, Hq, D), dtype=np.float64)
    for b in seqs:
        for j, Tj in enumerate(query_contexts(int(lens[b]), M)):
            if Tj == 0:
                continue
            keys = sketch_keys(qs_all[b, j][None], codes[b:b + 1], sk_scale[b:b + 1], [Tj],
                               S, k_top, L)[0]
            idx[b][j] = select_tokens(keys, Tj, S, k_top, L)
            out[b, j] = sparse_attention(q[b, j], k[b], v[b], None if ks is None else ks[b],
                                         None if vs is None else vs[b], idx[b][j], sm_scale,
                                         group, fmt)
    return qs_all, qscale_all, idx, out


PINS = {
    "query_contexts / token_step_multi": (
        "dense regime equals a textbook causal-masked attention in matrix form; "
        "the last query equals the single-query step at the full context; every "
        "pick lies inside its causal context with its own sinks and tail; equal "
        "queries give nested picks that differ by at most the one newly ranked "
        "position; a budget threshold crossed inside one step"),
}


# ----------------------------------------------------------------------------
# several query tokens through the host tier
# ----------------------------------------------------------------------------
# [P2] section "Where the tradeoffs bite": with multi-token verification the
# hot buffer must hold the rows of every verification token at once.
# Reading: the M pick lists of a sequence are resolved one after another with
# the same step number, each as a single-query step of the tier's policy
# (oracle.ClockTier / oracle.residency.LruTier); the rows placed for an
# earlier list are then marked used in this step, so a later list finds them
# and cannot evict them.  Positions are classified against the tier's context
# T (sinks below S, tail from T - L on, the middle in between), so a later
# query's tail positions below T - L are middle rows of the tier.


def tier_resolve_lists(tier, lists, T: int, S: int, L: int, s: int):
    """tier: a ClockTier or LruTier of one sequence; lists: ascending position
    lists, one per query token.  Returns (slot per middle pick of each list,
    hits, misses), the slots in list order."""
    out, hits, misses = [], 0, 0
    for lst in lists:
        p = np.asarray(lst, dtype=np.int64)
        mid = p[(p >= S) & (p < T - L)]
        slots, h, m = tier.step(mid, s)
        out.append(slots)
        hits += h
        misses += m
    return out, hits, misses


PINS.update({
    "tier_resolve_lists": "one list equals the single-query step; after the step every middle pick of every list is resident in the slot reported for it; a position shared by several lists is fetched at most once; with the hot buffer only just above the step's distinct rows nothing a list placed is evicted by a later one (a per-list step number would evict)",
})
