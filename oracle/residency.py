"""CPU oracle of the LRU hot buffer (HiSparse-style residency) of one sequence.
TEST INFRASTRUCTURE ONLY (same rules as oracle.step: only the tests, the
entry point's smoke check and the benchmark's CPU-baseline leg may use it; the
GPU library shares no code with it).

Source: page "vLLM's Hybrid HiSparse Triples Concurrent Requests on
Million-Token Contexts", section "Three residency states, one block pool"
(mixed residency: the tail stays on the GPU and is never evicted, older rows
live in host memory, the rows the indexer wants sit in a hot buffer; one
resolver reads resident rows in place, refreshes the LRU entry of a hot row,
and copies a missed row from pinned host memory into an LRU slot) and the
list after "What it composes with" (the default hot-buffer size per request is
twice the number of rows the indexer picks).

Reading (the page names LRU but gives no tie rules): each slot holds a
position and the step it was last used.  At step s, with the picked middle
positions in ascending order:
  1. every pick already in the buffer is a hit and its slot's last use
     becomes s;
  2. the misses need as many victims: the slots not used in step s, oldest
     last use first, an empty slot counting as older than every used one and
     equal last uses taken in slot order;
  3. the misses, in ascending position, fill the victims in ascending slot
     order (where a row lands inside the buffer is not specified; this order
     makes the placement one prefix sum), and those slots' last use becomes s.
The buffer must hold at least the picks of one step.

Residency states (same section): a request's K/V pages are either resident on
the GPU, read where they sit, or only in host memory behind a null
placeholder, their picked rows going through the hot buffer.  Full residency
maps every page, mixed residency some of them (the tail always stays), no
residency none.  PagedTier keeps the page table and sends only the picks of
unmapped pages to the hot buffer; which pages are mapped is decided between
steps by the caller (the page describes the decision as driven by memory
pressure).  Reading: a page is page_tokens consecutive positions; a mapped
page occupies one block of page_tokens rows in a pool, position p of page
p // page_tokens sitting in pool row block * page_tokens + p % page_tokens.
"""

from __future__ import annotations

from typing import Tuple

import numpy as np

EMPTY = -(1 << 40)


class LruTier:
    def __init__(self, n_slots: int, T: int):
        self.n = int(n_slots)
        self.pos = np.full(self.n, -1, dtype=np.int64)
        self.last = np.full(self.n, EMPTY, dtype=np.int64)
        self.slot_of = np.full(T, -1, dtype=np.int64)

    def step(self, picks: np.ndarray, s: int) -> Tuple[np.ndarray, int, int]:
        """picks: ascending middle positions.  Returns (slot per pick, hits, misses)."""
        picks = np.asarray(picks, dtype=np.int64)
        assert picks.size <= self.n
        slots = self.slot_of[picks].copy()
        hit = slots >= 0
        self.last[slots[hit]] = s
        miss = np.nonzero(~hit)[0]
        if miss.size:
            free = np.nonzero(self.last < s)[0]                 # not used in this step
            if free.size < miss.size:
                raise RuntimeError("the rows used in this step exceed the hot buffer")
            order = np.lexsort((free, self.last[free]))          # oldest first, then slot order
            victims = np.sort(free[order[:miss.size]])
            for i, x in zip(miss.tolist(), victims.tolist()):
                if self.pos[x] >= 0:
                    self.slot_of[self.pos[x]] = -1
                p = picks[i]
                self.pos[x] = p
                self.last[x] = s
                self.slot_of[p] = x
                slots[i] = x
        n_hit = int(hit.sum())
        return slots, n_hit, int(picks.size - n_hit)


IN_PLACE, HIT, MISS = 0, 1, 2


class PagedTier:
    """Page table over a hot buffer (LruTier or ClockTier) of one sequence."""

    def __init__(self, hot, page_tokens: int, n_pages: int):
        self.hot = hot
        self.P = int(page_tokens)
        self.block = np.full(int(n_pages), -1, dtype=np.int64)   # -1: placeholder (host only)

    def map_page(self, page: int, block: int) -> None:
        self.block[page] = block

    def unmap_page(self, page: int) -> None:
        self.block[page] = -1

    def step(self, picks: np.ndarray, s: int):
        """picks: ascending middle positions.  Returns (kind per pick, where per
        pick -- pool row if IN_PLACE, hot slot otherwise -- and the counts
        (in place, hits, misses))."""
        picks = np.asarray(picks, dtype=np.int64)
        blk = self.block[picks // self.P]
        inplace = blk >= 0
        kind = np.full(picks.size, IN_PLACE, dtype=np.int64)
        where = blk * self.P + picks % self.P
        rest = np.nonzero(~inplace)[0]
        # a pick of an unmapped page is a hit iff the hot buffer holds it
        # before the step
        hit = self.hot.slot_of[picks[rest]] >= 0
        slots, hits, misses = self.hot.step(picks[rest], s)
        where[rest] = slots
        kind[rest] = np.where(hit, HIT, MISS)
        return kind, where, (int(inplace.sum()), hits, misses)


PINS = {
    "PagedTier": "hand-traced fixture tests/golden/residency_trace.txt (in place, hits and misses "
                 "across mapping changes; full, mixed and no residency); in place + hits + misses = "
                 "picks; the hot buffer sees only the picks of unmapped pages; no mapped page equals "
                 "the hot buffer alone",
    "LruTier": "hand-traced fixture tests/golden/lru_trace.txt; hits + misses = picks; occupancy "
               "never above capacity; a slot used in the current step is never evicted; no kept "
               "unused slot is older than an evicted one; nothing is evicted while a slot is empty",
}
