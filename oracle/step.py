"""CPU oracle for the sparse-KV decode step (score -> select -> attend, plus
the host-RAM tier).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the
package entry point and the benchmark's CPU-baseline leg may import or call
this module.  The GPU library never uses it, and this module imports nothing
from the GPU library.

Plain, slow, meant to be checked against the pages by eye: numpy, loops over
sequences and heads, fp64 for every floating-point result the pages leave
open, exact integers for the sketch scores.  The one place that works in fp32
is the query sketch, because its result is an integer code and both sides must
take that decision in the same precision.

Sources (pages, by title):
  [P1] "8 agents x 250K context on two 3090s: sparse KV decode with a rank-64
       key sketch and a host-RAM tier" -- sections "The mechanism",
       "Measured results".
  [P3] "You can offload most of Qwen3.8-Flash-Next's KV cache to RAM with
       little decode slowdown" (single section; the byte closed forms).
  [P4] "3.14M Context on 3x 3090: The Power of an Architecture That Puts KV
       Cache in Host RAM" -- sections "Why", "No Need to Rewrite the Kernel",
       "What Needs to Stay in VRAM".

Parity status per function is listed in PINS at the bottom of this file.
"""

from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------


def f16_to_f64(x) -> np.ndarray:
    """fp16 values (numpy float16, or their uint16 bit patterns) -> float64, exactly."""
    a = np.asarray(x)
    if a.dtype == np.uint16 or a.dtype == np.int16:
        a = a.view(np.float16)
    return a.astype(np.float64)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16 / int16) -> float64, exactly (bf16 is the top
    half of an fp32)."""
    u = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def unpack_int4(codes: np.ndarray) -> np.ndarray:
    """Bytes -> signed 4-bit values; element 2j is the low nibble of byte j,
    element 2j+1 the high nibble, both two's complement."""
    c = np.asarray(codes, dtype=np.uint8)
    lo = (c & 0x0F).astype(np.int16)
    hi = (c >> 4).astype(np.int16)
    lo = (lo ^ 8) - 8
    hi = (hi ^ 8) - 8
    out = np.empty(c.shape[:-1] + (2 * c.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# ----------------------------------------------------------------------------
# A1  query sketch   [P1] "The mechanism": every token is scored through a
#     rank-64 projection onto a frozen basis, one pick shared by the KV heads;
#     the query side of the int4 sketch is an int8 vector.
# ----------------------------------------------------------------------------


def query_sketch(q: np.ndarray, basis: np.ndarray, group: int) -> Tuple[np.ndarray, np.ndarray]:
    """q [B][H_q][D] fp16, basis [H_kv][D][R] fp32 (basis vector r of KV head h
    is basis[h][:, r]) -> (qs int8 [B][H_kv*R], qscale fp32 [B]).

    Reading: the G query heads of a KV head are summed (scoring is linear, so
    the shared pick of a KV head is the sum of its heads' scores); the summed
    query is projected onto the basis; all H_kv*R values of a sequence share
    one int8 scale amax/127, with round-half-even and clamping to +-127.

    Fixed fp32 evaluation order (both sides take the int8 decision in fp32):
      qbar = ((q_0 + q_1) + q_2) + ...            (fp32 adds, ascending head)
      s    = 0;  for d ascending: s = s + (qbar_d * B_dr)   (separately rounded
             fp32 multiply and add; no fused multiply-add)
      qscale = amax / 127   (fp32, correctly rounded)
      qs   = clamp(rint(s / qscale), -127, 127), or 0 when amax == 0.
    """
    q32 = np.asarray(q).astype(np.float32)
    bas = np.asarray(basis, dtype=np.float32)
    B, Hq, D = q32.shape
    Hkv, Db, R = bas.shape
    assert Db == D and Hq == Hkv * group
    qbar = np.empty((B, Hkv, D), dtype=np.float32)
    for h in range(Hkv):
        acc = q32[:, h * group, :].copy()
        for j in range(1, group):
            acc = acc + q32[:, h * group + j, :]
        qbar[:, h, :] = acc
    s = np.zeros((B, Hkv, R), dtype=np.float32)
    for d in range(D):
        prod = qbar[:, :, d][:, :, None] * bas[None, :, d, :]
        s = s + prod
    s = s.reshape(B, Hkv * R)
    amax = np.abs(s).max(axis=1)
    qscale = (amax / np.float32(127.0)).astype(np.float32)
    qs = np.zeros((B, Hkv * R), dtype=np.int8)
    for b in range(B):
        if amax[b] == 0:
            qscale[b] = np.float32(0.0)
            continue
        r = np.rint(s[b] / qscale[b])
        qs[b] = np.clip(r, -127, 127).astype(np.int8)
    return qs, qscale


# ----------------------------------------------------------------------------
# A2  sketch scores   [P1] "The mechanism": int4 sketch per token, integer
#     scores; one ranking per layer for all KV heads.
# ----------------------------------------------------------------------------


def token_candidates(T: int, S: int, k: int, L: int) -> Optional[np.ndarray]:
    """Middle positions ranked by the indexer, or None when the sequence is dense.

    [P1] "The mechanism": the kept set is the top 2048 tokens plus 64 sink
    tokens plus the last 1024.  Reading: sinks and tail are always kept and are
    not ranked; a sequence is dense (every token attended) when T <= S + k + L.
    """
    if T <= S + k + L:
        return None
    return np.arange(S, T - L, dtype=np.int64)


def sketch_keys(qs: np.ndarray, codes: np.ndarray, sk_scale: np.ndarray,
                lens: Sequence[int], S: int, k: int, L: int) -> np.ndarray:
    """Exact ranking keys of the middle tokens, float64 [B][T_max] (NaN elsewhere).

    dot_t = sum_i qs[i] * code_t[i]          (exact integer)
    key_t = dot_t * scale_t                  (exact in fp64: <= 19 + 11 significant bits)
    The per-token fp16 scale is part of the key so keys rank like q.k would; the
    common positive factor qscale is left out.  -0 is stored as +0.
    Keys are computed for every middle position [S, T-L), also for dense sequences.
    """
    B, T_max, nb = codes.shape
    keys = np.full((B, T_max), np.nan, dtype=np.float64)
    for b in range(B):
        T = int(lens[b])
        lo, hi = S, max(S, T - L)
        if hi <= lo:
            continue
        qv = qs[b].astype(np.int32)
        for c0 in range(lo, hi, 65536):
            c1 = min(hi, c0 + 65536)
            c = unpack_int4(codes[b, c0:c1]).astype(np.int32)
            dot = c @ qv
            kk = dot.astype(np.float64) * f16_to_f64(sk_scale[b, c0:c1])
            keys[b, c0:c1] = kk + 0.0
    return keys


# ----------------------------------------------------------------------------
# A2' pooled-key scores   [P4] "Why", "What Needs to Stay in VRAM"; [P3]:
#     a 128-dim bf16 indexer key per 4-token block, every block scored each step.
# ----------------------------------------------------------------------------


def pooled_keys(qi: np.ndarray, kp: np.ndarray, lens: Sequence[int]) -> np.ndarray:
    """Keys of the complete 4-token blocks, float64 [B][T_max//4] (NaN elsewhere).

    key_b = sum_i qi[i] * kp_b[i], every product and partial sum in fp64.
    Inputs are bf16 bit patterns (uint16).  With every bf16 value 0 or of
    magnitude in [2^-8, 2^8) the sum is exact, hence order-free.
    """
    qd = bf16_to_f64(qi)
    kd_all = kp
    B, NB, Di = kd_all.shape
    keys = np.full((B, NB), np.nan, dtype=np.float64)
    for b in range(B):
        nb = int(lens[b]) // 4
        if nb == 0:
            continue
        kd = bf16_to_f64(kd_all[b, :nb])
        keys[b, :nb] = np.sum(kd * qd[b][None, :], axis=1) + 0.0
    return keys


# ----------------------------------------------------------------------------
# A3  selection   [P1] "The mechanism" (deterministic top-k, one pick per layer,
#     sinks + recent tail, dense/sparse switch); [P4] "Why" (dense until the
#     context exceeds 4*block_topk+3, then exactly the budget).
# ----------------------------------------------------------------------------


def top_k_positions(keys_row: np.ndarray, cand: np.ndarray, k: int) -> np.ndarray:
    """The k candidates with the largest keys; equal keys go to the lower position."""
    kv = keys_row[cand]
    order = np.lexsort((cand, -kv))   # primary: key descending, then position ascending
    return cand[order[:k]]


def select_tokens(keys_row: np.ndarray, T: int, S: int, k: int, L: int) -> np.ndarray:
    """Token mode: ascending unique positions attended by one sequence."""
    cand = token_candidates(T, S, k, L)
    if cand is None:
        return np.arange(T, dtype=np.int64)
    top = top_k_positions(keys_row, cand, k)
    sel = np.concatenate([np.arange(S, dtype=np.int64), top,
                          np.arange(T - L, T, dtype=np.int64)])
    return np.unique(sel)


def select_blocks(keys_row: np.ndarray, T: int, k_blocks: int) -> np.ndarray:
    """Block mode: ascending token positions attended by one sequence.

    Only complete 4-token blocks have pooled keys; the trailing T mod 4 tokens
    (which include the current token) are always attended.  Dense while
    floor(T/4) <= k_blocks, i.e. T <= 4*k_blocks + 3.
    """
    nb = T // 4
    if nb <= k_blocks:
        return np.arange(T, dtype=np.int64)
    blocks = top_k_positions(keys_row, np.arange(nb, dtype=np.int64), k_blocks)
    toks = (4 * blocks[:, None] + np.arange(4)[None, :]).reshape(-1)
    sel = np.concatenate([toks, np.arange(4 * nb, T, dtype=np.int64)])
    return np.unique(sel)


# ----------------------------------------------------------------------------
# A4  exact attention over the gathered rows   [P1] "The mechanism" (exact
#     attention on the kept tokens); [P4] "No Need to Rewrite the Kernel"
#     (rows addressed as (token * n_kv_heads + kv_head) * head_dim + d).
# ----------------------------------------------------------------------------


def dequant_rows(rows: np.ndarray, scales: Optional[np.ndarray], fmt: str) -> np.ndarray:
    """Stored rows [..., D] -> float64.  fmt: 'i8' (code * fp16 row scale),
    'f16' (fp16 values), 'bf16' (bf16 bit patterns)."""
    if fmt == "i8":
        return np.asarray(rows).astype(np.float64) * f16_to_f64(scales)[..., None]
    if fmt == "f16":
        return f16_to_f64(rows)
    if fmt == "bf16":
        return bf16_to_f64(rows)
    raise ValueError(fmt)


def attention_rows(q: np.ndarray, kd: np.ndarray, vd: np.ndarray, sm_scale: float,
                   group: int) -> np.ndarray:
    """Softmax attention of one sequence's H_q query heads over n given rows.

    q [H_q][D] float64; kd, vd [n][H_kv][D] float64 (rows in the order given).
    For query head j of KV head h = j // group:
      l_t = (q_j . k_t) * sm_scale;  p_t = exp(l_t - max l);  o_j = sum p_t v_t / sum p_t.
    Returns float64 [H_q][D]; all zeros when n == 0.  No BLAS: products and
    numpy sums only, so the same rows always give the same bits.
    """
    Hq, D = q.shape
    n = kd.shape[0]
    out = np.zeros((Hq, D), dtype=np.float64)
    if n == 0:
        return out
    for j in range(Hq):
        h = j // group
        logits = np.sum(kd[:, h, :] * q[j][None, :], axis=1) * sm_scale
        m = np.max(logits)
        p = np.exp(logits - m)
        out[j] = np.sum(p[:, None] * vd[:, h, :], axis=0) / np.sum(p)
    return out


def sparse_attention(q_b, k_b, v_b, ks_b, vs_b, idx, sm_scale, group, fmt):
    """Attention of one sequence over the rows at positions idx (ascending)."""
    idx = np.asarray(idx, dtype=np.int64)
    kd = dequant_rows(k_b[idx], None if ks_b is None else ks_b[idx], fmt)
    vd = dequant_rows(v_b[idx], None if vs_b is None else vs_b[idx], fmt)
    qd = f16_to_f64(q_b) if fmt != "bf16" else bf16_to_f64(q_b)
    return attention_rows(qd, kd, vd, sm_scale, group)


def dense_attention(q_b, k_b, v_b, ks_b, vs_b, T, sm_scale, group, fmt):
    """Textbook decode attention over every position [0, T) (no selection)."""
    kd = dequant_rows(k_b[:T], None if ks_b is None else ks_b[:T], fmt)
    vd = dequant_rows(v_b[:T], None if vs_b is None else vs_b[:T], fmt)
    qd = f16_to_f64(q_b) if fmt != "bf16" else bf16_to_f64(q_b)
    return attention_rows(qd, kd, vd, sm_scale, group)


# ----------------------------------------------------------------------------
# A5  host tier   [P1] "The mechanism": int4 host copy with 64-dim groups and
#     fp16 scales (272 B per token-head) turned back into int8 rows on fetch;
#     a GPU hot buffer of 2.5% of tokens under windowed CLOCK; a token missing
#     from the buffer is fetched by itself from the pinned host copy.
# ----------------------------------------------------------------------------

HOST_GROUP = 64


def host_row_dequant(row: np.ndarray, D: int) -> Tuple[np.ndarray, np.float16]:
    """One host K (or V) row -> (int8 codes [D], fp16 row scale).

    row: uint8 [D/2 + 2*(D/64)] = int4 codes, then one fp16 scale per 64 dims.
    Reading of "dequantized back to int8 rows on fetch": the int8 row keeps
    one fp16 scale s' = fp16(gmax * 7 / 127) with gmax the largest group scale,
    and r8_i = clamp(rint((c_i * g_i) / s'), -127, 127) where g_i is the scale
    of element i's group.  Every step is one fp32 operation on exact operands
    (c*g and gmax*7 are exact in fp32), so the result is reproducible bit for
    bit; if s' == 0 the row is all zeros.
    """
    row = np.asarray(row, dtype=np.uint8)
    ng = D // HOST_GROUP
    c = unpack_int4(row[:D // 2]).astype(np.float32)
    gs = row[D // 2:D // 2 + 2 * ng].copy().view(np.float16).astype(np.float32)
    gmax = np.float32(np.max(gs))
    sp = np.float16((gmax * np.float32(7.0)) / np.float32(127.0))
    if sp == 0:
        return np.zeros(D, dtype=np.int8), np.float16(0.0)
    g_of = np.repeat(gs, HOST_GROUP)
    x = c * g_of                                   # exact in fp32
    y = x / np.float32(sp)                         # one correctly rounded fp32 divide
    r8 = np.clip(np.rint(y), -127, 127).astype(np.int8)
    return r8, sp


class ClockTier:
    """Windowed-CLOCK hot buffer of one sequence (reading of "windowed CLOCK").

    Each slot holds (position, reference bit, last step used).  At step s:
      1. every picked token already in the buffer is a hit: ref = 1, last = s;
      2. the misses are placed in ascending position order; for each, the hand
         moves over the slots from where it stopped:
           empty slot                      -> take it,
           last > s - W  (in the window)   -> skip it,
           ref == 1                        -> clear ref, move on,
           otherwise                       -> evict its token and take it;
         a taken slot gets ref = 1, last = s, and the hand stops just past it.
    W = 1 pins exactly the slots used in the current step.  The buffer must
    hold more slots than the picks of W consecutive steps, so a victim is
    always found within two sweeps of the hand.
    """

    def __init__(self, n_slots: int, T: int, window: int = 1):
        self.n = int(n_slots)
        self.W = int(window)
        self.pos = np.full(self.n, -1, dtype=np.int64)
        self.ref = np.zeros(self.n, dtype=np.int8)
        self.last = np.full(self.n, -(1 << 40), dtype=np.int64)
        self.hand = 0
        self.slot_of = np.full(T, -1, dtype=np.int64)

    def step(self, picks: np.ndarray, s: int) -> Tuple[np.ndarray, int, int]:
        """picks: ascending positions.  Returns (slot per pick, hits, misses)."""
        picks = np.asarray(picks, dtype=np.int64)
        assert self.n > picks.size
        slots = self.slot_of[picks].copy()
        hit = slots >= 0
        self.ref[slots[hit]] = 1
        self.last[slots[hit]] = s
        for i in np.nonzero(~hit)[0]:
            p = picks[i]
            moves = 0
            while True:
                moves += 1
                if moves > 2 * self.n + 1:
                    raise RuntimeError("no slot can be evicted: more slots pinned than exist")
                x = self.hand
                self.hand = (self.hand + 1) % self.n
                if self.pos[x] < 0:
                    break
                if self.last[x] > s - self.W:
                    continue
                if self.ref[x] == 1:
                    self.ref[x] = 0
                    continue
                self.slot_of[self.pos[x]] = -1
                break
            self.pos[x] = p
            self.ref[x] = 1
            self.last[x] = s
            self.slot_of[p] = x
            slots[i] = x
        n_hit = int(hit.sum())
        return slots, n_hit, int(picks.size - n_hit)


def tier_attention(q_b, records_b, res_k, res_v, res_ks, res_vs, idx, T, S, L,
                   sm_scale, group, D):
    """Attention of one sequence in the host-tier layout: sinks [0,S) and tail
    [T-L,T) come from the resident int8 rows (sinks first, then tail); middle
    positions come from their host records turned into int8 rows."""
    idx = np.asarray(idx, dtype=np.int64)
    n_kv = records_b.shape[1]
    rb = D // 2 + 2 * (D // HOST_GROUP)
    n = idx.size
    kd = np.empty((n, n_kv, D))
    vd = np.empty((n, n_kv, D))
    for r, p in enumerate(idx.tolist()):
        if p < S or p >= T - L:
            ri = p if p < S else S + (p - (T - L))
            kd[r] = dequant_rows(res_k[ri], res_ks[ri], "i8")
            vd[r] = dequant_rows(res_v[ri], res_vs[ri], "i8")
        else:
            for h in range(n_kv):
                k8, ksc = host_row_dequant(records_b[p, h, :rb], D)
                v8, vsc = host_row_dequant(records_b[p, h, rb:], D)
                kd[r, h] = k8.astype(np.float64) * np.float64(ksc)
                vd[r, h] = v8.astype(np.float64) * np.float64(vsc)
    return attention_rows(f16_to_f64(q_b), kd, vd, sm_scale, group)


def paged_tier_attention(q_b, records_b, k8_b, v8_b, ks_b, vs_b, idx, T, S, L, page_block, P,
                         sm_scale, group, D):
    """Attention of one sequence under page residency (page "vLLM's Hybrid
    HiSparse Triples Concurrent Requests on Million-Token Contexts", section
    "Three residency states, one block pool": rows of resident pages are read
    in place, the rest through the hot buffer from host memory).  Sinks
    [0,S), tail [T-L,T) and middle positions whose page p // P is mapped
    (page_block[p // P] >= 0) use the sequence's own int8 rows k8_b/v8_b
    [T][H_kv][D] with fp16 row scales ks_b/vs_b [T][H_kv]; the other middle
    positions use their host records turned into int8 rows."""
    idx = np.asarray(idx, dtype=np.int64)
    n_kv = records_b.shape[1]
    rb = D // 2 + 2 * (D // HOST_GROUP)
    page_block = np.asarray(page_block, dtype=np.int64)
    n = idx.size
    kd = np.empty((n, n_kv, D))
    vd = np.empty((n, n_kv, D))
    for r, p in enumerate(idx.tolist()):
        if p < S or p >= T - L or page_block[p // P] >= 0:
            kd[r] = dequant_rows(k8_b[p], ks_b[p], "i8")
            vd[r] = dequant_rows(v8_b[p], vs_b[p], "i8")
        else:
            for h in range(n_kv):
                k8, ksc = host_row_dequant(records_b[p, h, :rb], D)
                v8, vsc = host_row_dequant(records_b[p, h, rb:], D)
                kd[r, h] = k8.astype(np.float64) * np.float64(ksc)
                vd[r, h] = v8.astype(np.float64) * np.float64(vsc)
    return attention_rows(f16_to_f64(q_b), kd, vd, sm_scale, group)


# ----------------------------------------------------------------------------
# byte counts   [P3] closed forms; [P4] "Why", "What Needs to Stay in VRAM"
# ----------------------------------------------------------------------------


def token_scan_bytes(n_cand: int, n_kv: int, R: int) -> int:
    """Sketch bytes read to score n_cand tokens: int4 codes + one fp16 scale each."""
    return n_cand * (n_kv * R // 2 + 2)


def block_scan_bytes(n_blocks: int, index_dim: int) -> int:
    """Pooled-key bytes read to score n_blocks blocks (bf16)."""
    return n_blocks * index_dim * 2


def kv_gather_bytes(n_sel: int, n_kv: int, D: int, elem_bytes: int, row_scale_bytes: int = 0) -> int:
    """K and V bytes read for n_sel attended tokens."""
    return 2 * n_sel * n_kv * (D * elem_bytes + row_scale_bytes)


def host_record_bytes(D: int) -> int:
    """Host bytes of one token-head (K row + V row)."""
    return 2 * (D // 2 + 2 * (D // HOST_GROUP))


# ----------------------------------------------------------------------------
# whole-layer convenience wrappers (what the parity tests compare against)
# ----------------------------------------------------------------------------


def token_step(q, basis, codes, sk_scale, k, v, ks, vs, lens, *, S, k_top, L, group,
               sm_scale, fmt, seqs: Optional[Sequence[int]] = None):
    """A1..A4 for the sequences in `seqs` (all by default).

    Returns (qs, qscale, keys, list of idx per sequence, out [B][H_q][D] float64);
    entries of sequences not in `seqs` are left NaN / empty."""
    qs, qscale = query_sketch(q, basis, group)
    B = codes.shape[0]
    seqs = list(range(B)) if seqs is None else list(seqs)
    keys = np.full(codes.shape[:2], np.nan)
    sub = sketch_keys(qs[seqs], codes[seqs], sk_scale[seqs], [lens[b] for b in seqs], S, k_top, L)
    keys[seqs] = sub
    idx: List[np.ndarray] = [np.zeros(0, np.int64)] * B
    out = np.full((B,) + q.shape[1:], np.nan)
    for b in seqs:
        idx[b] = select_tokens(keys[b], int(lens[b]), S, k_top, L)
        out[b] = sparse_attention(q[b], k[b], v[b], None if ks is None else ks[b],
                                  None if vs is None else vs[b], idx[b], sm_scale, group, fmt)
    return qs, qscale, keys, idx, out


def block_step(q, qi, kp, k, v, lens, *, k_blocks, group, sm_scale,
               seqs: Optional[Sequence[int]] = None):
    """A2', A3, A4 in block mode; same return layout as token_step minus qs/qscale."""
    B = kp.shape[0]
    seqs = list(range(B)) if seqs is None else list(seqs)
    keys = np.full(kp.shape[:2], np.nan)
    keys[seqs] = pooled_keys(qi[seqs], kp[seqs], [lens[b] for b in seqs])
    idx: List[np.ndarray] = [np.zeros(0, np.int64)] * B
    out = np.full((B,) + q.shape[1:], np.nan)
    for b in seqs:
        idx[b] = select_blocks(keys[b], int(lens[b]), k_blocks)
        out[b] = sparse_attention(q[b], k[b], v[b], None, None, idx[b], sm_scale, group, "bf16")
    return keys, idx, out


# What pins each function (tests/test_oracle_pins.py):
PINS = {
    "query_sketch": "identity-basis hand example; non-unit bases whose fp32 scale bits change under a fused multiply-add, another summation order or an fp64 sum (hand-derived, tests/golden/query_sketch.txt); orthonormal round trip with a permuted Hadamard basis; exact scale invariance; fp64 projection bound",
    "sketch_keys": "hand-decoded nibble fixture, exact-rational product check, needles recovered",
    "pooled_keys": "exact rational sum (fractions) on random in-domain data, needles recovered",
    "select_tokens/select_blocks": "brute-force rank counting, all-equal keys, thresholds 400/401, 3136/3137, 2051/2052, budget constancy",
    "attention_rows": "torch fp64 scaled_dot_product_attention on the dense case, one row -> v, q=0 -> mean of v, dense == sparse bitwise",
    "host_row_dequant": "hand-worked fixture, |r8| <= 127, monotone in the code within a group",
    "ClockTier": "hand-traced fixtures with W = 1 and W = 2 (the W = 2 trace separates the window from W = 1 and from a '>=' window test), hits+misses=picks, window-pinned slots never evicted, occupancy",
    "paged_tier_attention": "one-row selections read exactly the source the page rule names (sink, tail "
                            "boundary, mapped page edges, unmapped neighbours); no mapped page equals "
                            "tier_attention and every page mapped equals sparse_attention, bit for bit",
    "tier_attention": "equal bit for bit to sparse_attention over a plain int8 cache holding the rows the host records decode to (codes derived in exact rationals); hand-worked position -> row table for sinks, the first middle row, the tail boundary T-L and the last position",
    "byte counts": "4 MiB / 48 MiB, 64 MiB, 130 B, 272 B, 27.75 / 27.00 / 0.75 KiB closed forms",
    "attention output values": "parity unpinned by the pages (they print no worked values); pinned by the library routine and special cases above",
}
