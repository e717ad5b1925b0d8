"""CPU oracle of the decode-step append: the new token of every sequence is
written into the caches the step reads.  TEST INFRASTRUCTURE ONLY (same rules
as oracle.step: only the tests, the entry point's smoke check and the
benchmark's CPU-baseline leg may use it; the GPU library shares no code with
it).

Sources (pages, by title):
  [P1] "8 agents x 250K context on two 3090s: sparse KV decode with a rank-64
       key sketch and a host-RAM tier", section "The mechanism": every token
       has a rank-64 key sketch from a frozen basis (int4 codes, one fp16 scale
       per token), K/V rows are int8 with a per-row scale.
  [P4] "3.14M Context on 3x 3090: The Power of an Architecture That Puts KV
       Cache in Host RAM", section "No Need to Rewrite the Kernel": the paged
       cache update writes the new token's rows in place each step.

The pages do not spell the encodings out; the readings used (plainest
rounding, fixed fp32 order so that the integer codes are reproducible):
  int8 row   : s = fp16( fp32(amax / 127) ), codes = clamp(rint(x / s), +-127),
               all zero when s == 0; x / s a correctly rounded fp32 quotient.
  key sketch : v[h*R + r] = sum over d ascending of (k_h[d] * B_h[d][r]) in
               fp32, each product and sum rounded separately; one scale per
               token s = fp16( fp32(amax / 7) ) over all H_kv*R values, codes
               clamp(rint(v / s), +-7) (0 when s == 0), element 2j in the low
               nibble of byte j (two's complement).
  position   : row ctx_len[b] of sequence b, then ctx_len[b] += 1; a full
               sequence (ctx_len >= max_ctx) is left as it is.
"""

from __future__ import annotations

from typing import Tuple

import numpy as np


def _fp32_quotient(a: np.ndarray, c: float) -> np.ndarray:
    """a / c correctly rounded to fp32 (computed in fp64 and rounded once)."""
    return (np.asarray(a, dtype=np.float64) / c).astype(np.float32)


def row_i8(x16: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """fp16 rows [..., D] -> (int8 codes [..., D], fp16 scale [...])."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)
    amax = np.abs(x).max(axis=-1)
    s16 = _fp32_quotient(amax, 127.0).astype(np.float16)
    s = s16.astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0))
    q = np.rint(x / safe[..., None])          # fp32 / fp32: correctly rounded
    q = np.clip(q, -127, 127)
    q = np.where(s[..., None] > 0, q, 0)
    return q.astype(np.int8), s16


def pack_int4(c: np.ndarray) -> np.ndarray:
    """int4 values [..., 2n] (int8 in [-8, 7]) -> bytes [..., n]; element 2j in
    the low nibble of byte j, element 2j+1 in the high nibble."""
    c = np.asarray(c).astype(np.int16)
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def key_sketch(k16: np.ndarray, basis: np.ndarray) -> Tuple[np.ndarray, np.float16]:
    """One token's keys k16 [H_kv][D] fp16 and the basis [H_kv][D][R] fp32 ->
    (packed int4 codes [H_kv*R/2] uint8, fp16 scale)."""
    k = np.asarray(k16, dtype=np.float16).astype(np.float32)
    bas = np.asarray(basis, dtype=np.float32)
    Hkv, D, R = bas.shape
    v = np.zeros((Hkv, R), dtype=np.float32)
    for d in range(D):
        v = v + k[:, d][:, None] * bas[:, d, :]   # fp32 product, then fp32 sum
    v = v.reshape(Hkv * R)
    amax = np.abs(v).max()
    s16 = np.float16(_fp32_quotient(amax, 7.0))
    s = np.float32(s16)
    if s == 0:
        c = np.zeros(Hkv * R, dtype=np.int8)
    else:
        c = np.clip(np.rint(v / s), -7, 7).astype(np.int8)
    return pack_int4(c), s16


def append_tokens(ctx_len, k_new, v_new, basis, caches, max_ctx, kv_format="i8"):
    """Writes the new token of every sequence; returns the new ctx_len.

    caches: dict of numpy arrays updated in place --
      'codes' uint8 [B][max_ctx][H_kv*R/2], 'sk_scale' float16 [B][max_ctx],
      'k', 'v' int8 [B][max_ctx][H_kv][D] (+ 'k_scale', 'v_scale' float16
      [B][max_ctx][H_kv]) for kv_format "i8", or float16 rows for "f16".
    k_new, v_new: float16 [B][H_kv][D]."""
    ctx = np.asarray(ctx_len, dtype=np.int64).copy()
    for b in range(ctx.size):
        t = int(ctx[b])
        if t < 0 or t >= max_ctx:
            continue
        codes, s16 = key_sketch(k_new[b], basis)
        caches["codes"][b, t] = codes
        caches["sk_scale"][b, t] = s16
        if kv_format == "i8":
            kq, ks = row_i8(k_new[b])
            vq, vs = row_i8(v_new[b])
            caches["k"][b, t], caches["k_scale"][b, t] = kq, ks
            caches["v"][b, t], caches["v_scale"][b, t] = vq, vs
        else:
            caches["k"][b, t] = np.asarray(k_new[b], dtype=np.float16)
            caches["v"][b, t] = np.asarray(v_new[b], dtype=np.float16)
        ctx[b] = t + 1
    return ctx.astype(np.int32)


PINS = {
    "row_i8": "hand-worked fixture (tests/golden/append_rows.txt), zero row, |x - s*c| <= s/2 off the clamp, amax code +-127",
    "key_sketch": "unit-column basis copies coordinates (hand fixture); non-unit bases whose fp16 scale or codes change under a fused multiply-add or another summation order (hand-derived, tests/golden/append_rows.txt); fp64 projection within the fp32 rounding bound; nibble round trip through oracle.unpack_int4",
    "append_tokens": "row and ctx_len bookkeeping on a toy cache: only row ctx_len[b] changes, full sequences untouched",
}


# ----------------------------------------------------------------------------
# block mode: bf16 K/V rows, pooled indexer key when a 4-token block completes
# ----------------------------------------------------------------------------
# Page "3.14M Context on 3x 3090 ...", sections "Why" and "What Needs to Stay
# in VRAM": the indexer key of a 4-token block is the mean of its tokens' raw
# indexer keys (compress ratio 4), stored as bf16.  Reading: the sum of the
# four bf16 raw keys is exact (fp64), divided by 4 (exact), rounded to bf16
# (nearest even), then kept in the domain the scores are exact in: 0 when its
# magnitude is below 2^-8, clamped to +-255.

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 (finite, within the fp32 exponent range) -> bf16 bit patterns,
    rounded once to nearest even: the fp64 significand is rounded to bf16's 8
    bits directly on the bit pattern, after which the conversion to fp32 and
    the truncation to the top 16 bits are exact."""
    u = np.asarray(x, dtype=np.float64).view(np.uint64)
    u = ((u + np.uint64((1 << 44) - 1) + ((u >> np.uint64(45)) & np.uint64(1))) >> np.uint64(45)) << np.uint64(45)
    f = u.view(np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def pooled_from_raw(raw4: np.ndarray) -> np.ndarray:
    """raw4: bf16 bit patterns [4][index_dim] -> pooled key bf16 bits [index_dim]."""
    from .step import bf16_to_f64
    m = bf16_to_f64(raw4).sum(axis=0) / 4.0
    y = bf16_to_f64(bf16_bits(m))
    y = np.where(np.abs(y) < 2.0 ** -8, 0.0, y)
    y = np.clip(y, -255.0, 255.0)
    return bf16_bits(y)


def append_block_tokens(ctx_len, k_new, v_new, raw_new, stage, caches, max_ctx):
    """Block mode: writes the bf16 K/V rows (bit patterns) of the new token,
    puts its raw indexer key (bf16 bits [B][index_dim]) in stage[b][t % 4] and,
    when t % 4 == 3, the pooled key of block t // 4 into caches['kp'];
    returns the new ctx_len.  stage (uint16 [B][4][index_dim]) is updated in
    place; caches: 'k', 'v' uint16 [B][max_ctx][H_kv][D], 'kp' uint16
    [B][max_ctx // 4][index_dim]."""
    ctx = np.asarray(ctx_len, dtype=np.int64).copy()
    for b in range(ctx.size):
        t = int(ctx[b])
        if t < 0 or t >= max_ctx:
            continue
        caches["k"][b, t] = k_new[b]
        caches["v"][b, t] = v_new[b]
        stage[b, t % 4] = raw_new[b]
        if t % 4 == 3:
            caches["kp"][b, t // 4] = pooled_from_raw(stage[b])
        ctx[b] = t + 1
    return ctx.astype(np.int32)


PINS.update({
    "pooled_from_raw": "hand-worked fixture (exact mean, round to even, flush below 2^-8, clamp at 255), agreement with an exact-fraction mean; rounding the mean through fp32 first gives the same bits for every in-domain input (proof in the design notes), so no fixture can separate the two",
    "append_block_tokens": "staging slot t % 4, pooled key only on t % 4 == 3, full sequences untouched",
})


# ----------------------------------------------------------------------------
# host tier: the append also writes the token's host record and moves the tail
# ----------------------------------------------------------------------------
# Page "8 agents x 250K ...", section "The mechanism": the full K/V of every
# token lives in host RAM as int4 with 64-dim groups and fp16 group scales; the
# GPU keeps the sinks and the most recent tokens (the tail) as int8 rows.
# Reading (the page gives no encoding): a group's scale is
# g = fp16( fp32(amax / 7) ) and its codes clamp(rint(x / g), +-7) (0 when
# g == 0), x / g a correctly rounded fp32 quotient; the row is the D/2 code
# bytes (element 2j in the low nibble of byte j) followed by the D/64 fp16
# group scales.  Appending position T of a sequence: its host record is the
# K row then the V row in that format, the tail loses position T - L and gains
# T as an int8 row (the int8 row rule above), the key sketch is written as in
# the plain append, and the context becomes T + 1.

HOST_GROUP = 64


def host_row_i4(x16: np.ndarray) -> np.ndarray:
    """fp16 row [D] (D a multiple of 64) -> host row bytes [D/2 + 2*(D/64)]."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)
    D = x.size
    ng = D // HOST_GROUP
    codes = np.zeros(D, dtype=np.int8)
    scales = np.zeros(ng, dtype=np.float16)
    for g in range(ng):
        xs = x[g * HOST_GROUP:(g + 1) * HOST_GROUP]
        s16 = np.float16(_fp32_quotient(np.abs(xs).max(), 7.0))
        s = np.float32(s16)
        scales[g] = s16
        if s > 0:
            codes[g * HOST_GROUP:(g + 1) * HOST_GROUP] = np.clip(np.rint(xs / s), -7, 7)
    return np.concatenate([pack_int4(codes), scales.view(np.uint8)])


def tier_append_token(T, records_b, res_k, res_v, res_ks, res_vs, S, L, k16, v16):
    """Appends position T of one sequence in the host-tier layout; returns T + 1.

    records_b: uint8 [capacity][H_kv][2 * row bytes] (K row then V row), updated
    in place; res_k / res_v int8 [S+L][H_kv][D] and res_ks / res_vs fp16
    [S+L][H_kv] hold the sinks then the tail in position order (T-L .. T-1),
    updated in place.  k16, v16: fp16 [H_kv][D]."""
    H = k16.shape[0]
    for h in range(H):
        kr, vr = host_row_i4(k16[h]), host_row_i4(v16[h])
        records_b[T, h] = np.concatenate([kr, vr])
    if L > 0:
        kq, ks = row_i8(k16)
        vq, vs = row_i8(v16)
        for a, new in ((res_k, kq), (res_v, vq), (res_ks, ks), (res_vs, vs)):
            a[S:S + L - 1] = a[S + 1:S + L].copy()
            a[S + L - 1] = new
    return T + 1


PINS.update({
    "host_row_i4": "hand-worked fixture (tests/golden/host_record_i4.txt): exact scales, ties to even, zero group, nibble order; |x - g*c| <= g/2 off the clamp; the group amax maps to +-7; decoding through oracle.host_row_dequant stays within its rounding bound",
    "tier_append_token": "tail shift on a toy layout: sinks untouched, the tail holds the last L appended rows in position order, the record of position T only; ring-free position bookkeeping",
})
