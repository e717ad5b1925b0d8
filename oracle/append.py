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
    "key_sketch": "unit-column basis copies coordinates (hand fixture), fp64 projection within the fp32 rounding bound, nibble round trip through oracle.unpack_int4",
    "append_tokens": "row and ctx_len bookkeeping on a toy cache: only row ctx_len[b] changes, full sequences untouched",
}
