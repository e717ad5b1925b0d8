"""Seeded generators for every input of the sparse-KV decode step.

Workload shapes follow the pages' descriptions (rank-64 int4 key sketch per
token, int8 K/V rows with fp16 scales, 4 KV heads x 256 dims, 2048-token
budget with 64 sinks and a 1024-token tail; QSA layers with 2 KV heads x 256
dims of bf16 K/V and one 128-dim bf16 pooled indexer key per 4-token block;
a host tier of int4 records of 272 B per token-head).  Values are Gaussian;
the pages' real documents and model keys are not available, so seeded
Gaussian data with planted "needle" keys stands in for them.

Determinism: each bulk tensor is drawn in fixed chunks of CHUNK tokens, each
chunk from its own torch.Generator seeded from (seed, tensor id, sequence,
chunk).  The same seed and device therefore always give the same bytes, and a
case with a shorter buffer is a prefix of a longer one.  Small tensors
(queries, basis, needle positions, lengths, pick schedules) are always drawn
on the CPU so they do not depend on the device.

Encodings applied here (int8 rows, int4 sketch codes, pooled keys, int4 host
records) are the storage formats the step reads, produced by plain rounding;
they are not steps of the decode path, which only reads them.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

CHUNK = 8192  # tokens per generator chunk (multiple of 4)
_MUL = 1_000_003

# tensor ids for sub-seeding
_T_Q, _T_BASIS, _T_SKETCH, _T_K, _T_V, _T_NEEDLE = 1, 2, 3, 4, 5, 6
_T_QI, _T_RAWIDX, _T_HK, _T_HV, _T_RK, _T_RV, _T_DRIFT, _T_LEN = 7, 8, 9, 10, 11, 12, 13, 14
_T_MQ = 15
_T_PICKS = 16
_T_DRAFT = 17


def _subseed(seed: int, *ids: int) -> int:
    s = int(seed)
    for i in ids:
        s = (s * _MUL + int(i) + 1) % (1 << 62)
    return s


def _gen(device, seed: int, *ids: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_subseed(seed, *ids))
    return g


def _chunks(T_max: int):
    for c0 in range(0, T_max, CHUNK):
        yield c0 // CHUNK, c0, min(CHUNK, T_max - c0)


def _randn(device, seed, ids, shape):
    return torch.randn(shape, generator=_gen(device, seed, *ids), device=device,
                       dtype=torch.float32)


# ----------------------------------------------------------------------------
# storage encodings (plain rounding; used only to produce inputs)
# ----------------------------------------------------------------------------

def _rows_to_i8(x: torch.Tensor):
    """float rows [..., D] -> int8 codes and one fp16 scale per row (amax/127)."""
    amax = x.abs().amax(dim=-1)
    scale = (amax / 127.0).to(torch.float16)
    sc = scale.to(torch.float32)
    safe = torch.where(sc > 0, sc, torch.ones_like(sc))
    r = torch.round(x / safe.unsqueeze(-1)).clamp_(-127, 127)
    r = torch.where(sc.unsqueeze(-1) > 0, r, torch.zeros_like(r))
    return r.to(torch.int8), scale


def _vec_to_i4(x: torch.Tensor):
    """float vectors [..., n] -> int4 codes in [-7, 7] (as int8) and one fp16 scale (amax/7)."""
    amax = x.abs().amax(dim=-1)
    scale = (amax / 7.0).to(torch.float16)
    sc = scale.to(torch.float32)
    safe = torch.where(sc > 0, sc, torch.ones_like(sc))
    c = torch.round(x / safe.unsqueeze(-1)).clamp_(-7, 7)
    c = torch.where(sc.unsqueeze(-1) > 0, c, torch.zeros_like(c))
    return c.to(torch.int8), scale


def pack_int4(c: torch.Tensor) -> torch.Tensor:
    """int4 values (int8 tensor, last dim even) -> bytes; element 2j in the low
    nibble of byte j, element 2j+1 in the high nibble, two's complement."""
    c16 = c.to(torch.int16)
    lo = c16[..., 0::2] & 0xF
    hi = c16[..., 1::2] & 0xF
    return (lo | (hi << 4)).to(torch.uint8)


def flush_bf16_domain(x: torch.Tensor) -> torch.Tensor:
    """Round to bf16 and keep every value 0 or of magnitude in [2^-8, 2^8).

    In that domain a 128-term dot product of bf16 values is an exact multiple
    of 2^-30 below 2^53 in magnitude, so fp64 accumulation is exact in any
    order; the pooled-key scores are then bit-reproducible."""
    y = x.to(torch.bfloat16).to(torch.float32)
    y = torch.where(y.abs() < 2.0 ** -8, torch.zeros_like(y), y)
    y = y.clamp(-255.0, 255.0)
    return y.to(torch.bfloat16)


def orthonormal_basis(n_kv: int, D: int, R: int, seed: int) -> torch.Tensor:
    """Seeded random orthonormal basis [n_kv][D][R] fp32 (basis vector r of KV
    head h is column [h][:, r]); QR of a Gaussian matrix computed on the CPU in
    fp64.  It stands in for the frozen rank-64 eigenbasis of real post-RoPE
    keys, which is not available."""
    g = _gen("cpu", seed, _T_BASIS)
    a = torch.randn((n_kv, D, R), generator=g, dtype=torch.float64)
    out = torch.empty((n_kv, D, R), dtype=torch.float64)
    for h in range(n_kv):
        qm, rm = torch.linalg.qr(a[h])
        # fix the sign convention so the result does not depend on LAPACK's choice
        sgn = torch.sign(torch.diagonal(rm))
        sgn[sgn == 0] = 1
        out[h] = qm * sgn
    return out.to(torch.float32)


def _lengths(B, T_max, ctx_len):
    if ctx_len is None:
        return [T_max] * B
    lens = [int(x) for x in ctx_len]
    assert len(lens) == B and all(0 <= t <= T_max for t in lens)
    return lens


def mixed_lengths(B: int, lo: int, hi: int, seed: int) -> List[int]:
    """Sequence lengths drawn uniformly from the integers in [lo, hi]."""
    g = _gen("cpu", seed, _T_LEN)
    return torch.randint(lo, hi + 1, (B,), generator=g).tolist()


def multi_queries(B: int, M: int, n_q: int, D: int, seed: int, device="cpu") -> torch.Tensor:
    """Queries of M tokens per sequence (a verification step): N(0, 1) -> fp16
    [B][M][n_q][D]."""
    return _randn("cpu", seed, (_T_MQ,), (B, M, n_q, D)).to(torch.float16).to(device)


def prefill_picks(P: int, T: int, k_blocks: int, seed: int):
    """Selections of P prefill tokens at positions T-P .. T-1 (block mode): query
    p (context T_p = T-P+1+p) takes k_blocks distinct complete blocks drawn
    uniformly from [0, T_p // 4) -- all of them while there are at most
    k_blocks -- expanded to 4 tokens each, plus the tokens of its partial
    block.  Returns (idx int32 [P][4*k_blocks+3], n_sel int32 [P])."""
    g = np.random.default_rng(_subseed(seed, _T_PICKS))
    cap = 4 * k_blocks + 3
    idx = np.zeros((P, cap), dtype=np.int32)
    n_sel = np.zeros(P, dtype=np.int32)
    for p in range(P):
        Tp = T - P + 1 + p
        nb = Tp // 4
        if nb <= k_blocks:
            blocks = np.arange(nb)
        else:
            blocks = np.unique(g.integers(0, nb, size=k_blocks + k_blocks // 4 + 16))
            while blocks.size < k_blocks:
                blocks = np.unique(np.concatenate([blocks, g.integers(0, nb, size=k_blocks)]))
            blocks = np.sort(g.permutation(blocks)[:k_blocks])
        toks = (4 * blocks[:, None] + np.arange(4)[None, :]).reshape(-1)
        toks = np.concatenate([toks, np.arange(4 * nb, Tp)])
        idx[p, :toks.size] = toks
        n_sel[p] = toks.size
    return idx, n_sel


# ----------------------------------------------------------------------------
# token mode: int4 sketch + int8 (or fp16) K/V
# ----------------------------------------------------------------------------

@dataclass
class TokenCase:
    B: int
    T_max: int
    n_kv: int
    n_q: int
    D: int
    R: int
    S: int
    k: int
    L: int
    kv_format: str                   # "i8" (int8 + fp16 row scale) or "f16"
    lens: List[int]
    ctx_len: torch.Tensor            # int32 [B]
    q: torch.Tensor                  # fp16 [B][n_q][D]
    basis: torch.Tensor              # fp32 [n_kv][D][R]
    codes: torch.Tensor              # uint8 [B][T_max][n_kv*R/2]
    sk_scale: torch.Tensor           # fp16 [B][T_max]
    k_cache: torch.Tensor            # int8 or fp16 [B][T_max][n_kv][D]
    v_cache: torch.Tensor
    k_scale: Optional[torch.Tensor]  # fp16 [B][T_max][n_kv] (int8 only)
    v_scale: Optional[torch.Tensor]
    needles: List[torch.Tensor] = field(default_factory=list)  # int64 positions per sequence

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv


def _needle_positions(seed, b, lo, hi, n):
    if hi - lo < n or n == 0:
        return torch.zeros(0, dtype=torch.int64)
    g = _gen("cpu", seed, _T_NEEDLE, b)
    perm = torch.randperm(hi - lo, generator=g)[:n]
    return torch.sort(perm + lo).values


def make_token_case(B: int, T_max: int, ctx_len: Optional[Sequence[int]] = None, *,
                    n_kv: int, n_q: int, D: int, R: int = 64, S: int, k: int, L: int,
                    kv_format: str = "i8", n_needles: int = 8, alpha: float = 2.0,
                    seed: int, device="cpu") -> TokenCase:
    assert n_q % n_kv == 0 and (n_kv * R) % 2 == 0 and kv_format in ("i8", "f16")
    lens = _lengths(B, T_max, ctx_len)
    G = n_q // n_kv
    q = _randn("cpu", seed, (_T_Q,), (B, n_q, D)).to(torch.float16)
    basis = orthonormal_basis(n_kv, D, R, seed)
    nr = n_kv * R

    codes = torch.empty((B, T_max, nr // 2), dtype=torch.uint8, device=device)
    sk_scale = torch.empty((B, T_max), dtype=torch.float16, device=device)
    kv_dt = torch.int8 if kv_format == "i8" else torch.float16
    kk = torch.empty((B, T_max, n_kv, D), dtype=kv_dt, device=device)
    vv = torch.empty((B, T_max, n_kv, D), dtype=kv_dt, device=device)
    ks = torch.empty((B, T_max, n_kv), dtype=torch.float16, device=device) if kv_format == "i8" else None
    vs = torch.empty((B, T_max, n_kv), dtype=torch.float16, device=device) if kv_format == "i8" else None

    for b in range(B):
        for c, c0, n in _chunks(T_max):
            # sketch coordinates of an N(0, I) key through an orthonormal basis are N(0, I)
            s = _randn(device, seed, (_T_SKETCH, b, c), (CHUNK, nr))[:n]
            ci, sc = _vec_to_i4(s)
            codes[b, c0:c0 + n] = pack_int4(ci)
            sk_scale[b, c0:c0 + n] = sc
            for tid, dst, dsc in ((_T_K, kk, ks), (_T_V, vv, vs)):
                x = _randn(device, seed, (tid, b, c), (CHUNK, n_kv, D))[:n]
                if kv_format == "i8":
                    r8, rs = _rows_to_i8(x)
                    dst[b, c0:c0 + n] = r8
                    dsc[b, c0:c0 + n] = rs
                else:
                    dst[b, c0:c0 + n] = x.to(torch.float16)

    # planted needles: key = alpha * (group-mean query), stored through the
    # K format; its sketch is the projection of the stored key, int4-coded.
    needles = []
    qd = q.to(torch.float64)
    bas = basis.to(torch.float64)
    for b in range(B):
        pos = _needle_positions(seed, b, S, lens[b] - L, n_needles)
        needles.append(pos)
        if pos.numel() == 0:
            continue
        qbar = qd[b].view(n_kv, G, D).mean(dim=1)                      # [n_kv][D]
        key = (alpha * qbar).to(torch.float32)
        if kv_format == "i8":
            r8, rs = _rows_to_i8(key)
            kdeq = r8.to(torch.float64) * rs.to(torch.float64).unsqueeze(-1)
            for p in pos.tolist():
                kk[b, p] = r8.to(device)
                ks[b, p] = rs.to(device)
        else:
            kh = key.to(torch.float16)
            kdeq = kh.to(torch.float64)
            for p in pos.tolist():
                kk[b, p] = kh.to(device)
        sk = torch.einsum("hd,hdr->hr", kdeq, bas).reshape(nr)
        ci, sc = _vec_to_i4(sk.to(torch.float32).unsqueeze(0))
        packed = pack_int4(ci)[0]
        for p in pos.tolist():
            codes[b, p] = packed.to(device)
            sk_scale[b, p] = sc[0].to(device)

    return TokenCase(B=B, T_max=T_max, n_kv=n_kv, n_q=n_q, D=D, R=R, S=S, k=k, L=L,
                     kv_format=kv_format, lens=lens,
                     ctx_len=torch.tensor(lens, dtype=torch.int32, device=device),
                     q=q.to(device), basis=basis.to(device), codes=codes, sk_scale=sk_scale,
                     k_cache=kk, v_cache=vv, k_scale=ks, v_scale=vs, needles=needles)


# ----------------------------------------------------------------------------
# block mode: mean-pooled bf16 indexer keys + bf16 K/V
# ----------------------------------------------------------------------------

@dataclass
class BlockCase:
    B: int
    T_max: int
    n_kv: int
    n_q: int
    D: int
    index_dim: int
    k: int                    # budget in blocks
    lens: List[int]
    ctx_len: torch.Tensor     # int32 [B]
    q: torch.Tensor           # bf16 [B][n_q][D]
    qi: torch.Tensor          # bf16 [B][index_dim]
    kp: torch.Tensor          # bf16 [B][T_max//4][index_dim]
    k_cache: torch.Tensor     # bf16 [B][T_max][n_kv][D]
    v_cache: torch.Tensor
    needles: List[torch.Tensor] = field(default_factory=list)   # block indices per sequence

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv


def make_block_case(B: int, T_max: int, ctx_len: Optional[Sequence[int]] = None, *,
                    n_kv: int, n_q: int, D: int, index_dim: int = 128, k: int,
                    n_needles: int = 8, alpha: float = 2.0, seed: int,
                    device="cpu") -> BlockCase:
    assert n_q % n_kv == 0
    lens = _lengths(B, T_max, ctx_len)
    G = n_q // n_kv
    q = _randn("cpu", seed, (_T_Q,), (B, n_q, D)).to(torch.bfloat16)
    qi = flush_bf16_domain(_randn("cpu", seed, (_T_QI,), (B, index_dim)))
    nb_max = T_max // 4
    kp = torch.empty((B, nb_max, index_dim), dtype=torch.bfloat16, device=device)
    kc = torch.empty((B, T_max, n_kv, D), dtype=torch.bfloat16, device=device)
    vc = torch.empty((B, T_max, n_kv, D), dtype=torch.bfloat16, device=device)
    for b in range(B):
        for c, c0, n in _chunks(T_max):
            raw = _randn(device, seed, (_T_RAWIDX, b, c), (CHUNK // 4, 4, index_dim))
            pooled = raw.to(torch.float64).mean(dim=1)
            nb = n // 4
            kp[b, c0 // 4:c0 // 4 + nb] = flush_bf16_domain(pooled[:nb])
            kc[b, c0:c0 + n] = _randn(device, seed, (_T_K, b, c), (CHUNK, n_kv, D))[:n].to(torch.bfloat16)
            vc[b, c0:c0 + n] = _randn(device, seed, (_T_V, b, c), (CHUNK, n_kv, D))[:n].to(torch.bfloat16)
    needles = []
    for b in range(B):
        blocks = _needle_positions(seed, b, 0, lens[b] // 4, n_needles)
        needles.append(blocks)
        if blocks.numel() == 0:
            continue
        pk = flush_bf16_domain(alpha * qi[b].to(torch.float32))
        qbar = q[b].to(torch.float64).view(n_kv, G, D).mean(dim=1)
        krow = (alpha * qbar).to(torch.bfloat16)
        for blk in blocks.tolist():
            kp[b, blk] = pk.to(device)
            for t in range(4 * blk, 4 * blk + 4):
                kc[b, t] = krow.to(device)
    return BlockCase(B=B, T_max=T_max, n_kv=n_kv, n_q=n_q, D=D, index_dim=index_dim, k=k,
                     lens=lens, ctx_len=torch.tensor(lens, dtype=torch.int32, device=device),
                     q=q.to(device), qi=qi.to(device), kp=kp, k_cache=kc, v_cache=vc,
                     needles=needles)


# ----------------------------------------------------------------------------
# host tier: int4 host records, resident sink/tail rows, drifting picks
# ----------------------------------------------------------------------------

HOST_GROUP = 64


def host_row_bytes(D: int) -> int:
    """Bytes of one K (or V) row in the host format: D/2 code bytes + one fp16 per 64 dims."""
    return D // 2 + 2 * (D // HOST_GROUP)


@dataclass
class TierCase:
    B: int
    T: int
    n_kv: int
    n_q: int
    D: int
    S: int
    k: int
    L: int
    n_slots: int
    q: torch.Tensor            # fp16 [B][n_q][D]
    records: torch.Tensor      # uint8 [B][T][n_kv][2*host_row_bytes(D)]  (K row then V row)
    res_k: torch.Tensor        # int8 [B][S+L][n_kv][D]  sinks then tail
    res_v: torch.Tensor
    res_ks: torch.Tensor       # fp16 [B][S+L][n_kv]
    res_vs: torch.Tensor

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv


def _host_rows(x: torch.Tensor) -> torch.Tensor:
    """float rows [N][n_kv][D] -> host records [N][n_kv][host_row_bytes(D)]:
    D/2 bytes of int4 codes, then D/64 fp16 group scales (amax/7)."""
    N, H, D = x.shape
    xg = x.reshape(N, H, D // HOST_GROUP, HOST_GROUP)
    c, gs = _vec_to_i4(xg)                               # c [N][H][g][64], gs [N][H][g]
    packed = pack_int4(c.reshape(N, H, D))               # [N][H][D/2]
    sb = gs.contiguous().view(torch.uint8).reshape(N, H, 2 * (D // HOST_GROUP))
    return torch.cat([packed, sb], dim=-1)


def make_tier_case(B: int, T: int, *, n_kv: int, n_q: int, D: int, S: int, k: int, L: int,
                   hot_fraction: float = 0.025, seed: int, device="cpu") -> TierCase:
    assert D % HOST_GROUP == 0
    q = _randn("cpu", seed, (_T_Q,), (B, n_q, D)).to(torch.float16)
    rb = host_row_bytes(D)
    rec = torch.empty((B, T, n_kv, 2 * rb), dtype=torch.uint8, device=device)
    for b in range(B):
        for c, c0, n in _chunks(T):
            xk = _randn(device, seed, (_T_HK, b, c), (CHUNK, n_kv, D))[:n]
            xv = _randn(device, seed, (_T_HV, b, c), (CHUNK, n_kv, D))[:n]
            rec[b, c0:c0 + n, :, :rb] = _host_rows(xk)
            rec[b, c0:c0 + n, :, rb:] = _host_rows(xv)
    nres = S + L
    xk = _randn(device, seed, (_T_RK,), (B, nres, n_kv, D))
    xv = _randn(device, seed, (_T_RV,), (B, nres, n_kv, D))
    rk, rks = _rows_to_i8(xk)
    rv, rvs = _rows_to_i8(xv)
    n_slots = int(hot_fraction * T)
    return TierCase(B=B, T=T, n_kv=n_kv, n_q=n_q, D=D, S=S, k=k, L=L, n_slots=n_slots,
                    q=q.to(device), records=rec, res_k=rk, res_v=rv, res_ks=rks, res_vs=rvs)


def tier_page_rows(B: int, T: int, *, n_kv: int, D: int, seed: int, page_tokens: int, pages,
                   device="cpu"):
    """int8 rows + fp16 row scales of whole pages of a tier case: the same
    tokens as make_tier_case's host records (same random streams), stored the
    way a plain int8 cache holds them.  pages: list of (sequence, page);
    returns k8, ks, v8, vs shaped [len(pages)][page_tokens][n_kv][D] / [..][n_kv]
    (positions past T are zero rows)."""
    P = int(page_tokens)
    assert CHUNK % P == 0
    n = len(pages)
    k8 = torch.zeros((n, P, n_kv, D), dtype=torch.int8, device=device)
    v8 = torch.zeros((n, P, n_kv, D), dtype=torch.int8, device=device)
    ks = torch.zeros((n, P, n_kv), dtype=torch.float16, device=device)
    vs = torch.zeros((n, P, n_kv), dtype=torch.float16, device=device)
    cache = {}
    for j, (b, g) in enumerate(pages):
        p0 = g * P
        if p0 >= T:
            continue
        c = p0 // CHUNK
        if (b, c) not in cache:
            cache.clear()
            xk = _randn(device, seed, (_T_HK, b, c), (CHUNK, n_kv, D))
            xv = _randn(device, seed, (_T_HV, b, c), (CHUNK, n_kv, D))
            cache[(b, c)] = (_rows_to_i8(xk), _rows_to_i8(xv))
        (rk, rks), (rv, rvs) = cache[(b, c)]
        o = p0 - c * CHUNK
        m = min(P, T - p0)
        k8[j, :m], ks[j, :m] = rk[o:o + m], rks[o:o + m]
        v8[j, :m], vs[j, :m] = rv[o:o + m], rvs[o:o + m]
    return k8, ks, v8, vs


def drift_picks(B: int, T: int, S: int, L: int, k: int, n_steps: int, seed: int, *,
                sigma_c: float = 256.0, window: int = 65536, rho: float = 0.165) -> np.ndarray:
    """Drifting-locality pick schedule, int32 [n_steps][B][k], each row sorted.

    Per sequence a centre does a Gaussian random walk (step sd sigma_c tokens)
    inside the middle range [S, T-L).  Each previous pick survives a step with
    probability 1-rho; replacements are drawn uniformly from a window of
    `window` tokens around the centre, rejecting duplicates."""
    rng = np.random.Generator(np.random.PCG64(_subseed(seed, _T_DRIFT)))
    lo, hi = S, T - L
    assert hi - lo >= k
    half = window // 2
    out = np.empty((n_steps, B, k), dtype=np.int32)
    for b in range(B):
        if hi - lo > window:
            c = float(rng.integers(lo + half, hi - half + 1))
        else:
            c = (lo + hi) / 2.0
        cur = np.zeros(0, dtype=np.int64)
        for s in range(n_steps):
            if s > 0:
                c += rng.normal(0.0, sigma_c)
                if hi - lo > window:
                    c = min(max(c, lo + half), hi - half)
                keep = rng.random(cur.size) >= rho
                cur = cur[keep]
            wlo = max(lo, int(round(c)) - half)
            whi = min(hi, wlo + window)
            wlo = max(lo, whi - window)
            have = set(cur.tolist())
            need = k - len(have)
            while need > 0:
                cand = rng.integers(wlo, whi, size=2 * need + 16)
                for x in cand.tolist():
                    if x not in have:
                        have.add(x)
                        need -= 1
                        if need == 0:
                            break
            cur = np.array(sorted(have), dtype=np.int64)
            out[s, b] = cur
    return out


def draft_picks(base: np.ndarray, M: int, share: float, seed: int) -> np.ndarray:
    """Pick lists of M query tokens per sequence and step, int32
    [n_steps][B][M][k], each row sorted: query 0 takes the base picks
    ([n_steps][B][k], e.g. drift_picks); each later query (a drafted token)
    keeps a random round(share * k) of them and replaces the rest with
    positions drawn uniformly between the smallest and largest base pick,
    rejecting duplicates.  All positions stay inside the base picks' range."""
    rng = np.random.Generator(np.random.PCG64(_subseed(seed, _T_DRAFT)))
    n_steps, B, k = base.shape
    n_keep = int(round(share * k))
    out = np.empty((n_steps, B, M, k), dtype=np.int32)
    for s in range(n_steps):
        for b in range(B):
            bs = np.sort(base[s, b].astype(np.int64))
            out[s, b, 0] = bs
            lo, hi = int(bs[0]), int(bs[-1]) + 1
            for j in range(1, M):
                kept = bs[np.sort(rng.choice(k, n_keep, replace=False))]
                need = k - n_keep
                got = np.zeros(0, dtype=np.int64)
                while got.size < need:
                    cand = rng.integers(lo, hi, size=3 * need + 16)
                    pos = np.searchsorted(bs, cand)
                    fresh = cand[(pos >= k) | (bs[np.minimum(pos, k - 1)] != cand)]
                    got = np.unique(np.concatenate([got, fresh]))
                got = rng.permutation(got)[:need]
                out[s, b, j] = np.sort(np.concatenate([kept, got]))
    return out
