"""Pins of the CPU oracle to facts that do not come from the oracle itself:
hand-worked fixtures (tests/golden), the pages' closed forms, brute force on
tiny inputs, exact rational arithmetic, a library attention routine, and
special cases with known answers.

Pages (by title):
  [P1] "8 agents x 250K context on two 3090s: sparse KV decode with a rank-64
       key sketch and a host-RAM tier"
  [P3] "You can offload most of Qwen3.8-Flash-Next's KV cache to RAM with
       little decode slowdown"
  [P4] "3.14M Context on 3x 3090: The Power of an Architecture That Puts KV
       Cache in Host RAM"
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")
MiB = 1 << 20
KiB = 1 << 10


def _lines(name):
    with open(os.path.join(GOLD, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln


# --------------------------------------------------------------------------
# formats and scores
# --------------------------------------------------------------------------

def test_int4_nibbles_fixture():
    for ln in _lines("int4_nibbles.txt"):
        parts = ln.split()
        if parts[0] == "score":
            code_bytes = np.array([int(x, 16) for x in parts[1].split(",")], dtype=np.uint8)
            qv = np.array([int(x) for x in parts[2].split(",")], dtype=np.int8)
            scale = np.array([np.float16(float(parts[3]))])
            codes = code_bytes.reshape(1, 1, -1)
            keys = oracle.sketch_keys(qv.reshape(1, -1), codes, scale.reshape(1, 1), [1], 0, 0, 0)
            dot = int(np.dot(oracle.unpack_int4(code_bytes).astype(np.int64), qv.astype(np.int64)))
            assert dot == int(parts[4])
            assert keys[0, 0] == float(parts[5])
            continue
        byte = np.array([int(parts[0], 16)], dtype=np.uint8)
        got = oracle.unpack_int4(byte).tolist()
        assert got == [int(parts[1]), int(parts[2])], (parts, got)


def test_sketch_keys_exact_rational():
    """key = dot * scale with no rounding: compared with exact rationals and a
    per-bit brute-force decode of the nibbles."""
    rng = np.random.default_rng(7)
    B, T, nb = 2, 50, 16
    codes = rng.integers(0, 256, size=(B, T, nb), dtype=np.uint8)
    scale = rng.uniform(0.001, 3.0, size=(B, T)).astype(np.float16)
    qs = rng.integers(-127, 128, size=(B, 2 * nb), dtype=np.int8)
    keys = oracle.sketch_keys(qs, codes, scale, [T, T - 7], 3, 0, 5)
    for b in range(B):
        Tb = [T, T - 7][b]
        for t in range(T):
            if not (3 <= t < Tb - 5):
                assert np.isnan(keys[b, t])
                continue
            dot = 0
            for j in range(nb):
                byte = int(codes[b, t, j])
                for half in range(2):
                    nib = (byte >> (4 * half)) & 0xF
                    val = nib - 16 if nib & 0x8 else nib
                    dot += val * int(qs[b, 2 * j + half])
            exact = Fraction(dot) * Fraction(float(scale[b, t]))
            assert Fraction(keys[b, t]) == exact


def test_pooled_keys_exact_rational():
    """Pooled scores equal the exact rational dot product (in-domain bf16 data)."""
    g = torch.Generator().manual_seed(3)
    qi = synth.flush_bf16_domain(torch.randn(1, 128, generator=g) * 3)
    kp = synth.flush_bf16_domain(torch.randn(1, 20, 128, generator=g) * 5)
    qi_b = qi.view(torch.int16).numpy().view(np.uint16)
    kp_b = kp.view(torch.int16).numpy().view(np.uint16)
    keys = oracle.pooled_keys(qi_b, kp_b, [4 * 17 + 2])
    qf = qi.float().numpy()
    kf = kp.float().numpy()
    for blk in range(20):
        if blk >= 17:
            assert np.isnan(keys[0, blk])
            continue
        exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qf[0], kf[0, blk]))
        assert Fraction(keys[0, blk]) == exact


# --------------------------------------------------------------------------
# query sketch
# --------------------------------------------------------------------------

def _parse_sketch_case(ln):
    kv = dict(p.split("=", 1) for p in ln.split()[1:])
    G, D = int(kv["group"]), int(kv["D"])
    cols = [int(c) for c in kv["cols"].split(",")]
    qrows = [[float(x) for x in r.split(",")] for r in kv["q"].split(";")]
    basis = np.zeros((1, D, len(cols)), dtype=np.float32)
    for r, c in enumerate(cols):
        basis[0, c, r] = 1.0
    q = np.array(qrows, dtype=np.float16).reshape(1, G, D)
    return q, basis, G, [int(x) for x in kv["expect"].split(",")]


def test_query_sketch_fixture():
    for ln in _lines("query_sketch.txt"):
        if ln.startswith("basis "):
            continue
        q, basis, G, expect = _parse_sketch_case(ln)
        qs, qscale = oracle.query_sketch(q, basis, G)
        assert qs[0].tolist() == expect, ln
        if all(e == 0 for e in expect):
            assert qscale[0] == 0
        else:
            assert qscale[0] > 0


def _hexf(v):
    return [float.fromhex(x) for x in v.split(",")]


def test_query_sketch_nonunit_basis_fixture():
    """Hand-derived cases (tests/golden/query_sketch.txt, "basis" lines) whose
    fp32 scale changes if the products are fused into the sums or the sum is
    taken in another order (or in fp64)."""
    n = 0
    for ln in _lines("query_sketch.txt"):
        if not ln.startswith("basis "):
            continue
        kv = dict(p.split("=", 1) for p in ln.split()[2:])
        G, D = int(kv["group"]), int(kv["D"])
        q = np.array([_hexf(r) for r in kv["q"].split(";")], dtype=np.float64)
        assert np.array_equal(q.astype(np.float16).astype(np.float64), q), ln   # fp16-exact inputs
        basis = np.array(_hexf(kv["col"]), dtype=np.float64).reshape(1, D, 1)
        assert np.array_equal(basis.astype(np.float32).astype(np.float64), basis), ln
        qs, qscale = oracle.query_sketch(q.astype(np.float16).reshape(1, G, D), basis.astype(np.float32), G)
        assert qs[0].tolist() == [int(x) for x in kv["expect"].split(",")], ln
        assert int(np.asarray(qscale[0], dtype=np.float32).view(np.uint32)) == int(kv["qscale"], 16), ln
        n += 1
    assert n == 2


def test_query_sketch_orthonormal_round_trip():
    """A query in the span of an orthonormal basis projects back onto its
    coordinates.  The basis is a 4x4 Hadamard matrix / 2 with its columns
    permuted (orthonormal, entries +-0.5, not symmetric, so projecting with the
    transposed basis fails); every product and sum is exact in fp32."""
    H = 0.5 * np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], dtype=np.float64)
    Bm = H[:, [2, 0, 3, 1]]
    assert np.allclose(Bm.T @ Bm, np.eye(4)) and not np.allclose(Bm, Bm.T)
    c = np.array([8.0, -4.0, 2.0, 6.0])
    q = (Bm @ c).reshape(1, 1, 4)        # the query whose coordinates are c
    qs, qscale = oracle.query_sketch(q.astype(np.float16), Bm.reshape(1, 4, 4).astype(np.float32), 1)
    # s = c exactly; amax = 8, qscale = fp32(8/127); codes rint(c * 127/8):
    # 127, -63.5 -> -64 (half to even), 31.75 -> 32, 95.25 -> 95
    assert float(qscale[0]) == float(np.float32(8.0) / np.float32(127.0))
    assert qs[0].tolist() == [127, -64, 32, 95]


def test_query_sketch_scale_invariance():
    """Doubling the query doubles every fp32 intermediate exactly, so the int8
    codes are unchanged and the scale doubles."""
    c = synth.make_token_case(2, 64, n_kv=4, n_q=24, D=256, S=4, k=8, L=4, seed=11)
    q = c.q.numpy()
    qs1, sc1 = oracle.query_sketch(q, c.basis.numpy(), 6)
    qs2, sc2 = oracle.query_sketch((q.astype(np.float32) * 2).astype(np.float16), c.basis.numpy(), 6)
    assert np.array_equal(qs1, qs2)
    assert np.array_equal(sc2, sc1 * 2)


def test_query_sketch_projection_bound():
    """The int8 code times its scale is within half a step of the fp64 projection
    of the summed query (plus fp32 rounding)."""
    c = synth.make_token_case(3, 64, n_kv=4, n_q=24, D=256, S=4, k=8, L=4, seed=12)
    q = c.q.numpy().astype(np.float64)
    bas = c.basis.numpy().astype(np.float64)
    qs, sc = oracle.query_sketch(c.q.numpy(), c.basis.numpy(), 6)
    for b in range(3):
        qbar = q[b].reshape(4, 6, 256).sum(axis=1)
        s = np.einsum("hd,hdr->hr", qbar, bas).reshape(-1)
        err = np.abs(qs[b].astype(np.float64) * sc[b] - s)
        assert np.max(err) <= 0.5 * sc[b] + 1e-4 * np.max(np.abs(s))
        assert np.max(np.abs(qs[b])) == 127


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------

def _brute_topk(keys, cand, k):
    """Rank by counting: a candidate is kept iff fewer than k candidates beat
    it (larger key, or equal key at a lower position)."""
    keep = []
    for c in cand:
        beats = sum(1 for d in cand if keys[d] > keys[c] or (keys[d] == keys[c] and d < c))
        if beats < k:
            keep.append(c)
    return keep


@pytest.mark.parametrize("seed", range(6))
def test_select_tokens_bruteforce(seed):
    rng = np.random.default_rng(seed)
    S, k, L = 3, 7, 5
    for T in (0, 1, 14, 15, 16, 40, 64):
        keys = rng.integers(-4, 5, size=T).astype(np.float64)   # many exact ties
        got = oracle.select_tokens(keys, T, S, k, L)
        if T <= S + k + L:
            assert got.tolist() == list(range(T))
            continue
        mid = _brute_topk(keys, list(range(S, T - L)), k)
        want = sorted(set(range(S)) | set(mid) | set(range(T - L, T)))
        assert got.tolist() == want
        assert len(got) == S + k + L


@pytest.mark.parametrize("seed", range(6))
def test_select_blocks_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    kb = 5
    for T in (0, 3, 20, 23, 24, 25, 26, 27, 61):
        nb = T // 4
        keys = rng.integers(-3, 4, size=max(nb, 1)).astype(np.float64)
        got = oracle.select_blocks(keys, T, kb)
        if nb <= kb:
            assert got.tolist() == list(range(T))
            continue
        blocks = _brute_topk(keys, list(range(nb)), kb)
        want = sorted({4 * b + i for b in blocks for i in range(4)} | set(range(4 * nb, T)))
        assert got.tolist() == want


def test_select_all_equal_keys():
    """All keys equal: the tie rule keeps the first k candidates."""
    T, S, k, L = 1000, 10, 50, 20
    got = oracle.select_tokens(np.zeros(T), T, S, k, L)
    assert got.tolist() == list(range(S + k)) + list(range(T - L, T))
    gotb = oracle.select_blocks(np.ones(T // 4), T, 30)
    assert gotb.tolist() == list(range(120))


def test_dense_threshold_block_mode():
    """[P4] "Why": selection starts once the context exceeds 4*block_topk+3 =
    2051; above it exactly 2048 tokens of complete blocks are read."""
    kb = 512
    assert 4 * kb + 3 == 2051
    for T in (1, 2048, 2050, 2051):
        assert oracle.select_blocks(np.zeros(T // 4), T, kb).size == T
    got = oracle.select_blocks(np.arange(2052 // 4, dtype=np.float64), 2052, kb)
    assert got.size == 2048 and 0 not in got.tolist()   # exactly one block (the lowest-key one) dropped
    for T in (2052, 2053, 3000, 3_000_001, 1_048_576):
        nb = T // 4
        got = oracle.select_blocks(np.zeros(nb), T, kb)
        assert got.size == 2048 + T % 4      # budget does not grow with context


def test_dense_threshold_token_mode():
    """[P1] "The mechanism": top 2048 + 64 sinks + last 1024 (config shapes);
    dense exactly while T <= S + k + L."""
    for (S, k, L) in ((64, 2048, 1024), (16, 256, 128)):
        thr = S + k + L
        assert oracle.select_tokens(np.zeros(thr), thr, S, k, L).size == thr
        for T in (thr + 1, thr + 2, 250_000):
            assert oracle.select_tokens(np.zeros(T), T, S, k, L).size == thr
    assert 64 + 2048 + 1024 == 3136 and 16 + 256 + 128 == 400


def test_budget_fractions():
    """[P1]: 2048 of 250K is ~0.8%; with sinks and tail ~1% of tokens are read."""
    assert round(100 * 2048 / 250_000, 1) == 0.8
    assert 1.0 <= 100 * 3136 / 250_000 < 1.5


def test_needles_recovered_token_mode():
    c = synth.make_token_case(1, 4096, n_kv=2, n_q=8, D=128, S=16, k=256, L=128,
                              kv_format="f16", seed=1001)
    c2 = synth.make_token_case(2, 40_000, n_kv=4, n_q=24, D=256, S=64, k=2048, L=1024,
                               kv_format="i8", seed=1002)
    for case in (c, c2):
        qs, _ = oracle.query_sketch(case.q.numpy(), case.basis.numpy(), case.group)
        keys = oracle.sketch_keys(qs, case.codes.numpy(), case.sk_scale.numpy(), case.lens,
                                  case.S, case.k, case.L)
        for b in range(case.B):
            sel = oracle.select_tokens(keys[b], case.lens[b], case.S, case.k, case.L)
            assert len(case.needles[b]) == 8
            assert np.isin(case.needles[b].numpy(), sel).all()


def test_needles_recovered_block_mode():
    c = synth.make_block_case(1, 65_536, n_kv=2, n_q=16, D=256, k=512, seed=1003)
    keys = oracle.pooled_keys(c.qi.view(torch.int16).numpy(), c.kp.view(torch.int16).numpy(), c.lens)
    sel = oracle.select_blocks(keys[0], c.lens[0], c.k)
    for blk in c.needles[0].tolist():
        assert all(t in set(sel.tolist()) for t in range(4 * blk, 4 * blk + 4))


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def _small_token_case(kv_format="i8", T=300, seed=5):
    return synth.make_token_case(2, T, [T, T - 37], n_kv=2, n_q=6, D=64, S=4, k=1000, L=8,
                                 kv_format=kv_format, n_needles=0, seed=seed)


@pytest.mark.parametrize("fmt", ["i8", "f16"])
def test_attention_matches_torch_sdpa(fmt):
    """Dense decode attention equals torch's fp64 scaled_dot_product_attention."""
    c = _small_token_case(fmt)
    ks = None if c.k_scale is None else c.k_scale.numpy()
    vs = None if c.v_scale is None else c.v_scale.numpy()
    sm = 64 ** -0.5
    for b in range(c.B):
        T = c.lens[b]
        got = oracle.dense_attention(c.q[b].numpy(), c.k_cache[b].numpy(), c.v_cache[b].numpy(),
                                     None if ks is None else ks[b], None if vs is None else vs[b],
                                     T, sm, c.group, fmt)
        kd = c.k_cache[b, :T].double()
        vd = c.v_cache[b, :T].double()
        if fmt == "i8":
            kd = kd * c.k_scale[b, :T].double().unsqueeze(-1)
            vd = vd * c.v_scale[b, :T].double().unsqueeze(-1)
        kk = kd.permute(1, 0, 2).repeat_interleave(c.group, dim=0)   # [H_q][T][D]
        vv = vd.permute(1, 0, 2).repeat_interleave(c.group, dim=0)
        qq = c.q[b].double().unsqueeze(1)                             # [H_q][1][D]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=sm)[:, 0]
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


def test_attention_special_cases():
    c = _small_token_case("i8")
    k, v = c.k_cache[0].numpy(), c.v_cache[0].numpy()
    ks, vs = c.k_scale[0].numpy(), c.v_scale[0].numpy()
    # one selected row -> the output is that row of V, exactly
    out = oracle.sparse_attention(c.q[0].numpy(), k, v, ks, vs, [123], 0.125, c.group, "i8")
    vrow = v[123].astype(np.float64) * vs[123].astype(np.float64)[:, None]
    for j in range(c.n_q):
        assert np.array_equal(out[j], vrow[j // c.group])
    # zero query -> uniform weights -> mean of the selected V rows
    idx = np.array([3, 50, 51, 200])
    out = oracle.sparse_attention(np.zeros_like(c.q[0].numpy()), k, v, ks, vs, idx, 0.125, c.group, "i8")
    vd = v[idx].astype(np.float64) * vs[idx].astype(np.float64)[..., None]
    for j in range(c.n_q):
        np.testing.assert_allclose(out[j], vd[:, j // c.group].mean(axis=0), rtol=0, atol=1e-15)
    # nothing selected -> zeros
    out = oracle.sparse_attention(c.q[0].numpy(), k, v, ks, vs, [], 0.125, c.group, "i8")
    assert not out.any()


@pytest.mark.parametrize("fmt", ["i8", "f16"])
def test_dense_equals_sparse_bitwise(fmt):
    """North-star check 1: with a budget no smaller than the context, the
    selected-row attention equals dense attention bit for bit."""
    c = _small_token_case(fmt, T=500)
    qs, qsc = oracle.query_sketch(c.q.numpy(), c.basis.numpy(), c.group)
    keys = oracle.sketch_keys(qs, c.codes.numpy(), c.sk_scale.numpy(), c.lens, c.S, c.k, c.L)
    ks = None if c.k_scale is None else c.k_scale.numpy()
    vs = None if c.v_scale is None else c.v_scale.numpy()
    for b in range(c.B):
        T = c.lens[b]
        assert c.k >= T - c.S - c.L
        idx = oracle.select_tokens(keys[b], T, c.S, c.k, c.L)
        sp = oracle.sparse_attention(c.q[b].numpy(), c.k_cache[b].numpy(), c.v_cache[b].numpy(),
                                     None if ks is None else ks[b], None if vs is None else vs[b],
                                     idx, 0.125, c.group, fmt)
        de = oracle.dense_attention(c.q[b].numpy(), c.k_cache[b].numpy(), c.v_cache[b].numpy(),
                                    None if ks is None else ks[b], None if vs is None else vs[b],
                                    T, 0.125, c.group, fmt)
        assert np.array_equal(sp, de)
    # the same in block mode (budget 600 blocks >= T/4)
    cb = synth.make_block_case(1, 2000, n_kv=2, n_q=4, D=64, k=600, n_needles=0, seed=9)
    keys = oracle.pooled_keys(cb.qi.view(torch.int16).numpy(), cb.kp.view(torch.int16).numpy(), cb.lens)
    idx = oracle.select_blocks(keys[0], 2000, 600)
    kb = cb.k_cache[0].view(torch.int16).numpy()
    vb = cb.v_cache[0].view(torch.int16).numpy()
    qb = cb.q[0].view(torch.int16).numpy()
    sp = oracle.sparse_attention(qb, kb, vb, None, None, idx, 0.1, 2, "bf16")
    de = oracle.dense_attention(qb, kb, vb, None, None, 2000, 0.1, 2, "bf16")
    assert np.array_equal(sp, de)


# --------------------------------------------------------------------------
# byte closed forms
# --------------------------------------------------------------------------

def test_byte_closed_forms():
    # [P3], [P4] "Why": 2048 selected x 2 KV heads x 256 x (K and V) x 2 B = 4 MiB/layer, 48 MiB/token
    assert oracle.kv_gather_bytes(2048, 2, 256, 2) == 4 * MiB
    assert 12 * oracle.kv_gather_bytes(2048, 2, 256, 2) == 48 * MiB
    # [P3]: 2,048 B per token per QSA layer; 512 MiB per layer at 262,144 tokens; 6 GiB for 12
    assert oracle.kv_gather_bytes(1, 2, 256, 2) == 2048
    assert 262_144 * 2048 == 512 * MiB and 12 * 512 * MiB == 6 * 1024 * MiB
    # [P4] "What Needs to Stay in VRAM": pooled keys 128 x 2 B per block -> 64 MiB/layer at 1 Mi tokens
    assert oracle.block_scan_bytes(1_048_576 // 4, 128) == 64 * MiB
    # [P3]: pooled key 64 B per token + 2 B slot = 66 B per token per layer
    assert oracle.block_scan_bytes(1, 128) // 4 == 64 and 64 + 2 == 66
    # [P4] intro / "What Needs to Stay in VRAM": 27.75 KiB/token = 27.00 in RAM + 0.75 in VRAM (12 layers)
    assert 12 * (2048 + 256 + 64) == 27.75 * KiB
    assert 12 * (2048 + 256) == 27.00 * KiB and 12 * 64 == 0.75 * KiB
    # [P1] "The mechanism": int4 sketch ~2.1 KB per token over 16 layers
    per_layer = oracle.token_scan_bytes(1, 4, 64)
    assert per_layer == 130 and 16 * per_layer == 2080
    assert 0.52e9 <= 250_000 * 16 * per_layer <= 0.53e9            # "0.53 int4 sketch" GB/agent
    # [P1]: 272 B per token-head at int4; 4.4 GB per 250K agent (16 layers x 4 KV heads)
    assert oracle.host_record_bytes(256) == 272
    assert round(250_000 * 16 * 4 * 272 / 1e9, 1) == 4.4
    # the per-step K/V budget does not depend on context length ([P4] "Why")
    for T in (2052, 100_000, 3_000_000):
        n = oracle.select_blocks(np.zeros(T // 4), T - T % 4, 512).size
        assert oracle.kv_gather_bytes(n, 2, 256, 2) == 4 * MiB


# --------------------------------------------------------------------------
# host tier
# --------------------------------------------------------------------------

def test_host_dequant_fixture():
    lines = list(_lines("host_dequant.txt"))
    scales = [float(x) for x in lines[0].split()[1].split(",")]
    sprime = float(lines[1].split()[1])
    D = 128
    codes = np.zeros(D, dtype=np.int8)
    expect = np.zeros(D, dtype=np.int8)
    for ln in lines[2:]:
        i, cc, e = (int(x) for x in ln.split())
        codes[i], expect[i] = cc, e
    row = np.concatenate([synth.pack_int4(torch.from_numpy(codes)).numpy(),
                          np.array(scales, dtype=np.float16).view(np.uint8)])
    r8, sp = oracle.host_row_dequant(row, D)
    assert float(sp) == sprime
    assert r8.tolist() == expect.tolist()


def test_host_dequant_invariants():
    rng = np.random.default_rng(4)
    D = 256
    for _ in range(200):
        codes = rng.integers(-8, 8, size=D).astype(np.int8)
        gs = rng.uniform(0, 2, size=D // 64).astype(np.float16)
        row = np.concatenate([synth.pack_int4(torch.from_numpy(codes)).numpy(), gs.view(np.uint8)])
        r8, sp = oracle.host_row_dequant(row, D)
        assert np.all(np.abs(r8.astype(int)) <= 127)
        for g in range(D // 64):
            c = codes[64 * g:64 * g + 64].astype(int)
            r = r8[64 * g:64 * g + 64].astype(int)
            order = np.argsort(c, kind="stable")
            assert np.all(np.diff(r[order]) >= 0)          # monotone in the code
            assert np.all(np.sign(r) * np.sign(c) >= 0)     # sign preserved


def _rint_half_even(x: Fraction) -> int:
    n = x.numerator // x.denominator
    r = x - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def _host_row(codes, gscales):
    return np.concatenate([synth.pack_int4(torch.from_numpy(np.asarray(codes, np.int8))).numpy(),
                           np.array(gscales, dtype=np.float16).view(np.uint8)])


def test_tier_attention_equals_plain_cache():
    """oracle.tier_attention over host records equals oracle.sparse_attention
    over a plain int8 cache holding the rows those records decode to, bit for
    bit.  Group scales 127 * 2^-j make the fetched row scale s' = fp16(127 * 7 /
    127) = 7 exactly, so the expected int8 codes rint(c * g_j / 7) are computed
    here in exact rational arithmetic, independently of host_row_dequant."""
    rng = np.random.default_rng(31)
    n_kv, G, D, T, S, L = 2, 2, 256, 40, 4, 6
    ng = D // 64
    gs = [127.0 * 2.0 ** -j for j in range(ng)]
    rb = D // 2 + 2 * ng
    records = np.zeros((T, n_kv, 2 * rb), dtype=np.uint8)
    k8 = np.zeros((T, n_kv, D), np.int8)
    v8 = np.zeros((T, n_kv, D), np.int8)
    ks = np.zeros((T, n_kv), np.float16)
    vs = np.zeros((T, n_kv), np.float16)
    for p in range(S, T - L):
        for h in range(n_kv):
            for part, dst, sdst in ((0, k8, ks), (1, v8, vs)):
                c = rng.integers(-7, 8, size=D)
                records[p, h, part * rb:(part + 1) * rb] = _host_row(c, gs)
                dst[p, h] = [max(-127, min(127, _rint_half_even(Fraction(int(c[i])) * Fraction(gs[i // 64]) / 7)))
                             for i in range(D)]
                sdst[p, h] = 7.0
    # resident rows: the sinks, then the tail in position order
    res_k = rng.integers(-127, 128, size=(S + L, n_kv, D)).astype(np.int8)
    res_v = rng.integers(-127, 128, size=(S + L, n_kv, D)).astype(np.int8)
    res_ks = rng.uniform(0.001, 0.02, size=(S + L, n_kv)).astype(np.float16)
    res_vs = rng.uniform(0.001, 0.02, size=(S + L, n_kv)).astype(np.float16)
    pos = list(range(S)) + list(range(T - L, T))
    for r, p in enumerate(pos):
        k8[p], v8[p], ks[p], vs[p] = res_k[r], res_v[r], res_ks[r], res_vs[r]
    q = rng.standard_normal((n_kv * G, D)).astype(np.float16)
    sm = D ** -0.5
    for idx in (np.arange(T), np.array([0, 3, 4, 5, 17, 33, 34, 39]), np.array([6, 20, 21, 33])):
        a = oracle.tier_attention(q, records, res_k, res_v, res_ks, res_vs, idx, T, S, L, sm, G, D)
        b = oracle.sparse_attention(q, k8, v8, ks, vs, idx, sm, G, "i8")
        assert np.array_equal(a, b)


def test_tier_attention_position_rows():
    """Hand-worked map from positions to rows (T = 12, S = 2, L = 3, D = 64,
    one head): attending a single position returns its V row exactly.
    Resident rows 0..4 hold the sinks 0, 1 and the tail 9, 10, 11, each V row
    the constant 10 + row (scale 1); middle positions 2..8 come from host
    records with V codes c = p - 5 and group scale 127, decoded with s' = 7 to
    rint(c * 127 / 7) = 18c for |c| <= 3 (18.14c rounded), so value 7 * 18c.
    K codes are all 0 (equal logits)."""
    T, S, L, D = 12, 2, 3, 64
    rb = D // 2 + 2
    records = np.zeros((T, 1, 2 * rb), dtype=np.uint8)
    for p in range(S, T - L):
        records[p, 0, :rb] = _host_row(np.zeros(D, np.int8), [127.0])
        records[p, 0, rb:] = _host_row(np.full(D, p - 5, np.int8), [127.0])
    res_k = np.zeros((S + L, 1, D), np.int8)
    res_v = np.array([np.full((1, D), 10 + r, np.int8) for r in range(S + L)])
    ones = np.ones((S + L, 1), np.float16)
    q = np.ones((1, D), np.float16)
    expect = {0: 10, 1: 11, 2: -378, 3: -252, 4: -126, 5: 0, 6: 126, 7: 252, 8: 378, 9: 12, 10: 13, 11: 14}
    for p, val in expect.items():
        o = oracle.tier_attention(q, records, res_k, res_v, ones, ones, np.array([p]), T, S, L, 0.125, 1, D)
        assert np.all(o == val), (p, o[0, :4])


def test_residency_fixture():
    """Hand trace of page residency over an LRU hot buffer
    (tests/golden/residency_trace.txt): picks of mapped pages are read in
    place at block*P + p%P, the others go through the hot buffer; mapping
    changes between steps move picks between the two; full, mixed and no
    residency all appear."""
    lines = list(_lines("residency_trace.txt"))
    n_slots, P, n_pages = (int(lines[i].split()[1]) for i in range(3))
    tier = oracle.residency.PagedTier(oracle.residency.LruTier(n_slots, 100), P, n_pages)
    code = {oracle.residency.IN_PLACE: "R", oracle.residency.HIT: "H", oracle.residency.MISS: "M"}
    for ln in lines[3:]:
        w = ln.split()
        if w[0] == "map":
            tier.map_page(int(w[1]), int(w[2]))
        elif w[0] == "unmap":
            tier.unmap_page(int(w[1]))
        elif w[0] == "mapall":
            for g in range(n_pages):
                tier.map_page(g, g)
        elif w[0] == "unmapall":
            for g in range(n_pages):
                tier.unmap_page(g)
        elif w[0] == "final":
            assert tier.hot.pos.tolist() == [int(x) for x in w[1:]]
        else:
            s, picks, per, counts = (x.strip() for x in ln.split("|"))
            kind, where, cnt = tier.step(np.array([int(x) for x in picks.split()]), int(s))
            got = ["%s%d" % (code[int(k)], int(x)) for k, x in zip(kind, where)]
            assert got == per.split(), ln
            assert cnt == tuple(int(x) for x in counts.split()), ln


def test_residency_invariants_drifting_workload():
    """With pages mapped and unmapped at random between steps: in place + hits
    + misses = picks; in-place picks are exactly those of mapped pages, at
    their pool row; every other pick sits in the hot slot reported; and with
    no page ever mapped the slots equal those of the bare hot buffer."""
    T, S, L, k, P = 30_000, 64, 1024, 256, 64
    n_pages = (T + P - 1) // P
    picks = synth.drift_picks(1, T, S, L, k, 40, seed=45, window=4096, sigma_c=256.0)
    rng = np.random.default_rng(7)
    paged = oracle.residency.PagedTier(oracle.residency.LruTier(2 * k, T), P, n_pages)
    plain = oracle.residency.PagedTier(oracle.residency.LruTier(2 * k, T), P, n_pages)
    bare = oracle.residency.LruTier(2 * k, T)
    for s in range(40):
        for g in rng.choice(n_pages, size=20, replace=False).tolist():
            if paged.block[g] >= 0:
                paged.unmap_page(g)
            else:
                paged.map_page(g, int(rng.integers(0, 1000)))
        p = np.asarray(picks[s][0], dtype=np.int64)
        kind, where, (n_in, h, m) = paged.step(p, s)
        assert n_in + h + m == p.size
        mapped = paged.block[p // P] >= 0
        assert np.array_equal(kind == oracle.residency.IN_PLACE, mapped)
        assert np.array_equal(where[mapped], paged.block[p[mapped] // P] * P + p[mapped] % P)
        assert np.array_equal(paged.hot.pos[where[~mapped]], p[~mapped])
        k2, w2, c2 = plain.step(p, s)
        slots, h2, m2 = bare.step(p, s)
        assert np.array_equal(w2, slots) and c2 == (0, h2, m2)
        assert not (k2 == oracle.residency.IN_PLACE).any()


def test_paged_attention_one_row_sources():
    """Hand-worked sources (T = 16, S = 2, L = 3, pages of 4, pages 1 and 2
    mapped, D = 64, one head): attending one position returns the V row of the
    source the rule names.  The GPU-side int8 V row of position p is the
    constant 10 + p (scale 1); the host record of p has V codes c = p % 7 - 3
    with group scale 127, which decodes with s' = 7 to rint(127 c / 7) = 18c
    for |c| <= 3, i.e. the value 126 c.  Sinks 0, 1, tail 13..15 and the mapped
    positions 4..11 read 10 + p; the unmapped middle positions 2, 3, 12 read
    126 (p % 7 - 3).  K rows are zero (equal logits)."""
    T, S, L, P, D = 16, 2, 3, 4, 64
    rb = D // 2 + 2
    records = np.zeros((T, 1, 2 * rb), dtype=np.uint8)
    for p in range(T):
        records[p, 0, :rb] = _host_row(np.zeros(D, np.int8), [127.0])
        records[p, 0, rb:] = _host_row(np.full(D, p % 7 - 3, np.int8), [127.0])
    k8 = np.zeros((T, 1, D), np.int8)
    v8 = np.array([np.full((1, D), 10 + p, np.int8) for p in range(T)])
    ones = np.ones((T, 1), np.float16)
    page_block = np.array([-1, 0, 1, -1])
    q = np.ones((1, D), np.float16)
    expect = {0: 10, 1: 11, 2: -126, 3: 0, 4: 14, 5: 15, 6: 16, 7: 17, 8: 18, 9: 19, 10: 20, 11: 21,
              12: 252, 13: 23, 14: 24, 15: 25}
    for p, val in expect.items():
        o = oracle.paged_tier_attention(q, records, k8, v8, ones, ones, np.array([p]), T, S, L,
                                        page_block, P, 0.125, 1, D)
        assert np.all(o == val), (p, o[0, :4])


def test_paged_attention_reduces_to_tier_and_plain_attention():
    """No page mapped: equal bit for bit to tier_attention with the sinks and
    tail of the same int8 cache as its resident rows; every page mapped: equal
    bit for bit to sparse_attention over the int8 cache."""
    rng = np.random.default_rng(32)
    n_kv, G, D, T, S, L, P = 2, 2, 128, 40, 4, 6, 4
    rb = D // 2 + 2 * (D // 64)
    records = rng.integers(0, 256, size=(T, n_kv, 2 * rb), dtype=np.uint8)
    for part in (0, 1):   # finite, positive group scales
        off = part * rb + D // 2
        records[:, :, off:off + 2 * (D // 64)] = (
            rng.uniform(0.01, 2.0, size=(T, n_kv, D // 64)).astype(np.float16).view(np.uint8))
    k8 = rng.integers(-127, 128, size=(T, n_kv, D), dtype=np.int8)
    v8 = rng.integers(-127, 128, size=(T, n_kv, D), dtype=np.int8)
    ks = rng.uniform(0.001, 0.05, size=(T, n_kv)).astype(np.float16)
    vs = rng.uniform(0.001, 0.05, size=(T, n_kv)).astype(np.float16)
    q = rng.standard_normal((n_kv * G, D)).astype(np.float16)
    idx = np.sort(np.concatenate([np.arange(S), rng.choice(np.arange(S, T - L), 12, replace=False),
                                  np.arange(T - L, T)]))
    res = np.concatenate([np.arange(S), np.arange(T - L, T)])
    n_pages = T // P
    none = oracle.paged_tier_attention(q, records, k8, v8, ks, vs, idx, T, S, L, np.full(n_pages, -1), P,
                                       D ** -0.5, G, D)
    tier = oracle.tier_attention(q, records, k8[res], v8[res], ks[res], vs[res], idx, T, S, L, D ** -0.5, G, D)
    assert np.array_equal(none, tier)
    full = oracle.paged_tier_attention(q, records, k8, v8, ks, vs, idx, T, S, L, np.arange(n_pages), P,
                                       D ** -0.5, G, D)
    plain = oracle.sparse_attention(q, k8, v8, ks, vs, idx, D ** -0.5, G, "i8")
    assert np.array_equal(full, plain)
    assert not np.array_equal(none, plain)


def test_clock_fixture():
    lines = list(_lines("clock_trace.txt"))
    n = int(lines[0].split()[1])
    tier = oracle.ClockTier(n, 100, window=1)
    for ln in lines[1:]:
        if ln.startswith("final"):
            assert tier.pos.tolist() == [int(x) for x in ln.split()[1:]]
            continue
        s, picks, slots, hits, misses = (p.strip() for p in ln.split("|"))
        picks = np.array(sorted(int(x) for x in picks.split()))
        got, h, m = tier.step(picks, int(s))
        assert got.tolist() == [int(x) for x in slots.split()], ln
        assert (h, m) == (int(hits), int(misses))


def test_clock_fixture_window_two():
    """Hand trace with W = 2 (tests/golden/clock_trace_w2.txt): slots used in
    the previous step stay pinned, which changes the victims of step 3 against
    W = 1, and a '>=' window test would pin every slot at step 2."""
    lines = list(_lines("clock_trace_w2.txt"))
    head = lines[0].split()
    assert head[0] == "slots" and head[2] == "window"
    tier = oracle.ClockTier(int(head[1]), 100, window=int(head[3]))
    for ln in lines[1:]:
        if ln.startswith("final"):
            assert tier.pos.tolist() == [int(x) for x in ln.split()[1:]]
            continue
        s, picks, slots, hits, misses = (p.strip() for p in ln.split("|"))
        picks = np.array(sorted(int(x) for x in picks.split()))
        got, h, m = tier.step(picks, int(s))
        expect = dict(zip((int(x) for x in sorted(int(y) for y in ln.split("|")[1].split())),
                          (int(x) for x in slots.split())))
        assert got.tolist() == [expect[int(p)] for p in picks], ln
        assert (h, m) == (int(hits), int(misses)), ln


def test_clock_invariants_drifting_workload():
    T, S, L, k = 60_000, 64, 1024, 512
    picks = synth.drift_picks(1, T, S, L, k, 60, seed=77, window=8192, sigma_c=128)
    n_slots = 1500
    tier = oracle.ClockTier(n_slots, T, window=1)
    for s in range(picks.shape[0]):
        before = tier.pos.copy()
        last_before = tier.last.copy()
        slots, h, m = tier.step(picks[s, 0], s)
        assert h + m == k
        assert np.all(tier.pos[slots] == picks[s, 0])            # every pick resident
        assert len(set(slots.tolist())) == k
        occ = tier.pos[tier.pos >= 0]
        assert occ.size <= n_slots and np.unique(occ).size == occ.size
        # a slot used in the previous step (outside the W=1 window now) may be
        # evicted, but never one that a hit of this step used
        evicted = (before >= 0) & (tier.pos != before)
        assert np.all(last_before[evicted] < s)
        # slots used this step by hits are never the victims of this step's misses
        hit_slots = slots[np.isin(picks[s, 0], before)]
        assert np.all(tier.pos[hit_slots] == before[hit_slots])


@pytest.mark.slow
def test_drift_miss_rate_matches_pages():
    """[P1] "The mechanism": misses run at 14-16% with a 2.5% hot buffer.  The
    drifting-locality workload is calibrated so the oracle's CLOCK sees ~15%."""
    T, S, L, k = 250_000, 64, 1024, 2048
    picks = synth.drift_picks(1, T, S, L, k, 192, seed=1005)
    tier = oracle.ClockTier(int(0.025 * T), T, window=1)
    misses = picks_total = 0
    for s in range(picks.shape[0]):
        _, h, m = tier.step(picks[s, 0], s)
        if s >= 64:
            misses += m
            picks_total += h + m
    rate = misses / picks_total
    assert 0.13 <= rate <= 0.17, rate


# --------------------------------------------------------------------------
# append: the new token's int8 K/V rows and int4 key sketch
# --------------------------------------------------------------------------

def _kv(ln):
    return dict(f.split("=", 1) for f in ln.split()[1:])


def test_append_fixture():
    for ln in _lines("append_rows.txt"):
        f = _kv(ln)
        if ln.startswith("row "):
            x = np.array([float(v) for v in f["x"].split(",")], dtype=np.float16)[None]
            codes, s16 = oracle.append.row_i8(x)
            assert int(s16.view(np.uint16)[0]) == int(f["scale"], 16), ln
            assert codes[0].tolist() == [int(v) for v in f["codes"].split(",")], ln
        elif ln.startswith("sketch "):
            k = np.array([float(v) for v in f["k"].split(",")], dtype=np.float16)[None]
            cols = [int(v) for v in f["cols"].split(",")]
            basis = np.zeros((1, k.shape[1], len(cols)), dtype=np.float32)
            for r, c in enumerate(cols):
                basis[0, c, r] = 1.0
            packed, s16 = oracle.append.key_sketch(k, basis)
            assert int(np.array([s16]).view(np.uint16)[0]) == int(f["scale"], 16), ln
            assert packed.tolist() == [int(f["bytes"], 16)], ln
        elif ln.startswith("sketchb "):
            k = np.array([float(v) for v in f["k"].split(",")], dtype=np.float16)[None]
            cols = [_hexf(f["col0"]), _hexf(f["col1"])]
            basis = np.array(cols, dtype=np.float64).T[None]          # [1][D][2]
            assert np.array_equal(basis.astype(np.float32).astype(np.float64), basis), ln
            packed, s16 = oracle.append.key_sketch(k, basis.astype(np.float32))
            assert int(np.array([s16]).view(np.uint16)[0]) == int(f["scale"], 16), ln
            assert packed.tolist() == [int(f["bytes"], 16)], ln


def test_append_row_invariants():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((200, 256)) * rng.uniform(0.01, 30, (200, 1))).astype(np.float16)
    codes, s16 = oracle.append.row_i8(x)
    s = s16.astype(np.float64)
    xf = x.astype(np.float64)
    assert np.abs(codes).max() <= 127
    # the largest element lands on +-127 (up to the fp16 rounding of the scale)
    big = np.abs(codes[np.arange(200), np.abs(xf).argmax(axis=1)])
    assert (big >= 126).all()
    off = np.abs(codes) < 127
    err = np.abs(xf - s[:, None] * codes)
    assert (err[off] <= 0.5 * np.broadcast_to(s[:, None], err.shape)[off] * (1 + 1e-6)).all()


def test_append_sketch_projection_bound():
    """The fp32 projection stays within the fp32 rounding bound of the fp64
    projection, and the int4 codes round-trip through oracle.unpack_int4."""
    rng = np.random.default_rng(6)
    basis = synth.orthonormal_basis(4, 256, 64, 9).numpy().astype(np.float32)
    for _ in range(5):
        k = rng.standard_normal((4, 256)).astype(np.float16)
        packed, s16 = oracle.append.key_sketch(k, basis)
        c = oracle.unpack_int4(packed[None])[0].astype(np.float64)
        v64 = np.einsum("hd,hdr->hr", k.astype(np.float64), basis.astype(np.float64)).reshape(-1)
        s = float(s16)
        assert s > 0 and np.abs(c).max() == 7
        # |v - s*c| <= s/2 + the fp32 accumulation error of 256 terms
        bound = 0.5 * s + 256 * 2.0 ** -23 * np.abs(k.astype(np.float64)).sum(axis=1).max()
        assert np.abs(v64 - s * c).max() <= bound * (1 + 1e-9)


def test_append_bookkeeping():
    B, T, Hkv, D, R = 3, 10, 2, 8, 4
    rng = np.random.default_rng(7)
    caches = dict(codes=np.zeros((B, T, Hkv * R // 2), np.uint8), sk_scale=np.zeros((B, T), np.float16),
                  k=np.zeros((B, T, Hkv, D), np.int8), v=np.zeros((B, T, Hkv, D), np.int8),
                  k_scale=np.zeros((B, T, Hkv), np.float16), v_scale=np.zeros((B, T, Hkv), np.float16))
    before = {n: a.copy() for n, a in caches.items()}
    basis = rng.standard_normal((Hkv, D, R)).astype(np.float32)
    kn = rng.standard_normal((B, Hkv, D)).astype(np.float16)
    vn = rng.standard_normal((B, Hkv, D)).astype(np.float16)
    ctx = oracle.append.append_tokens(np.array([0, 4, T]), kn, vn, basis, caches, T)
    assert ctx.tolist() == [1, 5, T]
    for n, a in caches.items():
        changed = np.argwhere((a != before[n]).reshape(B, T, -1).any(axis=2))
        assert set(map(tuple, changed.tolist())) <= {(0, 0), (1, 4)}, n
    kq, ks = oracle.append.row_i8(kn[1])
    assert np.array_equal(caches["k"][1, 4], kq) and np.array_equal(caches["k_scale"][1, 4], ks)


def _bf16_bits_torch(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_pooled_key_fixture():
    for ln in _lines("append_rows.txt"):
        if not ln.startswith("pool "):
            continue
        f = _kv(ln)
        raw = _bf16_bits_torch([float(v) for v in f["raw"].split(",")])
        raw4 = np.repeat(raw[:, None], 3, axis=1)          # 3 identical columns
        got = oracle.append.pooled_from_raw(raw4)
        assert got.tolist() == [int(f["bits"], 16)] * 3, ln


def test_pooled_key_exact_mean():
    """Against an exact-fraction mean rounded to nearest-even bf16 by hand."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4, 512)) * rng.choice([0.01, 1.0, 50.0], (4, 512))
    raw = _bf16_bits_torch(x.ravel().tolist()).reshape(4, 512)
    got = oracle.append.pooled_from_raw(raw)
    vals = oracle.bf16_to_f64(raw)
    for i in range(512):
        m = sum(Fraction(float(v)) for v in vals[:, i]) / 4
        # nearest bf16 by exhaustive neighbour search around the fp64 value
        t = torch.tensor([float(m)], dtype=torch.float64)
        c0 = t.to(torch.float32).to(torch.bfloat16).to(torch.float64).item()
        ulp = 2.0 ** (np.floor(np.log2(abs(c0))) - 7) if c0 != 0 else 2.0 ** -133
        cands = [c0 - ulp, c0, c0 + ulp]
        best = min(cands, key=lambda c: (abs(Fraction(c) - m), int(torch.tensor([c]).to(torch.bfloat16).view(torch.int16).item()) & 1))
        want = 0.0 if abs(best) < 2.0 ** -8 else max(-255.0, min(255.0, best))
        assert oracle.bf16_to_f64(got[i:i + 1])[0] == want, (i, float(m), best)


def test_append_block_bookkeeping():
    B, T, Hkv, D, ID = 2, 12, 1, 4, 8
    rng = np.random.default_rng(9)
    caches = dict(k=np.zeros((B, T, Hkv, D), np.uint16), v=np.zeros((B, T, Hkv, D), np.uint16),
                  kp=np.zeros((B, T // 4, ID), np.uint16))
    stage = np.zeros((B, 4, ID), np.uint16)
    ctx = np.array([1, T])
    raws = []
    for step in range(3):
        kn = rng.integers(0, 1 << 15, (B, Hkv, D)).astype(np.uint16)
        vn = rng.integers(0, 1 << 15, (B, Hkv, D)).astype(np.uint16)
        raw = _bf16_bits_torch(rng.standard_normal(B * ID).tolist()).reshape(B, ID)
        raws.append(raw[0].copy())
        ctx = oracle.append.append_block_tokens(ctx, kn, vn, raw, stage, caches, T)
        assert np.array_equal(caches["k"][0, step + 1], kn[0])
        assert not caches["k"][1].any()                       # full sequence untouched
        if step < 2:
            assert not caches["kp"][0].any()                  # block 0 not complete yet
    assert ctx.tolist() == [4, T]
    # block 0 = tokens 0..3: slot 0 was never written in this test (zeros), 1..3 from the steps
    want = oracle.append.pooled_from_raw(np.stack([np.zeros(ID, np.uint16)] + raws))
    assert np.array_equal(caches["kp"][0, 0], want)


# --------------------------------------------------------------------------
# multi-query decode (verification tokens)
# --------------------------------------------------------------------------

def _mq_case(T, lens, M, S, k, L, seed, fmt="i8"):
    c = synth.make_token_case(len(lens), T, lens, n_kv=2, n_q=6, D=64, S=S, k=k, L=L,
                              kv_format=fmt, n_needles=0, seed=seed)
    q = synth.multi_queries(len(lens), M, 6, 64, seed)
    return c, q


def _run_mq(c, q, M, fmt="i8", sm=0.125):
    ks = None if c.k_scale is None else c.k_scale.numpy()
    vs = None if c.v_scale is None else c.v_scale.numpy()
    return oracle.multiquery.token_step_multi(
        q.numpy(), c.basis.numpy(), c.codes.numpy(), c.sk_scale.numpy(), c.k_cache.numpy(),
        c.v_cache.numpy(), ks, vs, c.lens, M=M, S=c.S, k_top=c.k, L=c.L, group=c.group,
        sm_scale=sm, fmt=fmt)


@pytest.mark.parametrize("fmt", ["i8", "f16"])
def test_multi_dense_equals_causal_attention(fmt):
    """With every query below the budget, the M outputs equal torch's fp64
    scaled_dot_product_attention of the M queries over the cache with a causal
    mask (query j sees positions 0 .. T-M+j)."""
    M, T = 5, 60
    c, q = _mq_case(T, [T, T - 9], M, S=4, k=50, L=8, seed=31, fmt=fmt)
    _, _, idx, out = _run_mq(c, q, M, fmt)
    for b in range(c.B):
        Tb = c.lens[b]
        kd = c.k_cache[b, :Tb].double()
        vd = c.v_cache[b, :Tb].double()
        if fmt == "i8":
            kd = kd * c.k_scale[b, :Tb].double().unsqueeze(-1)
            vd = vd * c.v_scale[b, :Tb].double().unsqueeze(-1)
        kk = kd.permute(1, 0, 2).repeat_interleave(c.group, dim=0)   # [H_q][T][D]
        vv = vd.permute(1, 0, 2).repeat_interleave(c.group, dim=0)
        qq = q[b].double().permute(1, 0, 2)                          # [H_q][M][D]
        pos = torch.arange(Tb)
        mask = pos[None, :] <= (Tb - M + torch.arange(M))[:, None]   # [M][T]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask,
                                                               scale=0.125)
        np.testing.assert_allclose(out[b], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        for j in range(M):
            assert np.array_equal(idx[b][j], np.arange(Tb - M + 1 + j))


def test_multi_last_query_is_the_single_step():
    """The last query token sees the whole cache: its pick and output are the
    single-query step's at ctx_len."""
    M, T = 4, 700
    c, q = _mq_case(T, [T, 613], M, S=8, k=64, L=16, seed=32)
    qs, qsc, idx, out = _run_mq(c, q, M)
    ks, vs = c.k_scale.numpy(), c.v_scale.numpy()
    s_qs, s_qsc, _, s_idx, s_out = oracle.token_step(
        q[:, M - 1].numpy(), c.basis.numpy(), c.codes.numpy(), c.sk_scale.numpy(),
        c.k_cache.numpy(), c.v_cache.numpy(), ks, vs, c.lens, S=c.S, k_top=c.k, L=c.L,
        group=c.group, sm_scale=0.125, fmt="i8")
    assert np.array_equal(qs[:, M - 1], s_qs) and np.array_equal(qsc[:, M - 1], s_qsc)
    for b in range(c.B):
        assert np.array_equal(idx[b][M - 1], s_idx[b])
        assert np.array_equal(out[b, M - 1], s_out[b])


def test_multi_picks_stay_causal():
    """Every pick of query j lies in its context T_j = T-M+1+j, holds its own
    sinks and tail, and has min(T_j, S+k+L) positions; a budget threshold
    crossed inside one step (S+k+L = 28, T = 30, M = 4) leaves the first two
    queries dense and the last two sparse; a context shorter than M leaves the
    first queries empty."""
    S, k, L, M = 4, 16, 8, 4
    c, q = _mq_case(40, [30, 3], M, S=S, k=k, L=L, seed=33)
    _, _, idx, out = _run_mq(c, q, M)
    assert oracle.multiquery.query_contexts(30, M) == [27, 28, 29, 30]
    assert oracle.multiquery.query_contexts(3, M) == [0, 1, 2, 3]
    for b in range(c.B):
        for j, Tj in enumerate(oracle.multiquery.query_contexts(c.lens[b], M)):
            sel = idx[b][j]
            assert len(sel) == min(Tj, S + k + L)
            assert np.all(np.diff(sel) > 0) and (len(sel) == 0 or sel[-1] < Tj)
            if Tj > S + k + L:
                assert set(range(S)) <= set(sel.tolist())
                assert set(range(Tj - L, Tj)) <= set(sel.tolist())
            else:
                assert np.array_equal(sel, np.arange(Tj))
            if Tj == 0:
                assert not out[b, j].any()
    assert [len(idx[0][j]) for j in range(M)] == [27, 28, 28, 28]


def test_multi_equal_queries_nested_picks():
    """M copies of one query: each step of the causal context moves one
    position from the tail into the ranked middle, so consecutive picks differ
    by at most that position coming in and one ranked position going out."""
    S, k, L, M, T = 4, 32, 8, 6, 900
    c, _ = _mq_case(T, [T], M, S=S, k=k, L=L, seed=34)
    q1 = synth.multi_queries(1, 1, 6, 64, 35)
    q = q1.expand(1, M, 6, 64).contiguous()
    _, _, idx, _ = _run_mq(c, q, M)
    for j in range(M - 1):
        Tj = T - M + 1 + j
        mid_a = set(idx[0][j].tolist()) - set(range(S)) - set(range(Tj - L, Tj))
        mid_b = set(idx[0][j + 1].tolist()) - set(range(S)) - set(range(Tj + 1 - L, Tj + 1))
        assert len(mid_a) == len(mid_b) == k
        assert mid_b - mid_a <= {Tj - L}
        assert len(mid_a - mid_b) == len(mid_b - mid_a)


# --------------------------------------------------------------------------
# prefill attention over host-resident K/V
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_prefill_attention_is_masked_sdpa(fmt):
    """Each prefill query attends exactly its own listed rows: all P outputs at
    once equal torch's fp64 SDPA with a boolean mask built from the lists; an
    empty list gives zeros."""
    T, P, n_kv, n_q, D = 700, 12, 2, 8, 64
    g = torch.Generator().manual_seed(41)
    k = torch.randn((T, n_kv, D), generator=g)
    v = torch.randn((T, n_kv, D), generator=g)
    q = torch.randn((P, n_q, D), generator=g)
    idx, n_sel = synth.prefill_picks(P, T, 24, 42)
    n_sel[3] = 0
    lists = [idx[p, :n_sel[p]].astype(np.int64) for p in range(P)]
    if fmt == "bf16":
        kb, vb, qb = (x.to(torch.bfloat16) for x in (k, v, q))
        args = [x.view(torch.int16).numpy().view(np.uint16) for x in (qb, kb, vb)]
    else:
        kb, vb, qb = (x.to(torch.float16) for x in (k, v, q))
        args = [x.numpy() for x in (qb, kb, vb)]
    out = oracle.prefill.prefill_attention(args[0], args[1], args[2], lists, 0.125, n_q // n_kv, fmt)
    mask = torch.zeros((P, T), dtype=torch.bool)
    for p in range(P):
        mask[p, lists[p]] = True
    kk = kb.double().permute(1, 0, 2).repeat_interleave(n_q // n_kv, dim=0)   # [H_q][T][D]
    vv = vb.double().permute(1, 0, 2).repeat_interleave(n_q // n_kv, dim=0)
    qq = qb.double().permute(1, 0, 2)                                          # [H_q][P][D]
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=0.125)
    ref = ref.permute(1, 0, 2).numpy()
    for p in range(P):
        if n_sel[p] == 0:
            assert not out[p].any()
        else:
            np.testing.assert_allclose(out[p], ref[p], rtol=0, atol=1e-12)


def test_prefill_transfer_closed_forms():
    """[P4] "The Downside to Keep in Mind": a 4096-token prefill chunk whose
    tokens each fetch their own 2048 picks moves 4096 x 2048 x 24 KiB (K and V,
    2 KV heads x 256 x bf16, 12 layers) = 192 GiB (the page prints 204 GiB,
    kept as an unreconciled figure); 256 such chunks for 1 Mi tokens take about
    half an hour at 26 GB/s; the chunk loop moves each history row once,
    independent of the working-buffer size."""
    per_layer = oracle.prefill.per_token_transfer_bytes([2048] * 4096, 2, 256, 2)
    assert 12 * per_layer == 192 * 1024 * MiB
    minutes = 256 * 12 * per_layer / 26e9 / 60
    assert 25 <= minutes <= 40
    T = 1 << 20
    once = oracle.prefill.chunked_transfer_bytes(T, 2, 256, 2)
    assert once == 2 * 1024 * MiB and 12 * once == 24 * 1024 * MiB
    assert per_layer // once == 8   # 4096 x 2048 picks vs 1 Mi rows


# --------------------------------------------------------------------------
# LRU hot buffer (HiSparse-style residency)
# --------------------------------------------------------------------------

def test_lru_fixture():
    lines = list(_lines("lru_trace.txt"))
    n = int(lines[0].split()[1])
    tier = oracle.residency.LruTier(n, 100)
    for ln in lines[1:]:
        if ln.startswith("final"):
            assert tier.pos.tolist() == [int(x) for x in ln.split()[1:]]
            continue
        s, picks, slots, hits, misses = (p.strip() for p in ln.split("|"))
        picks = np.array(sorted(int(x) for x in picks.split()))
        got, h, m = tier.step(picks, int(s))
        assert got.tolist() == [int(x) for x in slots.split()], ln
        assert (h, m) == (int(hits), int(misses))


def test_lru_invariants_drifting_workload():
    """Over a drifting-locality pick schedule: hits + misses = picks, the
    buffer never holds more than its slots, no slot used in the current step
    is evicted, nothing is evicted while a slot is empty, and no slot kept
    unused is older than an evicted one (ties by slot index)."""
    T, S, L, k = 60_000, 64, 1024, 512
    picks = synth.drift_picks(1, T, S, L, k, 60, seed=44, window=8192, sigma_c=256.0)
    n_slots = 2 * k
    tier = oracle.residency.LruTier(n_slots, T)
    for s in range(60):
        p = np.asarray(picks[s][0], dtype=np.int64)
        before_pos = tier.pos.copy()
        before_last = tier.last.copy()
        slots, h, m = tier.step(p, s)
        assert h + m == p.size and (tier.pos >= 0).sum() <= n_slots
        assert len(set(slots.tolist())) == p.size
        changed = np.nonzero(tier.pos != before_pos)[0]
        evicted = [x for x in changed.tolist() if before_pos[x] >= 0]
        if evicted:
            assert (tier.pos >= 0).all()                         # no slot left empty
            used_now = set(slots.tolist())
            kept_unused = [x for x in range(n_slots) if x not in used_now]
            oldest_kept = min(((before_last[x], x) for x in kept_unused), default=None)
            newest_evicted = max((before_last[x], x) for x in evicted)
            assert oldest_kept is None or newest_evicted < oldest_kept
        assert set(tier.pos[tier.pos >= 0].tolist()) >= set(p.tolist())


# --------------------------------------------------------------------------
# host record of an appended token (tier append)
# --------------------------------------------------------------------------

def _group_values(spec):
    x = np.zeros(64, dtype=np.float16)
    if spec.startswith("all:"):
        x[:] = float(spec[4:])
    elif spec:
        for item in spec.split(","):
            i, v = item.split(":")
            x[int(i)] = float(v)
    return x


def _group_bytes(spec):
    items = spec.split(",")
    out = []
    for it in items:
        if it.endswith("..."):
            b = int(it[:-3], 16)
            out += [b] * (32 - len(out))
        else:
            out.append(int(it, 16))
    assert len(out) == 32
    return out


def test_host_record_fixture():
    groups = [_kv(ln) for ln in _lines("host_record_i4.txt") if ln.startswith("group ")]
    assert len(groups) == 4
    row = np.concatenate([_group_values(g["nz"]) for g in groups])
    got = oracle.append.host_row_i4(row)
    assert got.size == 256 // 2 + 2 * 4
    for gi, g in enumerate(groups):
        assert got[32 * gi:32 * gi + 32].tolist() == _group_bytes(g["bytes"]), gi
        assert int(got[128:].view(np.uint16)[gi]) == int(g["scale"], 16), gi


def test_host_record_invariants():
    """Codes decoded by oracle.unpack_int4 (written independently of the
    packer) reconstruct each group within half a step; the largest element of
    a group lands on +-7; the fetch decoder (oracle.host_row_dequant) turns the
    record into an int8 row within its own rounding bound."""
    rng = np.random.default_rng(31)
    D = 256
    for trial in range(60):
        x = (rng.standard_normal(D) * rng.uniform(0.001, 40.0, D // 64).repeat(64)).astype(np.float16)
        if trial % 10 == 0:
            x[64:128] = 0
        rec = oracle.append.host_row_i4(x)
        c = oracle.unpack_int4(rec[:D // 2]).astype(np.float64)
        g = rec[D // 2:].view(np.float16).astype(np.float64)
        xf = x.astype(np.float64)
        for gi in range(D // 64):
            xs, cs, gs = xf[64 * gi:64 * gi + 64], c[64 * gi:64 * gi + 64], g[gi]
            amax = np.abs(xs).max()
            if amax == 0:
                assert gs == 0 and not cs.any()
                continue
            assert abs(gs - amax / 7) <= amax / 7 * 2.0 ** -11 * 1.0001   # one fp16 rounding
            assert np.abs(cs).max() <= 7 and np.abs(cs[np.argmax(np.abs(xs))]) == 7
            assert np.all(np.abs(xs - gs * cs) <= gs / 2 * (1 + 1e-6))
        r8, sp = oracle.host_row_dequant(rec, D)
        gmax = g.max()
        if gmax > 0:
            recon = r8.astype(np.float64) * float(sp)
            assert np.all(np.abs(xf - recon) <= g.repeat(64) / 2 + float(sp) / 2 + 1e-9 + gmax * 2.0 ** -9)


def test_tier_append_token_layout():
    """Five appends on a toy tier (S=2, L=3, one KV head, D=64): the sinks stay,
    the tail holds the last three appended int8 rows in position order, and
    only the appended positions' records are written."""
    rng = np.random.default_rng(32)
    S, L, H, D, cap, T0 = 2, 3, 1, 64, 20, 10
    rb = D // 2 + 2 * (D // 64)
    rec = np.zeros((cap, H, 2 * rb), dtype=np.uint8)
    res_k = np.arange((S + L) * H * D, dtype=np.int64).reshape(S + L, H, D).astype(np.int8)
    res_v = -res_k
    res_ks = np.arange(S + L, dtype=np.float16).reshape(S + L, 1) + np.float16(1)
    res_vs = res_ks * np.float16(2)
    sinks = (res_k[:S].copy(), res_v[:S].copy(), res_ks[:S].copy(), res_vs[:S].copy())
    T = T0
    news = []
    for _ in range(5):
        k16 = rng.standard_normal((H, D)).astype(np.float16)
        v16 = rng.standard_normal((H, D)).astype(np.float16)
        T = oracle.append.tier_append_token(T, rec, res_k, res_v, res_ks, res_vs, S, L, k16, v16)
        news.append((k16, v16))
    assert T == T0 + 5
    for a, b in zip((res_k[:S], res_v[:S], res_ks[:S], res_vs[:S]), sinks):
        assert np.array_equal(a, b)
    for i, (k16, v16) in enumerate(news[-L:]):
        kq, ks = oracle.append.row_i8(k16)
        vq, vs = oracle.append.row_i8(v16)
        assert np.array_equal(res_k[S + i], kq) and np.array_equal(res_ks[S + i], ks)
        assert np.array_equal(res_v[S + i], vq) and np.array_equal(res_vs[S + i], vs)
    for p in range(cap):
        if T0 <= p < T:
            k16, v16 = news[p - T0]
            want = np.concatenate([oracle.append.host_row_i4(k16[0]), oracle.append.host_row_i4(v16[0])])
            assert np.array_equal(rec[p, 0], want)
        else:
            assert not rec[p].any()


# --------------------------------------------------------------------------
# several query tokens through the host tier
# --------------------------------------------------------------------------

def _overlapping_lists(rng, M, T, S, L, k, shared):
    """M ascending middle lists sharing `shared` positions of each list."""
    base = rng.choice(np.arange(S, T - L), k, replace=False)
    lists = []
    for _ in range(M):
        own = rng.choice(np.setdiff1d(np.arange(S, T - L), base), k - shared, replace=False)
        lists.append(np.sort(np.concatenate([base[:shared], own])))
    return lists


@pytest.mark.parametrize("lru", [False, True])
def test_tier_lists_single_equals_step(lru):
    rng = np.random.default_rng(61)
    T, S, L, k, n = 5000, 16, 32, 64, 160
    mk = (lambda: oracle.residency.LruTier(n, T)) if lru else (lambda: oracle.ClockTier(n, T, window=1))
    a, b = mk(), mk()
    for s in range(12):
        lst = np.sort(rng.choice(np.arange(S, T - L), k, replace=False))
        sl_a, h_a, m_a = a.step(lst, s)
        (sl_b,), h_b, m_b = oracle.multiquery.tier_resolve_lists(b, [lst], T, S, L, s)
        assert np.array_equal(sl_a, sl_b) and (h_a, m_a) == (h_b, m_b)


@pytest.mark.parametrize("lru", [False, True])
def test_tier_lists_all_resident_and_fetched_once(lru):
    """After a step that filled the hot buffer with other rows, lists sharing
    positions: every pick of every list is resident afterwards in the slot
    reported for it, and a shared position is fetched once."""
    rng = np.random.default_rng(62)
    T, S, L, k, M, shared = 20_000, 16, 32, 64, 4, 40
    lists = _overlapping_lists(rng, M, T, S, L, k, shared)
    distinct = np.unique(np.concatenate(lists))
    n = distinct.size + 1
    tier = oracle.residency.LruTier(n, T) if lru else oracle.ClockTier(n, T, window=1)
    filler = np.sort(rng.choice(np.setdiff1d(np.arange(S, T - L), distinct), n - 1, replace=False))
    tier.step(filler, 0)
    slots, h, m = oracle.multiquery.tier_resolve_lists(tier, lists, T, S, L, 1)
    assert m == distinct.size and h == sum(l.size for l in lists) - distinct.size
    for sl, l in zip(slots, lists):
        assert np.array_equal(tier.pos[sl], l)


@pytest.mark.parametrize("lru", [False, True])
def test_tier_lists_must_fit_together(lru):
    """Each list fits the hot buffer but their union does not: resolving them
    at one step is refused (the buffer cannot hold every query's rows at
    once), whereas a step number per list would quietly evict rows an earlier
    query still needs."""
    rng = np.random.default_rng(63)
    T, S, L, k, M, shared = 20_000, 16, 32, 64, 4, 40
    lists = _overlapping_lists(rng, M, T, S, L, k, shared)
    n = np.unique(np.concatenate(lists)).size - 1
    mk = (lambda: oracle.residency.LruTier(n, T)) if lru else (lambda: oracle.ClockTier(n, T, window=1))
    with pytest.raises(RuntimeError):
        oracle.multiquery.tier_resolve_lists(mk(), lists, T, S, L, 0)
    tier = mk()
    for j, l in enumerate(lists):
        tier.step(l, j)
    assert not np.isin(lists[0], tier.pos).all()


def test_tier_lists_classify_against_tier_context():
    """A later query's tail position below T - L is a middle row of the tier."""
    T, S, L = 1000, 4, 8
    tier = oracle.ClockTier(20, T, window=1)
    lists = [np.concatenate([np.arange(S), [100, 200], np.arange(T - 1 - L, T - 1)]),
             np.concatenate([np.arange(S), [100, 300], np.arange(T - L, T)])]
    slots, h, m = oracle.multiquery.tier_resolve_lists(tier, lists, T, S, L, 0)
    assert [sl.size for sl in slots] == [3, 2]        # T - 1 - L is middle for the tier
    assert (h, m) == (1, 4)
