"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded bytes.  Index sets, query sketches and ranking keys must match
bit for bit; attention outputs within 2e-3 max abs error of the fp64 oracle.

Sizes span several score / select / attention tiles with ragged tails, the
dense/sparse boundaries, empty and tiny sequences, and the full workload
shapes (sampled sequences)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (ATOL, block_desc_of, compare_keys, compare_out, compare_sel, need_gpu,
                      np16, oracle_block, oracle_token, run_block_gpu, run_token_gpu, say,
                      token_desc_of)

pytestmark = pytest.mark.gpu


def _cfg1(B=1, T=4096, lens=None, seed=1001, **kw):
    return synth.make_token_case(B, T, lens, n_kv=2, n_q=8, D=128, S=16, k=256, L=128,
                                 kv_format="f16", seed=seed, **kw)


def _cfg2(B, T, lens=None, seed=1002, device="cpu", **kw):
    return synth.make_token_case(B, T, lens, n_kv=4, n_q=24, D=256, S=64, k=2048, L=1024,
                                 kv_format="i8", seed=seed, device=device, **kw)


def _cfg3(B, T, lens=None, seed=1003, device="cpu", **kw):
    return synth.make_block_case(B, T, lens, n_kv=2, n_q=16, D=256, k=512, seed=seed,
                                 device=device, **kw)


def _check_token(c, g, o, seqs=None, sm=None):
    seqs = range(c.B) if seqs is None else seqs
    assert np.array_equal(g["qs"], o["qs"]), "query sketch codes differ"
    assert np.array_equal(g["qscale"].view(np.uint32), o["qscale"].view(np.uint32)), "qscale differs"
    errs = []
    for b in seqs:
        T = c.lens[b]
        compare_keys(g["keys"], o["keys"], b, c.S, max(c.S, T - c.L))
        compare_sel(g, o, b)
        errs.append(compare_out(g, o, b))
        if len(c.needles[b]):
            assert np.isin(c.needles[b].numpy(), g["idx"][b, :g["n_sel"][b]]).all()
    return max(errs) if errs else 0.0


def test_config1_tiny_layer():
    skv = need_gpu()
    c = _cfg1()
    sm = 128 ** -0.5
    say("cfg1 B=1 T=4096")
    g = run_token_gpu(skv, c, sm)
    o = oracle_token(c, sm)
    err = _check_token(c, g, o)
    say("cfg1 max err", err)


@pytest.mark.parametrize("fused", [False, True])
def test_config2_shape_ragged(fused):
    """cfg-2 layer shape, 3 sequences with ragged lengths spanning several
    score / histogram tiles, one dense sequence, plus the boundary lengths."""
    skv = need_gpu()
    lens = [40_000, 3_137, 17_001, 3_136, 3_135]
    c = _cfg2(5, 40_960, lens)
    sm = 256 ** -0.5
    say("cfg2 ragged", lens, "fused", fused)
    g = run_token_gpu(skv, c, sm, fused=fused)
    o = oracle_token(c, sm)
    err = _check_token(c, g, o)
    assert g["n_sel"].tolist() == [3136, 3136, 3136, 3136, 3135]
    say("cfg2 ragged max err", err)


def test_config3_shape_boundaries():
    """QSA layer shape in block mode; dense until T > 4*512+3 = 2051."""
    skv = need_gpu()
    lens = [65_536, 2_051, 2_052, 2_053, 30_001, 4]
    c = _cfg3(len(lens), 65_536, lens)
    sm = 256 ** -0.5
    say("cfg3 boundaries", lens)
    g = run_block_gpu(skv, c, sm)
    o = oracle_block(c, sm)
    for b in range(c.B):
        compare_keys(g["keys"], o["keys"], b, 0, c.lens[b] // 4)
        compare_sel(g, o, b)
        compare_out(g, o, b)
    assert g["n_sel"].tolist() == [2048, 2051, 2048, 2049, 2049, 4]
    # needles (whole blocks) recovered
    for blk in c.needles[0].tolist():
        assert 4 * blk in set(g["idx"][0, :2048].tolist())


def test_pooled_keys_out_of_domain():
    """Block mode outside the bf16 range where an fp64 sum of products is
    exact in any order (the generator's inputs are flushed into it): inputs
    spanning 2^-20 .. 2^10, so products span about 60 bits.  Each product of
    two bf16 values is exact in fp32; the kernel sums them in fp64 in its own
    order, so a key is the exact dot product within the fp64 summation bound
    (127 units of 2^-53 times the sum of the products' magnitudes), and the
    picks are a top-k of the exact keys up to that bound.  Bit-exact parity is
    claimed inside the domain only."""
    import math
    skv = need_gpu()
    c = _cfg3(1, 40_000, device="cuda")
    g = torch.Generator().manual_seed(21)
    def wide(shape):
        e = torch.randint(-20, 10, shape, generator=g).to(torch.float32)
        return (torch.randn(shape, generator=g) * torch.exp2(e)).to(torch.bfloat16)
    c.qi = wide(tuple(c.qi.shape)).cuda()
    c.kp = wide(tuple(c.kp.shape)).cuda()
    say("pooled keys out of domain")
    gres = run_block_gpu(skv, c, 256 ** -0.5)
    nb = c.lens[0] // 4
    qi = c.qi[0].float().cpu().numpy().astype(np.float64)
    kp = c.kp[0, :nb].float().cpu().numpy().astype(np.float64)
    prods = kp * qi[None, :]                      # exact: two bf16 values
    exact = np.array([math.fsum(r) for r in prods])
    bound = 127 * 2.0 ** -53 * np.abs(prods).sum(axis=1)
    gk = gres["keys"][0, :nb]
    assert np.all(np.abs(gk - exact) <= bound), "a key outside the fp64 summation bound"
    # the picked blocks are a top-k of the exact keys, up to the bound
    n = int(gres["n_sel"][0])
    picked = np.unique(gres["idx"][0, :n] // 4)
    picked = picked[picked < nb]
    assert picked.size == c.k
    kth = np.sort(exact)[-c.k]
    slack = 2 * bound.max()
    assert exact[picked].min() >= kth - slack
    others = np.setdiff1d(np.arange(nb), picked)
    assert exact[others].max() <= kth + slack
    say("out of domain: max key error %.3g (bound %.3g)" % (np.abs(gk - exact).max(), bound.max()))


def test_empty_and_tiny_sequences():
    skv = need_gpu()
    lens = [0, 1, 2, 399, 400, 401, 1000]
    c = _cfg1(len(lens), 1024, lens, n_needles=0)
    sm = 0.1
    g = run_token_gpu(skv, c, sm)
    o = oracle_token(c, sm)
    _check_token(c, g, o)
    assert g["n_sel"].tolist() == [0, 1, 2, 399, 400, 400, 400]
    assert not g["out"][0].any()


@pytest.mark.parametrize("fused", [True, False])
def test_other_head_shapes(fused):
    """Sketch widths other than the cfg-2 one: 2 KV heads (64-byte rows, 4
    lanes per token) with 16 query heads each, and 8 KV heads (256-byte rows,
    16 lanes per token) with one query head each, fp16 K/V at head_dim 128."""
    skv = need_gpu()
    sm = 0.0625
    c = synth.make_token_case(2, 30_000, [30_000, 21_111], n_kv=2, n_q=32, D=256, S=16, k=512,
                              L=256, kv_format="i8", seed=71)
    say("2 KV x 16 q heads, fused", fused)
    g = run_token_gpu(skv, c, sm, fused=fused)
    _check_token(c, g, oracle_token(c, sm))
    c = synth.make_token_case(2, 30_000, [30_000, 9_999], n_kv=8, n_q=8, D=128, S=8, k=1024,
                              L=64, kv_format="f16", seed=72)
    say("8 KV x 1 q head, fused", fused)
    g = run_token_gpu(skv, c, sm, fused=fused)
    _check_token(c, g, oracle_token(c, sm))


def test_largest_context_and_budget():
    """The largest supported context (2,097,152 tokens: 8192 segments of 256)
    with the largest budget (k = 4096), cfg-2 layer shape, one sequence."""
    skv = need_gpu()
    T = 2_097_152
    say("largest context: generating 1 x", T)
    c = synth.make_token_case(1, T, None, n_kv=4, n_q=24, D=256, S=64, k=4096, L=1024,
                              kv_format="i8", seed=73, device="cuda")
    sm = 256 ** -0.5
    g = run_token_gpu(skv, c, sm, fused=True)
    say("largest context: oracle")
    o = oracle_token(c, sm)
    err = _check_token(c, g, o)
    assert g["n_sel"].tolist() == [64 + 4096 + 1024]
    # the capped sample lets about 9,000 candidates through at this budget:
    # more than the LDS lists hold (8,192), within the register path (12,288)
    assert g["flags"] == 0, g["flags"]
    say("largest context max err", err, "flags", g["flags"])


@pytest.mark.parametrize("case", ["two_clusters", "all_equal", "mid_bucket", "mid_bucket_regs"])
def test_topk_register_path_capacity(case):
    """Between 8,192 and 12,288 candidates the select keeps them in
    registers, and threshold buckets of up to 1,024 members are ranked
    pairwise.  two_clusters: 2,000 keys above 8,000 distinct keys of one
    threshold bucket, all kept as candidates, the bucket ranked in full;
    all_equal: 10,000 equal keys, one bucket larger than its LDS member list,
    so the exact path over the records runs (informational flag); mid_bucket:
    1,500 keys above a bucket of 700 distinct keys that holds the k-th
    largest (one thread per member) and 1,500 lower candidates, all in the
    LDS list; mid_bucket_regs: the same with 9,000 lower candidates, so the
    candidates sit in registers."""
    skv = need_gpu()
    S, k, L = 64, 2048, 1024
    T = {"two_clusters": 12_000, "all_equal": 11_088, "mid_bucket": 20_000, "mid_bucket_regs": 20_000}[case]
    desc = skv.token_desc(1, T, 4, 24, 256, topk=k, n_sink=S, n_tail=L)
    keys = np.ones((1, T))
    mid = np.arange(S, T - L)
    if case == "two_clusters":
        keys[0, mid[:2000]] = 10.0 + 1e-6 * np.arange(2000)
        keys[0, mid[2000:10000]] = 5.0 + 1e-9 * np.arange(8000)
    elif case == "all_equal":
        keys[0] = 3.0
    else:
        # interleaved so that every sampled line sees all three groups
        rng = np.random.default_rng(11)
        sel = rng.permutation(mid.size)
        top, bucket = mid[sel[:1500]], mid[sel[1500:2200]]
        keys[0, top] = 10.0 + 1e-6 * np.arange(1500)
        keys[0, bucket] = 5.0 + 1e-9 * rng.permutation(700)
        # below the bucket, the keys the threshold lands among (all kept as
        # candidates): 1,500 (candidates in the LDS list) or 9,000 (in registers)
        n3 = 9000 if case == "mid_bucket_regs" else 1500
        keys[0, mid[sel[2200:2200 + n3]]] = (4.9 if n3 == 9000 else 3.0) + 1e-9 * np.arange(n3)
    kt = torch.from_numpy(keys).cuda()
    ctx = torch.full((1,), T, dtype=torch.int32, device="cuda")
    cap = skv.select_capacity(desc)
    idx = torch.zeros((1, cap), dtype=torch.int32, device="cuda")
    nsel = torch.zeros((1,), dtype=torch.int32, device="cuda")
    ws = skv.workspace(desc)
    skv.topk(desc, ctx, kt, idx, nsel, ws)
    flags = skv.check(ws)
    want = oracle.select_tokens(keys[0], T, S, k, L)
    assert nsel[0].item() == want.size
    assert np.array_equal(idx.cpu().numpy()[0, :want.size], want)
    if case == "all_equal":
        assert flags == skv.SKV_FLAG_TOPK_SLOW, flags
    else:
        assert flags == 0, flags


def test_topk_ties_and_degenerate_keys():
    """Keys fed straight to sparsekv_topk: many exact ties, all-equal keys (the
    exact slow path), negative keys, and a single huge key."""
    skv = need_gpu()
    B, T = 6, 50_000
    S, k, L = 64, 2048, 1024
    desc = skv.token_desc(B, T, 4, 24, 256, topk=k, n_sink=S, n_tail=L)
    rng = np.random.default_rng(5)
    keys = np.zeros((B, T))
    keys[0] = rng.integers(-3, 4, size=T)                    # heavy ties
    keys[1] = 0.0                                            # all equal -> slow path
    keys[2] = -rng.random(T)                                 # all negative
    keys[3] = rng.standard_normal(T)
    keys[3, 12345] = 1e300
    keys[4] = np.round(rng.standard_normal(T) * 8) / 8       # coarse grid, ties
    keys[5] = -0.0                                           # negative zeros
    kt = torch.from_numpy(keys).cuda()
    ctx = torch.full((B,), T, dtype=torch.int32, device="cuda")
    cap = skv.select_capacity(desc)
    idx = torch.zeros((B, cap), dtype=torch.int32, device="cuda")
    nsel = torch.zeros((B,), dtype=torch.int32, device="cuda")
    ws = skv.workspace(desc)
    skv.topk(desc, ctx, kt, idx, nsel, ws)
    flags = skv.check(ws)
    assert flags & skv.SKV_FLAG_TOPK_SLOW
    gi = idx.cpu().numpy()
    for b in range(B):
        want = oracle.select_tokens(keys[b], T, S, k, L)
        assert nsel[b].item() == want.size
        assert np.array_equal(gi[b, :want.size], want), "sequence %d" % b


def test_determinism_and_graph_replay():
    """Two eager runs are bitwise identical; a captured HIP graph of the whole
    step replayed several times gives the eager result every time."""
    skv = need_gpu()
    c = _cfg2(3, 20_000, [20_000, 9_000, 3_000], device="cuda")
    sm = 256 ** -0.5
    a = run_token_gpu(skv, c, sm, fused=True)
    b = run_token_gpu(skv, c, sm, fused=True)
    for key in ("qs", "qscale", "idx", "n_sel", "out"):
        assert np.array_equal(a[key], b[key]), key
    desc = token_desc_of(skv, c)
    cap = skv.select_capacity(desc)
    ws = skv.workspace(desc)
    qs = torch.zeros((c.B, 256), dtype=torch.int8, device="cuda")
    qsc = torch.zeros((c.B,), dtype=torch.float32, device="cuda")
    idx = torch.zeros((c.B, cap), dtype=torch.int32, device="cuda")
    nsel = torch.zeros((c.B,), dtype=torch.int32, device="cuda")
    out = torch.zeros((c.B, c.n_q, c.D), dtype=torch.float32, device="cuda")
    kv = skv.kv_view(c.k_cache, c.v_cache, c.k_scale, c.v_scale)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on the capture stream
        skv.step(desc, c.ctx_len, c.q, c.basis, qs, qsc, None, c.codes, c.sk_scale, kv, idx,
                 nsel, sm, out, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        skv.step(desc, c.ctx_len, c.q, c.basis, qs, qsc, None, c.codes, c.sk_scale, kv, idx,
                 nsel, sm, out, ws)
    for rep in range(4):
        out.zero_()
        idx.zero_()
        graph.replay()
        torch.cuda.synchronize()
        _ = (out * 2).sum().item()   # unrelated eager work between replays
        assert np.array_equal(out.cpu().numpy().astype(np.float64), a["out"]), "replay %d" % rep
        for bb in range(c.B):
            n = int(a["n_sel"][bb])
            assert np.array_equal(idx.cpu().numpy()[bb, :n], a["idx"][bb, :n])


def test_micro_batches_on_streams():
    """The batch split into micro-batches of consecutive sequences, each on its
    own stream with its own workspace, several layer-steps in a row: every
    sequence gets the same picks and outputs as in the one-call step, and the
    outputs match the oracle."""
    skv = need_gpu()
    lens = [20_000, 9_000, 3_000, 15_500, 20_000, 3_136]
    c = _cfg2(6, 20_000, lens, device="cuda")
    sm = 256 ** -0.5
    say("micro-batches", lens)
    a = run_token_gpu(skv, c, sm, fused=True)
    o = oracle_token(c, sm)
    cap = skv.select_capacity(token_desc_of(skv, c))
    for m in (2, 3):
        g = _run_micro_batches(skv, c, sm, m, reps=3, flags=a["flags"])
        assert np.array_equal(g["qs"], a["qs"])
        assert np.array_equal(g["n_sel"], a["n_sel"])
        for b in range(c.B):
            n = int(a["n_sel"][b])
            assert np.array_equal(g["idx"][b, :n], a["idx"][b, :n]), (m, b)
            compare_sel(g, o, b)
            compare_out(g, o, b)
        say("micro-batches m=%d: max diff to the one-call step %.3g"
            % (m, float(np.abs(g["out"] - a["out"]).max())))


def _run_micro_batches(skv, c, sm, m, reps, flags):
    """The batch as m micro-batches of consecutive sequences, each a step call
    on views of the same buffers with its own workspace and stream, reps
    layer-steps in a row with nothing ordering the streams against each other
    (the schedule the benchmark times); every workspace must end with the
    given flags.  Returns the results as numpy arrays."""
    per = c.B // m
    cap = skv.select_capacity(token_desc_of(skv, c))
    qs = torch.zeros((c.B, c.n_kv * c.R), dtype=torch.int8, device="cuda")
    qsc = torch.zeros((c.B,), dtype=torch.float32, device="cuda")
    idx = torch.full((c.B, cap), -1, dtype=torch.int32, device="cuda")
    nsel = torch.zeros((c.B,), dtype=torch.int32, device="cuda")
    out = torch.zeros((c.B, c.n_q, c.D), dtype=torch.float32, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(m)]
    calls = []
    for g in range(m):
        sl = slice(g * per, (g + 1) * per)
        desc = skv.token_desc(per, c.T_max, c.n_kv, c.n_q, c.D, topk=c.k, n_sink=c.S,
                              n_tail=c.L, kv_dtype=skv.SKV_KV_I8_ROWSCALE)
        kv = skv.kv_view(c.k_cache[sl], c.v_cache[sl], c.k_scale[sl], c.v_scale[sl])
        calls.append((desc, c.ctx_len[sl], c.q[sl], c.basis, qs[sl], qsc[sl], None,
                      c.codes[sl], c.sk_scale[sl], kv, idx[sl], nsel[sl], sm, out[sl],
                      skv.workspace(desc)))
    ev = torch.cuda.Event()
    ev.record()
    for st in streams:
        st.wait_event(ev)
    for rep in range(reps):
        for st, args in zip(streams, calls):
            skv.step(*args, stream=st)
    for st in streams:
        torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    for args in calls:
        assert skv.check(args[-1]) == flags
    return dict(qs=qs.cpu().numpy(), qscale=qsc.cpu().numpy(), n_sel=nsel.cpu().numpy(),
                idx=idx.cpu().numpy(), out=out.cpu().numpy().astype(np.float64), flags=flags)


def test_device_flags():
    """Out-of-range ctx_len and attention indices are clamped/skipped and flagged."""
    skv = need_gpu()
    c = _cfg1(2, 1024, [1024, 500], n_needles=0)
    desc = token_desc_of(skv, c)
    cap = skv.select_capacity(desc)
    ws = skv.workspace(desc)
    ctx = torch.tensor([5000, 500], dtype=torch.int32, device="cuda")
    qs = torch.zeros((2, 128), dtype=torch.int8, device="cuda")
    keys = torch.zeros((2, 1024), dtype=torch.float64, device="cuda")
    skv.score(desc, ctx, qs, c.codes.cuda(), c.sk_scale.cuda(), keys, ws)
    with pytest.raises(skv.SkvError):
        skv.check(ws)
    idx = torch.full((2, cap), 7, dtype=torch.int32, device="cuda")
    idx[0, 3] = 99_999
    nsel = torch.tensor([10, 10], dtype=torch.int32, device="cuda")
    out = torch.zeros((2, 8, 128), dtype=torch.float32, device="cuda")
    kv = skv.kv_view(c.k_cache.cuda(), c.v_cache.cuda())
    skv.attend(desc, c.q.cuda(), kv, idx, nsel, 0.1, out, ws)
    with pytest.raises(skv.SkvError):
        skv.check(ws)
    assert skv.check(ws) == 0    # flags were cleared


# ---------------------------------------------------------------------------
# full workload sizes, generated on the device; every sequence checked
# ---------------------------------------------------------------------------

def test_full_config2_8x250k():
    skv = need_gpu()
    say("cfg2 full: generating 8 x 250,000")
    c = _cfg2(8, 250_000, device="cuda")
    sm = 256 ** -0.5
    g = run_token_gpu(skv, c, sm, fused=True)
    say("cfg2 full: oracle on all 8 sequences")
    o = oracle_token(c, sm)
    err = _check_token(c, g, o)
    assert g["n_sel"].tolist() == [3136] * 8
    assert g["flags"] == 0
    say("cfg2 full max err", err)
    _check_micro_batches(skv, c, sm, g, o, "cfg2")


def _check_micro_batches(skv, c, sm, g, o, name):
    """The launch configuration the benchmark times for a large batch: two
    micro-batches of B/2 sequences on two streams, several layer-steps in a
    row.  Every sequence gets the one-call step's sketch, picks and outputs,
    within tolerance of the oracle."""
    say("%s full: two micro-batches on two streams" % name)
    mb = _run_micro_batches(skv, c, sm, 2, reps=4, flags=g["flags"])
    assert np.array_equal(mb["qs"], g["qs"])
    assert np.array_equal(mb["n_sel"], g["n_sel"])
    assert np.array_equal(mb["idx"], g["idx"])
    for b in range(c.B):
        compare_out(mb, o, b)
    say("%s full, micro-batches: max diff to the one-call step %.3g"
        % (name, float(np.abs(mb["out"] - g["out"]).max())))


def test_full_config3_1m():
    skv = need_gpu()
    say("cfg3 full: generating 1 x 1,048,576")
    c = _cfg3(1, 1_048_576, device="cuda")
    sm = 256 ** -0.5
    g = run_block_gpu(skv, c, sm, fused=True)
    o = oracle_block(c, sm)
    compare_keys(g["keys"], o["keys"], 0, 0, 262_144)
    compare_sel(g, o, 0)
    err = compare_out(g, o, 0)
    assert g["n_sel"][0] == 2048
    say("cfg3 full max err", err)


def test_full_config4a_32x128k():
    skv = need_gpu()
    say("cfg4a full: generating 32 x 131,072")
    c = _cfg2(32, 131_072, seed=1004, device="cuda")
    sm = 256 ** -0.5
    g = run_token_gpu(skv, c, sm, fused=True)
    say("cfg4a full: oracle on all 32 sequences")
    o = oracle_token(c, sm)
    _check_token(c, g, o)
    assert g["flags"] == 0
    _check_micro_batches(skv, c, sm, g, o, "cfg4a")


def test_full_config4b_mixed():
    skv = need_gpu()
    lens = synth.gen.mixed_lengths(32, 2048, 250_000, seed=1014)
    lens[:3] = [3135, 3136, 3137]
    say("cfg4b mixed lengths, min", min(lens), "max", max(lens))
    c = _cfg2(32, 250_000, lens, seed=1014, device="cuda")
    sm = 256 ** -0.5
    g = run_token_gpu(skv, c, sm, fused=True)
    say("cfg4b full: oracle on all 32 sequences")
    o = oracle_token(c, sm)
    _check_token(c, g, o)
    for b in range(32):
        assert g["n_sel"][b] == min(lens[b], 3136)
    _check_micro_batches(skv, c, sm, g, o, "cfg4b")


def test_full_top4096_8x250k():
    """The largest budget at the headline shape: 8 x 250,000 with top-4096 +
    64 sinks + 1,024 tail (5,184 rows per sequence), every sequence against
    the oracle, then as the two micro-batches the benchmark times."""
    skv = need_gpu()
    say("top-4096 full: generating 8 x 250,000")
    c = synth.make_token_case(8, 250_000, None, n_kv=4, n_q=24, D=256, S=64, k=4096, L=1024,
                              kv_format="i8", seed=1002, device="cuda")
    sm = 256 ** -0.5
    g = run_token_gpu(skv, c, sm, fused=True)
    say("top-4096 full: oracle on all 8 sequences")
    o = oracle_token(c, sm)
    err = _check_token(c, g, o)
    assert g["n_sel"].tolist() == [64 + 4096 + 1024] * 8
    assert g["flags"] == 0, g["flags"]
    say("top-4096 full max err", err)
    _check_micro_batches(skv, c, sm, g, o, "top-4096")


@pytest.mark.parametrize("mode", ["token", "block"])
def test_score_topk_matches_separate_calls(mode):
    """The fused score+select entry point (no keys materialized) gives the
    index sets of sparsekv_score followed by sparsekv_topk, bit for bit."""
    skv = need_gpu()
    if mode == "token":
        c = _cfg2(4, 60_000, [60_000, 30_000, 3_500, 3_100], device="cuda")
        desc = token_desc_of(skv, c)
        qs = torch.zeros((c.B, 256), dtype=torch.int8, device="cuda")
        qsc = torch.zeros((c.B,), dtype=torch.float32, device="cuda")
        ws = skv.workspace(desc)
        skv.qsketch(desc, c.q, c.basis, qs, qsc, ws)
        iq, ik, isc, nkeys = qs, c.codes, c.sk_scale, c.T_max
    else:
        c = _cfg3(3, 80_000, [80_000, 40_001, 2_055], device="cuda")
        desc = block_desc_of(skv, c)
        ws = skv.workspace(desc)
        iq, ik, isc, nkeys = c.qi, c.kp, None, c.T_max // 4
    cap = skv.select_capacity(desc)
    res = []
    for fused in (False, True):
        idx = torch.full((c.B, cap), -1, dtype=torch.int32, device="cuda")
        nsel = torch.zeros((c.B,), dtype=torch.int32, device="cuda")
        if fused:
            skv.score_topk(desc, c.ctx_len, iq, ik, isc, idx, nsel, ws)
        else:
            keys = torch.full((c.B, nkeys), float("nan"), dtype=torch.float64, device="cuda")
            skv.score(desc, c.ctx_len, iq, ik, isc, keys, ws)
            skv.topk(desc, c.ctx_len, keys, idx, nsel, ws)
        assert skv.check(ws) & skv.SKV_FLAG_TOPK_SLOW == 0
        res.append((idx.cpu().numpy(), nsel.cpu().numpy()))
    (i0, n0), (i1, n1) = res
    assert np.array_equal(n0, n1)
    for b in range(c.B):
        assert np.array_equal(i0[b, :n0[b]], i1[b, :n1[b]])


def _fused_select_vs_oracle(skv, c, qs_np):
    """sparsekv_score_topk with the given int8 query sketch against the oracle
    select on the oracle's keys; returns the device flags."""
    desc = token_desc_of(skv, c)
    cap = skv.select_capacity(desc)
    ws = skv.workspace(desc)
    idx = torch.full((c.B, cap), -1, dtype=torch.int32, device="cuda")
    nsel = torch.zeros((c.B,), dtype=torch.int32, device="cuda")
    skv.score_topk(desc, c.ctx_len, torch.from_numpy(qs_np).cuda(), c.codes, c.sk_scale, idx, nsel, ws)
    flags = skv.check(ws)
    keys = oracle.sketch_keys(qs_np, c.codes.cpu().numpy(), c.sk_scale.cpu().numpy(), c.lens, c.S,
                              c.k, c.L)
    gi, gn = idx.cpu().numpy(), nsel.cpu().numpy()
    for b in range(c.B):
        sel = oracle.select_tokens(keys[b], c.lens[b], c.S, c.k, c.L)
        assert gn[b] == sel.size
        assert np.array_equal(gi[b, :gn[b]], sel), "seq %d" % b
    return flags


@pytest.mark.parametrize("B", [1, 2])
def test_fused_select_all_keys_equal(B):
    """A zero query sketch makes every key 0: every candidate ties, there are
    more candidates than the select holds in LDS, and the budget goes to the
    lowest positions (the select over the candidate records in memory).  One
    sequence takes the threshold over every sampled digit, two over the front
    workgroups' summary rows."""
    skv = need_gpu()
    c = _cfg2(B, 40_000, [40_000, 25_000][:B], device="cuda")
    qs = np.zeros((c.B, 256), dtype=np.int8)
    flags = _fused_select_vs_oracle(skv, c, qs)
    assert flags & skv.SKV_FLAG_TOPK_SLOW


@pytest.mark.parametrize("B", [1, 2])
def test_fused_select_sample_overshoot(B):
    """Large keys planted on three of the sixteen keys of every sampled line
    make the threshold too high: every sampled workgroup's largest digits are
    planted ones, yet the planted keys are fewer than the budget, so the
    select recomputes every key of the sequence (the exact fallback).  One
    sequence takes the threshold over every sampled digit, two over the front
    workgroups' summary rows."""
    skv = need_gpu()
    c = _cfg2(B, 120_000, [120_000] * B, n_needles=0, device="cuda")
    qs = np.zeros((B, 256), dtype=np.int8)
    qs[:, :] = 1
    n = c.lens[0] - c.S - c.L
    s = max(n // (4 * c.k), 1)                    # the sample takes every s-th line of 16
    lines = (n + 15) // 16
    nsl = (lines + s - 1) // s
    codes = c.codes.cpu().numpy()
    scale = c.sk_scale.cpu().numpy().view(np.uint16).copy()
    sampled = np.array([c.S + 16 * s * j + e for j in range(nsl) for e in range(3)])
    assert s == 14 and 1000 < sampled.size < c.k
    # all codes +7 (nibbles 0x7 in both halves): dot = 7 * 256 with qs = 1
    codes[:, sampled] = 0x77
    scale[:, sampled] = np.float16(8.0).view(np.uint16)
    c.codes.copy_(torch.from_numpy(codes))
    c.sk_scale.copy_(torch.from_numpy(scale.view(np.float16)))
    flags = _fused_select_vs_oracle(skv, c, qs)
    assert flags & skv.SKV_FLAG_TOPK_SLOW
