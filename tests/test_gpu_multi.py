"""GPU parity of the multi-query step (several query tokens per sequence, as in
the verification of drafted tokens): sparsekv_step_multi through the C ABI
against oracle.multiquery on the same seeded bytes.  Query sketches, their
scales and the index set of every query bit for bit; attention outputs within
2e-3 max abs error of the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import ATOL, need_gpu, say, to_dev, token_desc_of

pytestmark = pytest.mark.gpu


def _case(B, T, lens, *, n_kv=4, n_q=24, D=256, R=64, S=64, k=2048, L=1024, kv="i8", seed=1002,
          device="cpu"):
    return synth.make_token_case(B, T, lens, n_kv=n_kv, n_q=n_q, D=D, R=R, S=S, k=k, L=L,
                                 kv_format=kv, n_needles=0, seed=seed, device=device)


def _run_multi(skv, c, q, M, sm):
    dev = to_dev(c, ["ctx_len", "basis", "codes", "sk_scale", "k_cache", "v_cache", "k_scale",
                     "v_scale"])
    desc = token_desc_of(skv, c)
    cap = skv.select_capacity(desc)
    ws = skv.workspace_multi(desc, M)
    qs = torch.zeros((c.B, M, c.n_kv * c.R), dtype=torch.int8, device="cuda")
    qsc = torch.zeros((c.B, M), dtype=torch.float32, device="cuda")
    idx = torch.full((c.B, M, cap), -1, dtype=torch.int32, device="cuda")
    nsel = torch.full((c.B, M), -1, dtype=torch.int32, device="cuda")
    out = torch.full((c.B, M, c.n_q, c.D), float("nan"), dtype=torch.float32, device="cuda")
    kv = skv.kv_view(dev["k_cache"], dev["v_cache"], dev["k_scale"], dev["v_scale"])
    skv.step_multi(desc, M, dev["ctx_len"], q.cuda(), dev["basis"], qs, qsc, dev["codes"],
                   dev["sk_scale"], kv, idx, nsel, sm, out, ws)
    flags = skv.check(ws, raise_on_error=False)
    return dict(qs=qs.cpu().numpy(), qscale=qsc.cpu().numpy(), idx=idx.cpu().numpy(),
                n_sel=nsel.cpu().numpy(), out=out.cpu().numpy().astype(np.float64), flags=flags)


def _host(t, b):
    return None if t is None else t[b:b + 1].cpu().numpy()


def _oracle_multi(c, q, M, sm, seqs):
    """oracle.multiquery on the listed sequences, one at a time (host copies of
    just that sequence's caches)."""
    res = {}
    for b in seqs:
        qs, qsc, idx, out = oracle.multiquery.token_step_multi(
            q[b:b + 1].numpy(), c.basis.cpu().numpy(), _host(c.codes, b), _host(c.sk_scale, b),
            _host(c.k_cache, b), _host(c.v_cache, b), _host(c.k_scale, b), _host(c.v_scale, b),
            [c.lens[b]], M=M, S=c.S, k_top=c.k, L=c.L, group=c.group, sm_scale=sm,
            fmt=c.kv_format)
        res[b] = (qs[0], qsc[0], idx[0], out[0])
    return res


def _compare(g, o, M):
    worst = 0.0
    for b, (qs, qsc, idx, out) in o.items():
        assert np.array_equal(g["qs"][b], qs), "seq %d: query sketch codes differ" % b
        assert np.array_equal(g["qscale"][b].view(np.uint32), qsc.view(np.uint32)), \
            "seq %d: query scales differ" % b
        for j in range(M):
            n = int(g["n_sel"][b, j])
            assert n == idx[j].size, "seq %d query %d: n_sel %d vs oracle %d" % (b, j, n, idx[j].size)
            if not np.array_equal(g["idx"][b, j, :n], idx[j]):
                miss = np.setdiff1d(idx[j], g["idx"][b, j, :n])
                raise AssertionError("seq %d query %d: index sets differ (%d missing, e.g. %s)"
                                     % (b, j, miss.size, miss[:5]))
            err = float(np.max(np.abs(g["out"][b, j] - out[j])))
            assert err <= ATOL, "seq %d query %d: max abs error %.3g" % (b, j, err)
            worst = max(worst, err)
    return worst


def test_multi_query_ragged_and_threshold():
    """cfg-2 layer shape, 8 query tokens per sequence; one sequence crosses the
    budget threshold inside the step (S+k+L = 3136: contexts 3133..3140, the
    first four dense), lengths spanning several 256-token segments with ragged
    tails."""
    skv = need_gpu()
    M = 8
    lens = [21_000, 3_140, 9_001]
    c = _case(3, 21_504, lens, seed=2101)
    q = synth.multi_queries(3, M, 24, 256, 2101)
    sm = 256 ** -0.5
    say("multi ragged", lens, "M", M)
    g = _run_multi(skv, c, q, M, sm)
    o = _oracle_multi(c, q, M, sm, range(3))
    err = _compare(g, o, M)
    assert g["n_sel"][1].tolist() == [3133, 3134, 3135, 3136, 3136, 3136, 3136, 3136]
    assert g["flags"] & ~skv.SKV_FLAG_TOPK_SLOW == 0
    say("multi ragged max err", err)


@pytest.mark.parametrize("shape", ["cfg1", "wide"])
def test_multi_query_other_sketch_widths(shape):
    """64 sketch bytes per token (2 KV heads x rank 64, fp16 K/V, head_dim 128)
    and 256 (8 KV heads x rank 64), 5 query tokens."""
    skv = need_gpu()
    M = 5
    if shape == "cfg1":
        c = _case(2, 4096, [4096, 2999], n_kv=2, n_q=8, D=128, S=16, k=256, L=128, kv="f16",
                  seed=2102)
    else:
        c = _case(2, 6000, [6000, 5003], n_kv=8, n_q=16, D=128, S=16, k=512, L=64, kv="f16",
                  seed=2103)
    q = synth.multi_queries(2, M, c.n_q, c.D, 2104)
    sm = c.D ** -0.5
    say("multi", shape, "M", M)
    g = _run_multi(skv, c, q, M, sm)
    err = _compare(g, _oracle_multi(c, q, M, sm, range(2)), M)
    say("multi", shape, "max err", err)


def test_multi_query_one_query_is_the_step():
    """n_query = 1 is sparsekv_step: the same sketch, index set and output bits."""
    skv = need_gpu()
    lens = [12_000, 3_000]
    c = _case(2, 12_288, lens, seed=2105)
    sm = 256 ** -0.5
    q1 = c.q.unsqueeze(1).contiguous()           # [B][1][H_q][D]
    g = _run_multi(skv, c, q1, 1, sm)
    dev = to_dev(c, ["ctx_len", "q", "basis", "codes", "sk_scale", "k_cache", "v_cache", "k_scale",
                     "v_scale"])
    desc = token_desc_of(skv, c)
    cap = skv.select_capacity(desc)
    ws = skv.workspace(desc)
    qs = torch.zeros((c.B, c.n_kv * c.R), dtype=torch.int8, device="cuda")
    qsc = torch.zeros((c.B,), dtype=torch.float32, device="cuda")
    idx = torch.full((c.B, cap), -1, dtype=torch.int32, device="cuda")
    nsel = torch.zeros((c.B,), dtype=torch.int32, device="cuda")
    out = torch.zeros((c.B, c.n_q, c.D), dtype=torch.float32, device="cuda")
    kv = skv.kv_view(dev["k_cache"], dev["v_cache"], dev["k_scale"], dev["v_scale"])
    skv.step(desc, dev["ctx_len"], dev["q"], dev["basis"], qs, qsc, None, dev["codes"],
             dev["sk_scale"], kv, idx, nsel, sm, out, ws)
    skv.check(ws, raise_on_error=False)
    assert np.array_equal(g["qs"][:, 0], qs.cpu().numpy())
    assert np.array_equal(g["qscale"][:, 0], qsc.cpu().numpy())
    assert np.array_equal(g["n_sel"][:, 0], nsel.cpu().numpy())
    for b in range(c.B):
        n = int(nsel[b])
        assert np.array_equal(g["idx"][b, 0, :n], idx[b, :n].cpu().numpy())
    assert np.array_equal(g["out"][:, 0], out.cpu().numpy().astype(np.float64))


def test_multi_query_short_contexts():
    """Contexts shorter than the step: queries with T_j <= 0 select nothing and
    output zeros; the rest are dense."""
    skv = need_gpu()
    M = 6
    lens = [3, 0, 6, 1]
    c = _case(4, 64, lens, seed=2106)
    q = synth.multi_queries(4, M, 24, 256, 2106)
    sm = 256 ** -0.5
    g = _run_multi(skv, c, q, M, sm)
    err = _compare(g, _oracle_multi(c, q, M, sm, range(4)), M)
    assert g["n_sel"].tolist() == [[0, 0, 0, 1, 2, 3], [0] * 6, [1, 2, 3, 4, 5, 6],
                                   [0, 0, 0, 0, 0, 1]]
    assert not g["out"][1].any() and not g["out"][0, :3].any()
    say("multi short max err", err)


def test_multi_query_full_8x250k():
    """8 x 250,000 tokens with 8 query tokens each (the workload bench.py's
    multi-query line times); two sequences checked against the oracle."""
    skv = need_gpu()
    M = 8
    say("multi full: generating 8 x 250,000")
    c = _case(8, 250_000, None, seed=1002, device="cuda")
    q = synth.multi_queries(8, M, 24, 256, 1006)
    sm = 256 ** -0.5
    g = _run_multi(skv, c, q, M, sm)
    assert g["n_sel"].tolist() == [[3136] * M] * 8
    assert g["flags"] == 0
    say("multi full: oracle on sequences 2, 7")
    err = _compare(g, _oracle_multi(c, q, M, sm, [2, 7]), M)
    say("multi full max err", err)


def test_multi_query_determinism_and_graph_replay():
    """Two eager runs are bitwise identical; a captured HIP graph of the
    multi-query step, replayed several times with eager work in between,
    gives the eager result every time."""
    skv = need_gpu()
    M = 6
    lens = [15_000, 3_200, 7_777]
    c = _case(3, 15_360, lens, seed=2107, device="cuda")
    q = synth.multi_queries(3, M, 24, 256, 2107, device="cuda")
    sm = 256 ** -0.5
    a = _run_multi(skv, c, q, M, sm)
    b = _run_multi(skv, c, q, M, sm)
    for key in ("qs", "qscale", "idx", "n_sel", "out"):
        assert np.array_equal(a[key], b[key]), key
    desc = token_desc_of(skv, c)
    cap = skv.select_capacity(desc)
    ws = skv.workspace_multi(desc, M)
    qs = torch.zeros((c.B, M, 256), dtype=torch.int8, device="cuda")
    qsc = torch.zeros((c.B, M), dtype=torch.float32, device="cuda")
    idx = torch.zeros((c.B, M, cap), dtype=torch.int32, device="cuda")
    nsel = torch.zeros((c.B, M), dtype=torch.int32, device="cuda")
    out = torch.zeros((c.B, M, c.n_q, c.D), dtype=torch.float32, device="cuda")
    kv = skv.kv_view(c.k_cache, c.v_cache, c.k_scale, c.v_scale)

    def call():
        skv.step_multi(desc, M, c.ctx_len, q, c.basis, qs, qsc, c.codes, c.sk_scale, kv, idx, nsel,
                       sm, out, ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on the capture stream
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(4):
        out.zero_()
        idx.zero_()
        graph.replay()
        torch.cuda.synchronize()
        _ = (out * 2).sum().item()   # unrelated eager work between replays
        assert np.array_equal(out.cpu().numpy().astype(np.float64), a["out"]), "replay %d" % rep
        gi = idx.cpu().numpy()
        for bb in range(c.B):
            for j in range(M):
                n = int(a["n_sel"][bb, j])
                assert np.array_equal(gi[bb, j, :n], a["idx"][bb, j, :n])
    assert skv.check(ws) == 0
