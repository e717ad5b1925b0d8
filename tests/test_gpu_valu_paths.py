"""GPU parity of the vector-ALU kernels, the measurement aid that
sparsekv_set_contraction_path selects in place of the matrix-core kernels.

Single-query int8 attention: on the config-2 layer shape with ragged and tiny
lengths the outputs must be within 2e-3 of the fp64 oracle, like the
matrix-core kernel's, and the two kernels must agree to fp32 rounding (same
rows, same per-chunk partials, same merge).  Shapes it does not serve take the
matrix-core kernel; out-of-range indices are flagged as there.

Multi-query sketch score: integer dots, so every query's index set, its keys'
order and the outputs are bit-identical to the matrix-core path's, and equal
to the oracle's."""

import numpy as np
import pytest
import torch

import synth
from gpu_util import compare_out, need_gpu, oracle_token, run_token_gpu, say, token_desc_of
from test_gpu_multi import _case, _compare, _oracle_multi, _run_multi

pytestmark = pytest.mark.gpu


def _cfg2(B, T, lens, seed, **kw):
    return synth.make_token_case(B, T, lens, n_kv=4, n_q=24, D=256, S=64, k=2048, L=1024,
                                 kv_format="i8", seed=seed, **kw)


def _both_paths(skv, c, sm, fused):
    try:
        skv.set_contraction_path(skv.SKV_PATH_MFMA)
        a = run_token_gpu(skv, c, sm, fused=fused)
        skv.set_contraction_path(skv.SKV_PATH_VALU)
        v = run_token_gpu(skv, c, sm, fused=fused)
    finally:
        skv.set_contraction_path(skv.SKV_PATH_MFMA)
    return a, v


@pytest.mark.parametrize("fused", [True, False])
def test_valu_attention_config2_ragged(fused):
    skv = need_gpu()
    lens = [40_000, 3_137, 17_001, 3_136, 3_135]
    c = _cfg2(5, 40_960, lens, seed=1002)
    sm = 256 ** -0.5
    say("valu attention cfg2 ragged", lens, "fused", fused)
    a, v = _both_paths(skv, c, sm, fused)
    o = oracle_token(c, sm)
    assert a["flags"] == 0 and v["flags"] == 0
    for key in ("qs", "idx", "n_sel"):
        assert np.array_equal(a[key], v[key]), key
    errs = [compare_out(v, o, b) for b in range(c.B)]
    diff = float(np.max(np.abs(a["out"] - v["out"])))
    say("valu max err vs oracle", max(errs), "valu vs mfma", diff)
    assert diff <= 1e-4


def test_valu_attention_tiny_and_empty():
    skv = need_gpu()
    lens = [0, 1, 700, 3_137]
    c = _cfg2(4, 4_096, lens, seed=1012, n_needles=0)
    sm = 256 ** -0.5
    say("valu attention tiny", lens)
    a, v = _both_paths(skv, c, sm, fused=False)
    o = oracle_token(c, sm)
    for b in range(c.B):
        compare_out(v, o, b)
    assert not v["out"][0].any()
    assert float(np.max(np.abs(a["out"] - v["out"]))) <= 1e-4


def test_valu_attention_other_shapes_take_mfma():
    """16 query heads per KV head need more LDS than the vector-ALU kernel
    takes: the matrix-core kernel runs, and the results are bit-identical."""
    skv = need_gpu()
    c = synth.make_token_case(2, 30_000, [30_000, 21_111], n_kv=2, n_q=32, D=256, S=16, k=512,
                              L=256, kv_format="i8", seed=71)
    sm = 0.0625
    a, v = _both_paths(skv, c, sm, fused=True)
    assert np.array_equal(a["out"], v["out"])
    o = oracle_token(c, sm)
    for b in range(c.B):
        compare_out(v, o, b)


def test_valu_attention_flags_bad_indices():
    skv = need_gpu()
    c = _cfg2(2, 4_096, [4_096, 500], seed=1013, n_needles=0)
    desc = token_desc_of(skv, c)
    cap = skv.select_capacity(desc)
    ws = skv.workspace(desc)
    idx = torch.full((2, cap), 7, dtype=torch.int32, device="cuda")
    idx[0, 3] = 99_999
    nsel = torch.tensor([300, 10], dtype=torch.int32, device="cuda")
    out = torch.zeros((2, 24, 256), dtype=torch.float32, device="cuda")
    kv = skv.kv_view(c.k_cache.cuda(), c.v_cache.cuda(), c.k_scale.cuda(), c.v_scale.cuda())
    try:
        skv.set_contraction_path(skv.SKV_PATH_VALU)
        skv.attend(desc, c.q.cuda(), kv, idx, nsel, 0.1, out, ws)
        with pytest.raises(skv.SkvError):
            skv.check(ws)
        assert skv.check(ws) == 0
    finally:
        skv.set_contraction_path(skv.SKV_PATH_MFMA)


@pytest.mark.parametrize("shape", ["cfg2", "cfg1", "wide"])
def test_valu_multi_query_score(shape):
    """Sketch rows of 128 bytes (config-2 shape, 8 queries, one sequence
    crossing the budget threshold inside the step) and 64 bytes take the
    vector-ALU score; 256-byte rows take the matrix-core one."""
    skv = need_gpu()
    if shape == "cfg2":
        M, lens = 8, [21_000, 3_140, 9_001]
        c = _case(3, 21_504, lens, seed=2101)
    elif shape == "cfg1":
        M = 5
        c = _case(2, 4096, [4096, 2999], n_kv=2, n_q=8, D=128, S=16, k=256, L=128, kv="f16", seed=2102)
    else:
        M = 5
        c = _case(2, 6000, [6000, 5003], n_kv=8, n_q=16, D=128, S=16, k=512, L=64, kv="f16", seed=2103)
    q = synth.multi_queries(c.B, M, c.n_q, c.D, 2101 if shape == "cfg2" else 2104)
    sm = c.D ** -0.5
    say("valu multi-query score", shape, "M", M)
    try:
        skv.set_contraction_path(skv.SKV_PATH_MFMA)
        a = _run_multi(skv, c, q, M, sm)
        skv.set_contraction_path(skv.SKV_PATH_VALU)
        v = _run_multi(skv, c, q, M, sm)
    finally:
        skv.set_contraction_path(skv.SKV_PATH_MFMA)
    for key in ("qs", "qscale", "n_sel", "idx", "out"):
        assert np.array_equal(a[key], v[key]), key
    assert v["flags"] & ~skv.SKV_FLAG_TOPK_SLOW == 0
    err = _compare(v, _oracle_multi(c, q, M, sm, range(c.B)), M)
    say("valu multi-query", shape, "max err", err)
