"""GPU parity of the decode-step append (sparsekv_append): the new token's
int8 K/V rows and scales (or fp16 rows), its int4 key sketch and scale, and the
ctx_len advance must equal the oracle's bit for bit; a full sequence is left
unchanged and flagged.  Then a step over the appended caches must match the
oracle like any other step."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import need_gpu, oracle_token, run_token_gpu, say, token_desc_of
from test_gpu_parity import _check_token

pytestmark = pytest.mark.gpu


def _new_rows(B, n_kv, D, seed):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((B, n_kv, D), generator=g) * 1.5
    v = torch.randn((B, n_kv, D), generator=g)
    k[0, 0] = 0.0                      # a zero row: scale 0, codes 0
    v[1, -1] *= 300.0                  # a large row
    return k.to(torch.float16), v.to(torch.float16)


def _append_gpu(skv, c, k_new, v_new):
    desc = token_desc_of(skv, c)
    ws = skv.workspace(desc)
    dev = {n: getattr(c, n).cuda().clone() for n in ("codes", "sk_scale", "k_cache", "v_cache")}
    for n in ("k_scale", "v_scale"):
        dev[n] = getattr(c, n).cuda().clone() if getattr(c, n) is not None else None
    ctx = c.ctx_len.cuda().clone()
    kv = skv.kv_view(dev["k_cache"], dev["v_cache"], dev["k_scale"], dev["v_scale"])
    skv.append(desc, ctx, k_new.cuda(), v_new.cuda(), c.basis.cuda(), kv, dev["codes"], dev["sk_scale"], ws)
    flags = skv.check(ws, raise_on_error=False)
    return {n: (t.cpu() if t is not None else None) for n, t in dev.items()}, ctx.cpu(), flags


def _append_oracle(c, k_new, v_new):
    caches = dict(codes=c.codes.numpy().copy(), sk_scale=c.sk_scale.numpy().copy(),
                  k=c.k_cache.numpy().copy(), v=c.v_cache.numpy().copy())
    if c.kv_format == "i8":
        caches["k_scale"] = c.k_scale.numpy().copy()
        caches["v_scale"] = c.v_scale.numpy().copy()
    ctx = oracle.append.append_tokens(c.ctx_len.numpy(), k_new.numpy(), v_new.numpy(),
                                      c.basis.numpy(), caches, c.T_max, c.kv_format)
    return caches, ctx


def _compare(g, gctx, o, octx, fmt):
    assert gctx.tolist() == octx.tolist()
    assert np.array_equal(g["codes"].numpy(), o["codes"]), "sketch codes"
    assert np.array_equal(g["sk_scale"].numpy().view(np.uint16), o["sk_scale"].view(np.uint16)), "sketch scales"
    if fmt == "i8":
        assert np.array_equal(g["k_cache"].numpy(), o["k"]) and np.array_equal(g["v_cache"].numpy(), o["v"])
        assert np.array_equal(g["k_scale"].numpy().view(np.uint16), o["k_scale"].view(np.uint16))
        assert np.array_equal(g["v_scale"].numpy().view(np.uint16), o["v_scale"].view(np.uint16))
    else:
        assert np.array_equal(g["k_cache"].numpy().view(np.uint16), o["k"].view(np.uint16))
        assert np.array_equal(g["v_cache"].numpy().view(np.uint16), o["v"].view(np.uint16))


def test_append_int8_rows_and_sketch():
    skv = need_gpu()
    T = 8192
    c = synth.make_token_case(4, T, [100, 8191, 5000, 8192], n_kv=4, n_q=24, D=256, S=64, k=2048,
                              L=1024, kv_format="i8", seed=81)
    k_new, v_new = _new_rows(4, 4, 256, 82)
    say("append int8: lens", c.lens)
    g, gctx, flags = _append_gpu(skv, c, k_new, v_new)
    o, octx = _append_oracle(c, k_new, v_new)
    _compare(g, gctx, o, octx, "i8")
    assert gctx.tolist() == [101, 8192, 5001, 8192]
    assert flags == skv.SKV_FLAG_CTX_RANGE          # the full sequence


def test_append_fp16_rows():
    skv = need_gpu()
    c = synth.make_token_case(3, 4096, [0, 4095, 17], n_kv=2, n_q=8, D=128, S=16, k=256, L=128,
                              kv_format="f16", seed=83)
    k_new, v_new = _new_rows(3, 2, 128, 84)
    g, gctx, flags = _append_gpu(skv, c, k_new, v_new)
    o, octx = _append_oracle(c, k_new, v_new)
    _compare(g, gctx, o, octx, "f16")
    assert flags == 0


def test_step_after_append():
    """Three appends, then the fused step: the new tokens sit in the tail and
    the step must match the oracle on the appended caches."""
    skv = need_gpu()
    c = synth.make_token_case(2, 20_000, [12_000, 19_000], n_kv=4, n_q=24, D=256, S=64, k=2048,
                              L=1024, kv_format="i8", seed=85)
    for r in range(3):
        k_new, v_new = _new_rows(2, 4, 256, 86 + r)
        g, gctx, _ = _append_gpu(skv, c, k_new, v_new)
        o, octx = _append_oracle(c, k_new, v_new)
        _compare(g, gctx, o, octx, "i8")
        c.codes, c.sk_scale = g["codes"], g["sk_scale"]
        c.k_cache, c.v_cache, c.k_scale, c.v_scale = g["k_cache"], g["v_cache"], g["k_scale"], g["v_scale"]
        c.ctx_len = gctx.to(torch.int32)
        c.lens = gctx.tolist()
    assert c.lens == [12_003, 19_003]
    sm = 256 ** -0.5
    gs = run_token_gpu(skv, c, sm, fused=True)
    _check_token(c, gs, oracle_token(c, sm))


def _u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_append_block_mode():
    """Block mode: seven appends to a sequence that starts inside a block
    (two blocks complete), one full sequence; every byte against the oracle,
    then a step over the appended caches."""
    from gpu_util import block_desc_of, oracle_block, run_block_gpu
    from test_gpu_parity import _cfg3
    skv = need_gpu()
    c = _cfg3(2, 4096, [2049, 4096])
    desc = block_desc_of(skv, c)
    ws = skv.workspace(desc)
    kc, vc, kp = c.k_cache.cuda().clone(), c.v_cache.cuda().clone(), c.kp.cuda().clone()
    stage = torch.zeros((2, 4, c.index_dim), dtype=torch.bfloat16, device="cuda")
    ctx = c.ctx_len.cuda().clone()
    kv = skv.kv_view(kc, vc)
    o = dict(k=_u16(c.k_cache).copy(), v=_u16(c.v_cache).copy(), kp=_u16(c.kp).copy())
    ostage = np.zeros((2, 4, c.index_dim), np.uint16)
    octx = c.ctx_len.numpy()
    g = torch.Generator().manual_seed(92)
    flags = 0
    for step in range(7):
        kn = torch.randn((2, c.n_kv, c.D), generator=g).to(torch.bfloat16)
        vn = torch.randn((2, c.n_kv, c.D), generator=g).to(torch.bfloat16)
        raw = (torch.randn((2, c.index_dim), generator=g) * 3).to(torch.bfloat16)
        skv.append_block(desc, ctx, kn.cuda(), vn.cuda(), raw.cuda(), stage, kv, kp, ws)
        flags |= skv.check(ws, raise_on_error=False)
        octx = oracle.append.append_block_tokens(octx, _u16(kn), _u16(vn), _u16(raw), ostage, o, c.T_max)
        assert ctx.cpu().tolist() == octx.tolist()
        assert np.array_equal(_u16(kc.cpu()), o["k"]) and np.array_equal(_u16(vc.cpu()), o["v"])
        assert np.array_equal(_u16(kp.cpu()), o["kp"]), "pooled keys, step %d" % step
        assert np.array_equal(_u16(stage.cpu()), ostage)
    assert octx.tolist() == [2056, 4096] and flags == skv.SKV_FLAG_CTX_RANGE
    assert o["kp"][0, 512].any() and o["kp"][0, 513].any()
    c.k_cache, c.v_cache, c.kp = kc.cpu(), vc.cpu(), kp.cpu()
    c.ctx_len = torch.from_numpy(octx.astype(np.int32))
    c.lens = octx.tolist()
    sm = 256 ** -0.5
    gs = run_block_gpu(skv, c, sm, fused=True)
    os_ = oracle_block(c, sm)
    from gpu_util import compare_keys, compare_out, compare_sel
    for b in range(2):
        compare_keys(gs["keys"], os_["keys"], b, 0, c.lens[b] // 4)
        compare_sel(gs, os_, b)
        compare_out(gs, os_, b)


def test_multi_query_step_after_appends():
    """A verification step as served: the current token and 4 drafted ones are
    appended (5 appends), then the multi-query step verifies all 5 at their
    causal contexts; must match the oracle on the appended caches."""
    from test_gpu_multi import _compare as _compare_multi, _oracle_multi, _run_multi
    skv = need_gpu()
    M = 5
    c = synth.make_token_case(2, 20_000, [12_000, 3_134], n_kv=4, n_q=24, D=256, S=64, k=2048,
                              L=1024, kv_format="i8", n_needles=0, seed=87)
    for r in range(M):
        k_new, v_new = _new_rows(2, 4, 256, 88 + r)
        g, gctx, _ = _append_gpu(skv, c, k_new, v_new)
        o, octx = _append_oracle(c, k_new, v_new)
        _compare(g, gctx, o, octx, "i8")
        c.codes, c.sk_scale = g["codes"], g["sk_scale"]
        c.k_cache, c.v_cache, c.k_scale, c.v_scale = g["k_cache"], g["v_cache"], g["k_scale"], g["v_scale"]
        c.ctx_len = gctx.to(torch.int32)
        c.lens = gctx.tolist()
    assert c.lens == [12_005, 3_139]     # the second sequence crosses S+k+L = 3136 within the step
    q = synth.multi_queries(2, M, 24, 256, 89)
    sm = 256 ** -0.5
    gm = _run_multi(skv, c, q, M, sm)
    _compare_multi(gm, _oracle_multi(c, q, M, sm, range(2)), M)
    assert gm["n_sel"][1].tolist() == [3135, 3136, 3136, 3136, 3136]
