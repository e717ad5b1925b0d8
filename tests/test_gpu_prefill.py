"""GPU parity of the prefill attention over host-resident K/V
(sparsekv_prefill_attend through the C ABI) against oracle.prefill on the same
seeded bytes: outputs within 2e-3 max abs error of the fp64 oracle, for
several working-buffer sizes (the result must not depend on how the history
is chunked), with ragged last chunks, empty picks, both element types and
head groupings, and device flags for bad lists."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import ATOL, need_gpu, say

pytestmark = pytest.mark.gpu


def _case(T, P, n_kv, n_q, D, k_blocks, fmt, seed):
    g = torch.Generator().manual_seed(seed)
    dt = torch.bfloat16 if fmt == "bf16" else torch.float16
    k = torch.empty((T, n_kv, D), dtype=dt, pin_memory=True)
    v = torch.empty((T, n_kv, D), dtype=dt, pin_memory=True)
    k.copy_(torch.randn((T, n_kv, D), generator=g).to(dt))
    v.copy_(torch.randn((T, n_kv, D), generator=g).to(dt))
    q = torch.randn((P, n_q, D), generator=g).to(dt)
    idx, n_sel = synth.prefill_picks(P, T, k_blocks, seed)
    return k, v, q, idx, n_sel


def _desc(skv, n_kv, n_q, D, fmt, max_ctx):
    if fmt == "bf16":
        return skv.block_desc(1, max_ctx, n_kv, n_q, D, topk_blocks=64)
    return skv.token_desc(1, max_ctx, n_kv, n_q, D, topk=64, n_sink=4, n_tail=8,
                          kv_dtype=skv.SKV_KV_F16)


def _run(skv, desc, k, v, q, idx, n_sel, chunk_tokens, sm, raise_on_error=True):
    P, n_q, D = q.shape
    row = 2 * k.shape[1] * D * 2          # K and V rows of one token
    buf = torch.empty((2 * chunk_tokens * row,), dtype=torch.uint8, device="cuda")   # two halves
    ws = torch.zeros((skv.prefill_workspace_size(desc, P),), dtype=torch.uint8, device="cuda")
    out = torch.full((P, n_q, D), float("nan"), dtype=torch.float32, device="cuda")
    skv.prefill_attend(desc, q.cuda(), torch.from_numpy(idx).cuda(), torch.from_numpy(n_sel).cuda(),
                       k, v, buf, sm, out, ws)
    flags = skv.check(ws, raise_on_error=raise_on_error)
    return out.cpu().numpy().astype(np.float64), flags


def _oracle(k, v, q, idx, n_sel, sm, group, fmt, queries):
    if fmt == "bf16":
        kk, vv, qq = (x.view(torch.int16).numpy().view(np.uint16) for x in (k, v, q))
    else:
        kk, vv, qq = k.numpy(), v.numpy(), q.numpy()
    lists = [idx[p, :n_sel[p]].astype(np.int64) for p in queries]
    return oracle.prefill.prefill_attention(qq[queries], kk, vv, lists, sm, group, fmt)


@pytest.mark.parametrize("fmt,n_kv,n_q,D", [("bf16", 2, 16, 256), ("f16", 4, 24, 128),
                                            ("bf16", 1, 16, 128)])
def test_prefill_matches_oracle_any_chunking(fmt, n_kv, n_q, D):
    skv = need_gpu()
    T, P, kb = 5003, 40, 48
    k, v, q, idx, n_sel = _case(T, P, n_kv, n_q, D, kb, fmt, 3101)
    n_sel[5] = 0                                   # a query with nothing picked
    idx[6, :n_sel[6]] = np.arange(1200, 1200 + n_sel[6])   # all picks inside one chunk
    desc = _desc(skv, n_kv, n_q, D, fmt, T)
    sm = D ** -0.5
    ref = _oracle(k, v, q, idx, n_sel, sm, n_q // n_kv, fmt, list(range(P)))
    outs = []
    for ct in (700, 1024, 5003, 9000, 37, 1):
        say("prefill", fmt, n_kv, n_q, D, "chunk tokens", ct)
        got, flags = _run(skv, desc, k, v, q, idx, n_sel, ct, sm)
        assert flags == 0
        err = float(np.max(np.abs(got - ref)))
        assert err <= ATOL, (ct, err)
        assert not got[5].any()
        outs.append(got)
    for o in outs[1:]:
        assert float(np.max(np.abs(o - outs[0]))) <= 1e-5


def test_prefill_flags_bad_lists():
    """Positions past the history, below zero, or n_sel past cap are skipped /
    clamped and raise SKV_FLAG_INDEX_RANGE; the remaining rows still attend."""
    skv = need_gpu()
    T, P = 3000, 6
    k, v, q, idx, n_sel = _case(T, P, 2, 16, 256, 32, "bf16", 3102)
    desc = _desc(skv, 2, 16, 256, "bf16", T)
    idx2, n2 = idx.copy(), n_sel.copy()
    idx2[1, n2[1] - 1] = T + 5          # past the end (still ascending)
    idx2[2, 0] = -3                     # below zero
    n2[3] = idx.shape[1] + 7            # past cap
    got, flags = _run(skv, desc, k, v, q, idx2, n2, 512, 0.0625, raise_on_error=False)
    assert flags & skv.SKV_FLAG_INDEX_RANGE
    ok = [0, 4, 5]
    ref = _oracle(k, v, q, idx2, n2, 0.0625, 8, "bf16", ok)
    assert float(np.max(np.abs(got[ok] - ref))) <= ATOL
    lists = [idx2[1, :n2[1] - 1], idx2[2, 1:n2[2]]]
    ref12 = oracle.prefill.prefill_attention(
        q.view(torch.int16).numpy().view(np.uint16)[[1, 2]], k.view(torch.int16).numpy().view(np.uint16),
        v.view(torch.int16).numpy().view(np.uint16), lists, 0.0625, 8, "bf16")
    assert float(np.max(np.abs(got[[1, 2]] - ref12))) <= ATOL


def test_prefill_large_history_sampled():
    """262,144-token history, 512 prefill queries with 512 picked blocks each,
    a 32 MiB working buffer; 12 queries checked against the oracle."""
    skv = need_gpu()
    T, P = 262_144, 512
    say("prefill large: generating")
    k, v, q, idx, n_sel = _case(T, P, 2, 16, 256, 512, "bf16", 3103)
    desc = _desc(skv, 2, 16, 256, "bf16", T)
    ct = (32 << 20) // (2 * 2 * 2 * 256 * 2)   # 32 MiB in two halves
    got, flags = _run(skv, desc, k, v, q, idx, n_sel, ct, 0.0625)
    assert flags == 0
    queries = [0, 1, 100, 255, 256, 300, 400, 500, 509, 510, 511, 77]
    ref = _oracle(k, v, q, idx, n_sel, 0.0625, 8, "bf16", queries)
    err = float(np.max(np.abs(got[queries] - ref)))
    assert err <= ATOL
    say("prefill large max err", err)
