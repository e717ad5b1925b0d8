"""GPU parity of several query tokens per sequence through the host tier
(sparsekv_tier_resolve_multi + sparsekv_attend_multi through the C ABI)
against oracle.multiquery.tier_resolve_lists and oracle.tier_attention: slot
tables, hit / miss counts and the resident row of every pick equal the
oracle's every step; every query's attention over the resolved rows is within
2e-3 of the fp64 oracle; a step whose rows exceed the hot buffer is flagged."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import ATOL, need_gpu, say

pytestmark = pytest.mark.gpu

H, NQ, D, R = 4, 24, 256, 64


def _lists(rng, T, M, S, L, k, shared):
    """Pick lists of M query tokens at contexts T - M + 1 + j: each query's
    middle picks share `shared` positions with the others (drafted tokens
    attend much the same rows), plus its own sinks and tail."""
    lo, hi = S, T - M + 1 - L              # the middle range of the first query
    base = rng.choice(np.arange(lo, hi), shared, replace=False)
    out = []
    for j in range(M):
        Tj = T - M + 1 + j
        own = rng.choice(np.setdiff1d(np.arange(lo, hi), base), k - shared, replace=False)
        mid = np.sort(np.concatenate([base, own]))
        out.append(np.concatenate([np.arange(S), mid, np.arange(Tj - L, Tj)]).astype(np.int32))
    return out


def _run(B, T, S, L, k, M, n_slots, n_steps, shared, seed, lru=False, device="cpu", check_seqs=None,
         appends=0):
    skv = need_gpu()
    say("tier multi B=%d T=%d M=%d k=%d slots=%d lru=%s appends=%d" % (B, T, M, k, n_slots, lru, appends))
    c = synth.make_tier_case(B, T, n_kv=H, n_q=NQ, D=D, S=S, k=k, L=L, seed=seed, device=device)
    cap_ctx = T + appends
    desc = skv.token_desc(B, cap_ctx, H, NQ, D, topk=k, n_sink=S, n_tail=L)
    tier = skv.Tier(desc, T, n_slots, 1, policy=skv.SKV_TIER_LRU if lru else skv.SKV_TIER_CLOCK)
    check_seqs = list(range(B)) if check_seqs is None else check_seqs
    try:
        rec = np.zeros((B, cap_ctx, H, c.records.shape[-1]), dtype=np.uint8)
        rec[:, :T] = c.records.cpu().numpy()
        tier.host_records()[:, :T] = rec[:, :T]
        tier.load_resident(c.res_k.cuda(), c.res_v.cuda(), c.res_ks.cuda(), c.res_vs.cuda())
        rk, rv = c.res_k.cpu().numpy().copy(), c.res_v.cpu().numpy().copy()
        rks, rvs = c.res_ks.cpu().numpy().copy(), c.res_vs.cpu().numpy().copy()
        Tc = T
        if appends:
            # the drafted tokens are appended first (the tier's context moves on)
            basis = synth.orthonormal_basis(H, D, R, seed).cuda()
            codes = torch.zeros((B, cap_ctx, H * R // 2), dtype=torch.uint8, device="cuda")
            sksc = torch.zeros((B, cap_ctx), dtype=torch.float16, device="cuda")
            ctx = torch.full((B,), T, dtype=torch.int32, device="cuda")
            g = torch.Generator().manual_seed(seed + 5)
            for _ in range(appends):
                kn = torch.randn((B, H, D), generator=g).to(torch.float16)
                vn = torch.randn((B, H, D), generator=g).to(torch.float16)
                tier.append(ctx, kn.cuda(), vn.cuda(), basis, codes, sksc)
                for b in range(B):
                    oracle.append.tier_append_token(Tc, rec[b], rk[b], rv[b], rks[b], rvs[b], S, L,
                                                    kn[b].numpy(), vn[b].numpy())
                Tc += 1
        cap = skv.select_capacity(desc)
        q = synth.multi_queries(B, M, NQ, D, seed)
        ws = skv.workspace_multi(desc, M)
        rows = torch.zeros((B, M, cap), dtype=torch.int32, device="cuda")
        nsel = torch.full((B, M), cap, dtype=torch.int32, device="cuda")
        out = torch.zeros((B, M, NQ, D), dtype=torch.float32, device="cuda")
        ref = [oracle.residency.LruTier(n_slots, cap_ctx) if lru else oracle.ClockTier(n_slots, cap_ctx, window=1)
               for _ in range(B)]
        rng = np.random.default_rng(seed)
        prev = tier.stats()
        sm = D ** -0.5
        for s in range(n_steps):
            lists = [_lists(rng, Tc, M, S, L, k, shared) for _ in range(B)]
            idx_np = np.stack([np.stack(lb) for lb in lists])
            tier.resolve_multi(M, torch.from_numpy(idx_np).cuda(), nsel, s, rows)
            skv.attend_multi(desc, M, q.cuda(), tier.resident(), rows, nsel, sm, out, ws)
            st = tier.stats()
            slots = tier.slots()
            h_s = m_s = 0
            gr = rows.cpu().numpy()
            for b in range(B):
                sl, h, m = oracle.multiquery.tier_resolve_lists(ref[b], lists[b], Tc, S, L, s)
                h_s += h
                m_s += m
                assert np.array_equal(slots[b], ref[b].pos.astype(np.int32)), (s, b)
                for j in range(M):
                    p = lists[b][j].astype(np.int64)
                    want = np.where(p < S, p, np.where(p >= Tc - L, S + (p - T) % max(L, 1), -1))
                    want[want < 0] = S + L + sl[j]
                    assert np.array_equal(gr[b, j], want), (s, b, j)
            assert st.hits - prev.hits == h_s and st.misses - prev.misses == m_s, s
            prev = st
            assert skv.check(ws) == 0
            go = out.cpu().numpy()
            for b in check_seqs:
                for j in range(M):
                    o = oracle.tier_attention(q[b, j].numpy(), rec[b], rk[b], rv[b], rks[b], rvs[b],
                                              idx_np[b, j], Tc, S, L, sm, NQ // H, D)
                    err = float(np.max(np.abs(go[b, j] - o)))
                    assert err <= ATOL, (s, b, j, err)
    finally:
        tier.close()


@pytest.mark.parametrize("lru", [False, True])
def test_tier_multi_small(lru):
    _run(B=2, T=6000, S=16, L=32, k=64, M=4, n_slots=300, n_steps=5, shared=48, seed=5101, lru=lru)


def test_tier_multi_eight_queries_after_appends():
    """Eight query tokens after seven appended drafts: later queries' tail
    positions below the tier's tail are middle rows served by the buffer."""
    _run(B=2, T=6000, S=16, L=32, k=64, M=8, n_slots=700, n_steps=4, shared=40, seed=5102,
         appends=7)


@pytest.mark.parametrize("lru", [False, True])
def test_tier_multi_over_capacity_flagged(lru):
    """Lists that fit one by one but not together: the step is flagged, and the
    slot table it leaves is the same on every run (LRU: the misses outnumber
    the slots not used in the step, so every such slot is taken in slot order)."""
    skv = need_gpu()
    B, T, S, L, k, M = 1, 6000, 16, 32, 64, 4
    say("tier multi over capacity lru=%s" % lru)
    c = synth.make_tier_case(B, T, n_kv=H, n_q=NQ, D=D, S=S, k=k, L=L, seed=5103)
    desc = skv.token_desc(B, T, H, NQ, D, topk=k, n_sink=S, n_tail=L)
    lists = _lists(np.random.default_rng(5103), T, M, S, L, k, shared=8)   # ~232 distinct rows
    tables = []
    for _ in range(2):
        tier = skv.Tier(desc, T, 100, 1, policy=skv.SKV_TIER_LRU if lru else skv.SKV_TIER_CLOCK)
        try:
            tier.host_records()[:] = c.records.numpy()
            tier.load_resident(c.res_k.cuda(), c.res_v.cuda(), c.res_ks.cuda(), c.res_vs.cuda())
            cap = skv.select_capacity(desc)
            rows = torch.zeros((B, M, cap), dtype=torch.int32, device="cuda")
            nsel = torch.full((B, M), cap, dtype=torch.int32, device="cuda")
            # one list first, then all four at the next step number
            tier.resolve_multi(1, torch.from_numpy(np.stack(lists[:1])[None]).cuda(), nsel[:, :1].contiguous(), 0,
                               rows[:, :1].contiguous())
            tier.resolve_multi(M, torch.from_numpy(np.stack(lists)[None]).cuda(), nsel, 1, rows)
            with pytest.raises(skv.SkvError, match="0x8"):
                tier.stats()
            tables.append(tier.slots().copy())
        finally:
            tier.close()
    assert np.array_equal(tables[0], tables[1])


def test_tier_multi_full_config5():
    """Four sequences of 250,000 tokens (the host-tier benchmark shape), four
    query tokens sharing most picks, two steps; sequences 0 and 3 checked
    against the oracle attention, every sequence's slots and rows."""
    _run(B=4, T=250_000, S=64, L=1024, k=2048, M=4, n_slots=6250, n_steps=2, shared=1800,
         seed=5104, device="cuda", check_seqs=[0, 3])
