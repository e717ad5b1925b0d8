"""GPU parity of page residency in the host-RAM tier (full, mixed and no
residency over one page pool): every step, the resident row of every pick
(in place in a mapped page, hot slot, or a miss placed in a slot), the slot
table of the hot buffer and the in-place / hit / miss / host-byte counters must
equal the oracle's exactly; attention over the resolved rows within 2e-3 of the
fp64 oracle.  Pages are mapped and unmapped between steps, as a scheduler
under memory pressure would."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import ATOL, need_gpu, say

pytestmark = pytest.mark.gpu


def _schedule_mixed(n_pages, first_mid_page, last_mid_page, pool_pages, n_steps, churn, seed):
    """Per step, the (op, page, block) changes applied before it: the most
    recent middle pages start mapped; every 4 steps the `churn` lowest mapped
    pages are given up and as many random unmapped middle pages take their
    blocks."""
    rng = np.random.default_rng(seed)
    mapped = {}   # page -> block
    first = max(first_mid_page, last_mid_page - pool_pages + 1)
    ops = {0: [("map", g, i) for i, g in enumerate(range(first, last_mid_page + 1))]}
    for _, g, blk in ops[0]:
        mapped[g] = blk
    for s in range(4, n_steps, 4):
        out = []
        for g in sorted(mapped)[:churn]:
            out.append(("unmap", g, mapped.pop(g)))
        free = [blk for (_, _, blk) in out]
        cand = [g for g in range(first_mid_page, last_mid_page + 1) if g not in mapped]
        for blk, g in zip(free, rng.choice(cand, size=len(free), replace=False).tolist()):
            out.append(("map", g, blk))
            mapped[g] = blk
        ops[s] = out
    return ops


def _run(B, T, S, L, k, n_slots, P, pool_pages, n_steps, ops_of, check_out_steps, seed, lru,
         device="cpu"):
    skv = need_gpu()
    say("residency B=%d T=%d P=%d pool=%d slots=%d steps=%d lru=%s" % (B, T, P, pool_pages, n_slots,
                                                                     n_steps, lru))
    c = synth.make_tier_case(B, T, n_kv=4, n_q=24, D=256, S=S, k=k, L=L, seed=seed, device=device)
    picks = synth.drift_picks(B, T, S, L, k, n_steps, seed=seed,
                              window=min(65536, (T - S - L) // 2), sigma_c=256.0)
    desc = skv.token_desc(B, T, 4, 24, 256, topk=k, n_sink=S, n_tail=L)
    n_pages = (T + P - 1) // P
    tier = skv.Tier(desc, T, n_slots, 1, policy=skv.SKV_TIER_LRU if lru else skv.SKV_TIER_CLOCK,
                    page_tokens=P, pool_pages=pool_pages)
    try:
        tier.host_records()[:] = c.records.cpu().numpy()
        tier.load_resident(c.res_k.cuda(), c.res_v.cuda(), c.res_ks.cuda(), c.res_vs.cuda())
        cap = skv.select_capacity(desc)
        ws = skv.workspace(desc)
        rows = torch.zeros((B, cap), dtype=torch.int32, device="cuda")
        nsel = torch.full((B,), cap, dtype=torch.int32, device="cuda")
        out = torch.zeros((B, 24, 256), dtype=torch.float32, device="cuda")
        q = c.q.cuda()
        sm = 256 ** -0.5
        hot = [oracle.residency.LruTier(n_slots, T) if lru else oracle.ClockTier(n_slots, T) for _ in range(B)]
        ref = [oracle.residency.PagedTier(h, P, n_pages) for h in hot]
        rec_np = c.records.cpu().numpy()
        # the int8 rows the GPU holds for each sequence: sinks, tail, mapped pages
        k8 = np.zeros((B, T, 4, 256), np.int8)
        v8 = np.zeros((B, T, 4, 256), np.int8)
        ks = np.zeros((B, T, 4), np.float16)
        vs = np.zeros((B, T, 4), np.float16)
        res_np = [t.cpu().numpy() for t in (c.res_k, c.res_v, c.res_ks, c.res_vs)]

        def put_resident():
            # sinks and tail come from the resident rows whatever page holds them
            for b in range(B):
                for arr, x in zip((k8, v8, ks, vs), res_np):
                    arr[b, :S] = x[b, :S]
                    arr[b, T - L:] = x[b, S:]

        put_resident()
        prev = tier.stats()
        n_in_tot = n_h_tot = n_m_tot = 0
        for s in range(n_steps):
            ops = ops_of(s)
            if ops:
                pages = [(b, g) for (b, op, g, blk) in ops if op == "map"]
                rk, rks, rv, rvs = synth.tier_page_rows(B, T, n_kv=4, D=256, seed=seed, page_tokens=P,
                                                        pages=pages, device="cuda")
                j = 0
                for (b, op, g, blk) in ops:
                    if op == "unmap":
                        tier.unmap_page(b, g)
                        ref[b].unmap_page(g)
                    else:
                        tier.map_page(b, g, blk, rk[j], rv[j], rks[j], rvs[j])
                        ref[b].map_page(g, blk)
                        m = min(P, T - g * P)
                        k8[b, g * P:g * P + m] = rk[j, :m].cpu().numpy()
                        v8[b, g * P:g * P + m] = rv[j, :m].cpu().numpy()
                        ks[b, g * P:g * P + m] = rks[j, :m].cpu().numpy()
                        vs[b, g * P:g * P + m] = rvs[j, :m].cpu().numpy()
                        j += 1
                put_resident()
            idx_np = np.concatenate([np.broadcast_to(np.arange(S), (B, S)), picks[s],
                                     np.broadcast_to(np.arange(T - L, T), (B, L))], axis=1).astype(np.int32)
            idx = torch.from_numpy(idx_np).cuda()
            tier.resolve(idx, nsel, s, rows)
            tier.attend(q, rows, nsel, sm, out, ws)
            st = tier.stats()
            slots = tier.slots()
            gr = rows.cpu().numpy()
            n_in = n_h = n_m = 0
            for b in range(B):
                kind, where, (a_in, a_h, a_m) = ref[b].step(picks[s, b], s)
                n_in += a_in
                n_h += a_h
                n_m += a_m
                pool0 = S + L + n_slots
                mid = np.where(kind == oracle.residency.IN_PLACE, pool0 + where, S + L + where)
                want_rows = np.concatenate([np.arange(S), mid, S + np.arange(L)])
                assert np.array_equal(gr[b], want_rows), "step %d seq %d rows" % (s, b)
                assert np.array_equal(slots[b], hot[b].pos.astype(np.int32)), "step %d seq %d slots" % (s, b)
            d = (st.in_place - prev.in_place, st.hits - prev.hits, st.misses - prev.misses)
            assert d == (n_in, n_h, n_m), "step %d counts %s vs %s" % (s, d, (n_in, n_h, n_m))
            assert st.picks - prev.picks == n_in + n_h + n_m
            assert st.host_bytes - prev.host_bytes == n_m * 4 * 272
            prev = st
            n_in_tot += n_in
            n_h_tot += n_h
            n_m_tot += n_m
            if s in check_out_steps:
                go = out.cpu().numpy()
                for b in range(B):
                    o = oracle.paged_tier_attention(c.q[b].cpu().numpy(), rec_np[b], k8[b], v8[b], ks[b],
                                                    vs[b], idx_np[b], T, S, L, ref[b].block, P, sm, 6, 256)
                    err = float(np.max(np.abs(go[b] - o)))
                    assert err <= ATOL, "step %d seq %d err %g" % (s, b, err)
        assert skv.check(ws) == 0
        say("residency in place / hits / misses", n_in_tot, n_h_tot, n_m_tot)
        return n_in_tot, n_h_tot, n_m_tot
    finally:
        tier.close()


def _per_seq(B, sched):
    """The same page schedule for every sequence (block ids per sequence)."""
    return lambda s: [(b, op, g, blk) for b in range(B) for (op, g, blk) in sched.get(s, [])]


def test_residency_mixed_small_lru():
    B, T, S, L, k, P, pool = 2, 40_000, 64, 1024, 256, 64, 160
    n_pages = (T + P - 1) // P
    sched = _schedule_mixed(n_pages, S // P + 1, (T - L) // P - 1, pool, 24, churn=16, seed=3)
    n_in, h, m = _run(B, T, S, L, k, 512, P, pool, 24, _per_seq(B, sched), {0, 4, 13, 23}, seed=61,
                      lru=True)
    assert n_in > 0 and h > 0 and m > 0


def test_residency_mixed_small_clock():
    B, T, S, L, k, P, pool = 1, 30_000, 16, 128, 200, 32, 200
    n_pages = (T + P - 1) // P
    sched = _schedule_mixed(n_pages, S // P + 1, (T - L) // P - 1, pool, 16, churn=24, seed=4)
    n_in, h, m = _run(B, T, S, L, k, 750, P, pool, 16, _per_seq(B, sched), {2, 15}, seed=62, lru=False)
    assert n_in > 0 and h > 0 and m > 0


def test_residency_none_full_none():
    """No residency for 4 steps, then every page mapped (full residency: every
    middle pick in place, the hot buffer untouched), then every page given up
    again (the hot rows left from the first phase are hits again)."""
    B, T, S, L, k, P = 1, 20_000, 16, 128, 200, 64
    n_pages = (T + P - 1) // P
    sched = {4: [("map", g, g) for g in range(n_pages)], 8: [("unmap", g, g) for g in range(n_pages)]}
    n_in, h, m = _run(B, T, S, L, k, 600, P, n_pages, 12, _per_seq(B, sched), {3, 5, 8, 11}, seed=63,
                      lru=True)
    assert n_in == 4 * k


def test_residency_mixed_config5():
    """Config-5 shape (4 x 250,000, LRU hot buffer of 2 x 2048 slots) with a
    pool of 1,024 pages of 64 tokens (26% of each sequence resident), the
    mapping changing every 4 steps."""
    B, T, S, L, k, P, pool = 4, 250_000, 64, 1024, 2048, 64, 1024
    n_pages = (T + P - 1) // P
    sched = _schedule_mixed(n_pages, S // P + 1, (T - L) // P - 1, pool, 24, churn=128, seed=5)
    n_in, h, m = _run(B, T, S, L, k, 4096, P, pool, 24, _per_seq(B, sched), {0, 23}, seed=1005,
                      lru=True, device="cuda")
    assert n_in > 0 and h > 0 and m > 0
