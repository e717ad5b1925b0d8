"""GPU parity of the host-RAM tier: slot assignment of the windowed CLOCK and
of the LRU hot buffer, hit / miss counts and host bytes must equal the
oracle's exactly, every step; attention over the resolved rows within 2e-3 of
the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import ATOL, need_gpu, say

pytestmark = pytest.mark.gpu


def _run(B, T, S, L, k, n_slots, n_steps, check_out_steps, seed, window=1, device="cpu",
         lru=False):
    skv = need_gpu()
    say("tier B=%d T=%d k=%d slots=%d steps=%d lru=%s" % (B, T, k, n_slots, n_steps, lru))
    c = synth.make_tier_case(B, T, n_kv=4, n_q=24, D=256, S=S, k=k, L=L, seed=seed, device=device)
    picks = synth.drift_picks(B, T, S, L, k, n_steps, seed=seed,
                              window=min(65536, (T - S - L) // 2), sigma_c=256.0)
    desc = skv.token_desc(B, T, 4, 24, 256, topk=k, n_sink=S, n_tail=L)
    tier = skv.Tier(desc, T, n_slots, window,
                    policy=skv.SKV_TIER_LRU if lru else skv.SKV_TIER_CLOCK)
    try:
        tier.host_records()[:] = c.records.cpu().numpy()
        tier.load_resident(c.res_k.cuda(), c.res_v.cuda(), c.res_ks.cuda(), c.res_vs.cuda())
        res = tier.resident()
        cap = skv.select_capacity(desc)
        ws = skv.workspace(desc)
        rows = torch.zeros((B, cap), dtype=torch.int32, device="cuda")
        nsel = torch.full((B,), cap, dtype=torch.int32, device="cuda")
        out = torch.zeros((B, 24, 256), dtype=torch.float32, device="cuda")
        q = c.q.cuda()
        sm = 256 ** -0.5
        ref = [oracle.residency.LruTier(n_slots, T) if lru else oracle.ClockTier(n_slots, T, window=window)
               for _ in range(B)]
        rec_np = c.records.cpu().numpy()
        rk, rv = c.res_k.cpu().numpy(), c.res_v.cpu().numpy()
        rks, rvs = c.res_ks.cpu().numpy(), c.res_vs.cpu().numpy()
        tot_h = tot_m = 0
        prev = tier.stats()
        for s in range(n_steps):
            idx_np = np.concatenate([np.broadcast_to(np.arange(S), (B, S)), picks[s],
                                     np.broadcast_to(np.arange(T - L, T), (B, L))], axis=1).astype(np.int32)
            idx = torch.from_numpy(idx_np).cuda()
            tier.resolve(idx, nsel, s, rows)
            tier.attend(q, rows, nsel, sm, out, ws)
            st = tier.stats()
            slots = tier.slots()
            h_s = m_s = 0
            for b in range(B):
                sl, h, m = ref[b].step(picks[s, b], s)
                h_s += h
                m_s += m
                assert np.array_equal(slots[b], ref[b].pos.astype(np.int32)), "step %d seq %d slot table" % (s, b)
            assert st.hits - prev.hits == h_s and st.misses - prev.misses == m_s, "step %d counts" % s
            assert st.host_bytes - prev.host_bytes == m_s * 4 * 272
            prev = st
            tot_h += h_s
            tot_m += m_s
            if s in check_out_steps:
                go = out.cpu().numpy()
                gr = rows.cpu().numpy()
                for b in range(B):
                    want_rows = np.concatenate([np.arange(S), S + L + ref[b].slot_of[picks[s, b]],
                                                S + np.arange(L)])
                    assert np.array_equal(gr[b], want_rows), "step %d seq %d rows" % (s, b)
                    o = oracle.tier_attention(c.q[b].cpu().numpy(), rec_np[b], rk[b], rv[b], rks[b], rvs[b],
                                              idx_np[b], T, S, L, sm, 6, 256)
                    err = float(np.max(np.abs(go[b] - o)))
                    assert err <= ATOL, "step %d seq %d err %g" % (s, b, err)
        assert skv.check(ws) == 0
        return tot_h, tot_m
    finally:
        tier.close()


def test_tier_small():
    h, m = _run(B=2, T=40_000, S=64, L=1024, k=256, n_slots=1000, n_steps=24,
                check_out_steps={0, 5, 23}, seed=55)
    say("tier small miss rate", m / (h + m))


def test_tier_window_two():
    _run(B=1, T=30_000, S=16, L=128, k=200, n_slots=750, n_steps=16, check_out_steps={3, 15},
         seed=56, window=2)


def test_tier_full_config5():
    """Config-5 shape: 4 x 250,000 tokens, 6,250 hot slots (2.5%), drifting picks."""
    h, m = _run(B=4, T=250_000, S=64, L=1024, k=2048, n_slots=6250, n_steps=40,
                check_out_steps={0, 39}, seed=1005, device="cuda")
    say("tier cfg5 miss rate over 40 steps", m / (h + m))


def test_tier_lru_small():
    """LRU hot buffer of 2 x top-k slots (the HiSparse default)."""
    h, m = _run(B=2, T=40_000, S=64, L=1024, k=256, n_slots=512, n_steps=24,
                check_out_steps={0, 7, 23}, seed=57, lru=True)
    say("tier lru small miss rate", m / (h + m))


def test_tier_lru_exact_capacity():
    """n_slots = top-k: every slot not hit this step is a candidate."""
    _run(B=1, T=20_000, S=16, L=128, k=200, n_slots=200, n_steps=12, check_out_steps={11},
         seed=58, lru=True)


def test_tier_lru_full_config5():
    """Config-5 shape with the LRU policy at 2 x 2048 = 4096 slots."""
    h, m = _run(B=4, T=250_000, S=64, L=1024, k=2048, n_slots=4096, n_steps=40,
                check_out_steps={0, 39}, seed=1005, device="cuda", lru=True)
    say("tier lru cfg5 miss rate over 40 steps", m / (h + m))
