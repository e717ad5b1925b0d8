"""GPU parity of the tier append (sparsekv_tier_append through the C ABI)
against oracle.append on the same bytes: the host record of every appended
token, the int8 rows in the tail ring, the key sketch and the contexts are
bit-exact; resolve + attention over a tier that has appended past its tail
(so appended tokens are served from their host records) stay within 2e-3 of
the fp64 oracle; a full sequence and a sequence whose context disagrees with
the tier are left unchanged and flagged."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import ATOL, need_gpu, say

pytestmark = pytest.mark.gpu

H, NQ, D, R = 4, 24, 256, 64


class _Dev:
    """Borrowed view of device memory the library owns (for reading it back)."""

    def __init__(self, ptr, shape, typestr):
        self.__cuda_array_interface__ = {"shape": tuple(shape), "typestr": typestr,
                                         "data": (int(ptr), False), "version": 2}


def _resident(res, B, rows):
    k = torch.as_tensor(_Dev(res.k, (B, rows, H, D), "|i1"), device="cuda").cpu().numpy()
    v = torch.as_tensor(_Dev(res.v, (B, rows, H, D), "|i1"), device="cuda").cpu().numpy()
    ks = torch.as_tensor(_Dev(res.k_scale, (B, rows, H), "<f2"), device="cuda").cpu().numpy()
    vs = torch.as_tensor(_Dev(res.v_scale, (B, rows, H), "<f2"), device="cuda").cpu().numpy()
    return k, v, ks, vs


class _Setup:
    def __init__(self, skv, B, T0, cap, S, L, k, n_slots, seed, device="cpu"):
        self.skv, self.B, self.T0, self.cap, self.S, self.L, self.k = skv, B, T0, cap, S, L, k
        c = synth.make_tier_case(B, T0, n_kv=H, n_q=NQ, D=D, S=S, k=k, L=L, seed=seed, device=device)
        self.c = c
        self.q_np = c.q.cpu().numpy()
        recs = c.records.cpu().numpy()
        self.desc = skv.token_desc(B, cap, H, NQ, D, topk=k, n_sink=S, n_tail=L)
        self.tier = skv.Tier(self.desc, T0, n_slots, 1)
        self.tier.host_records()[:, :T0] = recs
        self.tier.load_resident(c.res_k.cuda(), c.res_v.cuda(), c.res_ks.cuda(), c.res_vs.cuda())
        self.basis = synth.orthonormal_basis(H, D, R, seed).cuda()
        self.codes = torch.zeros((B, cap, H * R // 2), dtype=torch.uint8, device="cuda")
        self.sksc = torch.zeros((B, cap), dtype=torch.float16, device="cuda")
        self.ctx = torch.full((B,), T0, dtype=torch.int32, device="cuda")
        # oracle state: records by position, sinks + tail in position order
        rb = c.records.shape[-1]
        self.rec = np.zeros((B, cap, H, rb), dtype=np.uint8)
        self.rec[:, :T0] = recs
        del recs
        self.rk, self.rv = c.res_k.cpu().numpy().copy(), c.res_v.cpu().numpy().copy()
        self.rks, self.rvs = c.res_ks.cpu().numpy().copy(), c.res_vs.cpu().numpy().copy()
        self.T = [T0] * B
        self.want_codes = {}
        self.g = torch.Generator().manual_seed(seed + 7)

    def append(self, active=None):
        B = self.B
        kn = (torch.randn((B, H, D), generator=self.g) * 2.0).to(torch.float16)
        vn = torch.randn((B, H, D), generator=self.g).to(torch.float16)
        self.tier.append(self.ctx, kn.cuda(), vn.cuda(), self.basis, self.codes, self.sksc)
        bas = self.basis.cpu().numpy()
        for b in range(B):
            if active is not None and not active[b]:
                continue
            if self.T[b] >= self.cap:
                continue
            t = self.T[b]
            self.want_codes[(b, t)] = oracle.append.key_sketch(kn[b].numpy(), bas)
            self.T[b] = oracle.append.tier_append_token(
                t, self.rec[b], self.rk[b], self.rv[b], self.rks[b], self.rvs[b], self.S, self.L,
                kn[b].numpy(), vn[b].numpy())

    def check_state(self):
        torch.cuda.synchronize()
        B, S, L = self.B, self.S, self.L
        assert self.ctx.cpu().numpy().tolist() == self.T
        hr = self.tier.host_records()
        assert np.array_equal(hr, self.rec), "host records"
        codes, sk = self.codes.cpu().numpy(), self.sksc.cpu().numpy()
        for (b, t), (cw, sw) in self.want_codes.items():
            assert np.array_equal(codes[b, t], cw) and sk[b, t].view(np.uint16) == np.float16(sw).view(np.uint16), (b, t)
        rk, rv, rks, rvs = _resident(self.tier.resident(), B, S + L + self.tier.n_slots)
        for b in range(B):
            T = self.T[b]
            assert np.array_equal(rk[b, :S], self.rk[b, :S]) and np.array_equal(rks[b, :S], self.rks[b, :S])
            for i in range(L):
                p = T - L + i
                row = S + (p - self.T0) % L
                assert np.array_equal(rk[b, row], self.rk[b, S + i]), (b, p)
                assert np.array_equal(rv[b, row], self.rv[b, S + i]), (b, p)
                assert np.array_equal(rks[b, row].view(np.uint16), self.rks[b, S + i].view(np.uint16)), (b, p)
                assert np.array_equal(rvs[b, row].view(np.uint16), self.rvs[b, S + i].view(np.uint16)), (b, p)

    def step_and_check(self, s, rng, force=()):
        """Resolve + attend with middle picks drawn from the current middle
        range (including the given positions), checked against the oracle."""
        skv, B, S, L, k = self.skv, self.B, self.S, self.L, self.k
        cap = skv.select_capacity(self.desc)
        idx_np = np.zeros((B, cap), dtype=np.int32)
        for b in range(B):
            T = self.T[b]
            mid = [p for p in force if S <= p < T - L]
            pool = np.setdiff1d(np.arange(S, T - L), mid)
            pick = np.sort(np.concatenate([mid, rng.choice(pool, k - len(mid), replace=False)]))
            idx_np[b] = np.concatenate([np.arange(S), pick, np.arange(T - L, T)])
        idx = torch.from_numpy(idx_np).cuda()
        nsel = torch.full((B,), cap, dtype=torch.int32, device="cuda")
        rows = torch.zeros((B, cap), dtype=torch.int32, device="cuda")
        out = torch.zeros((B, NQ, D), dtype=torch.float32, device="cuda")
        ws = skv.workspace(self.desc)
        self.tier.resolve(idx, nsel, s, rows)
        skv.attend(self.desc, self.c.q.cuda(), self.tier.resident(), rows, nsel, D ** -0.5, out, ws)
        self.tier.stats()                      # raises on any tier flag
        assert skv.check(ws) == 0
        gr, go = rows.cpu().numpy(), out.cpu().numpy()
        for b in range(B):
            T = self.T[b]
            tail = gr[b, S + k:]
            assert tail.tolist() == [S + (p - self.T0) % L for p in range(T - L, T)], b
            o = oracle.tier_attention(self.q_np[b], self.rec[b], self.rk[b], self.rv[b],
                                      self.rks[b], self.rvs[b], idx_np[b], T, S, L, D ** -0.5,
                                      NQ // H, D)
            err = float(np.max(np.abs(go[b] - o)))
            assert err <= ATOL, (s, b, err)


def test_tier_append_ring_and_records():
    """40 appends through a 24-row tail ring (wrapping it), states checked
    after several of them, and steps whose picks include appended tokens that
    have left the tail (served from the records the append wrote)."""
    skv = need_gpu()
    B, T0, cap, S, L, k = 2, 3000, 3100, 16, 24, 64
    say("tier append ring B=%d T0=%d L=%d" % (B, T0, L))
    st = _Setup(skv, B, T0, cap, S, L, k, 200, seed=4101)
    rng = np.random.default_rng(4101)
    try:
        st.step_and_check(0, rng)
        for n in range(1, 41):
            st.append()
            if n in (1, 5, 24, 25, 40):
                st.check_state()
            if n in (30, 40):
                st.step_and_check(n, rng, force=list(range(T0, T0 + n - L)))
    finally:
        st.tier.close()


def test_tier_append_capacity_and_mismatch_flags():
    """At capacity the append leaves the sequence unchanged and raises
    SKV_FLAG_CTX_RANGE; a ctx_len that differs from the tier's context skips
    that sequence (SKV_FLAG_TIER_INPUT) while the others append."""
    skv = need_gpu()
    B, T0, S, L, k = 2, 3000, 16, 24, 64
    st = _Setup(skv, B, T0, T0 + 2, S, L, k, 200, seed=4102)
    try:
        st.append()
        st.append()
        st.check_state()
        st.append()                               # both sequences full
        st.check_state()
        with pytest.raises(skv.SkvError, match="0x1"):
            st.tier.stats()
    finally:
        st.tier.close()
    st = _Setup(skv, B, T0, T0 + 50, S, L, k, 200, seed=4103)
    try:
        st.append()
        st.ctx[1] += 1                            # sequence 1 disagrees with the tier
        st.append(active=[True, False])
        st.ctx[1] -= 1
        st.check_state()
        with pytest.raises(skv.SkvError, match="0x8"):
            st.tier.stats()
    finally:
        st.tier.close()


def test_tier_append_no_tail():
    """With no tail the append writes the host record and the sketch only;
    the appended token is then a middle position served from its record."""
    skv = need_gpu()
    B, T0, S, L, k = 2, 2000, 16, 0, 64
    st = _Setup(skv, B, T0, T0 + 8, S, L, k, 200, seed=4104)
    rng = np.random.default_rng(4104)
    try:
        for _ in range(5):
            st.append()
        st.check_state()
        st.step_and_check(1, rng, force=list(range(T0, T0 + 5)))
    finally:
        st.tier.close()


def test_tier_append_full_config5():
    """Four sequences of 250,000 tokens (the host-tier benchmark shape), three
    appends, then a step whose picks include an appended token; sequence 0 and
    3 are checked against the oracle."""
    skv = need_gpu()
    B, T0, S, L, k = 4, 250_000, 64, 1024, 2048
    say("tier append full size: generating")
    st = _Setup(skv, B, T0, T0 + 16, S, L, k, int(0.025 * T0), seed=4105, device="cuda")
    try:
        for _ in range(3):
            st.append()
        torch.cuda.synchronize()
        assert st.ctx.cpu().numpy().tolist() == [T0 + 3] * B
        hr = st.tier.host_records()
        for b in range(B):
            assert np.array_equal(hr[b, T0:T0 + 3], st.rec[b, T0:T0 + 3])
        rng = np.random.default_rng(4105)
        # one step over the batch; the oracle checks two sequences
        cap = skv.select_capacity(st.desc)
        idx_np = np.zeros((B, cap), dtype=np.int32)
        for b in range(B):
            T = st.T[b]
            pick = np.sort(rng.choice(np.arange(S, T - L), k, replace=False))
            idx_np[b] = np.concatenate([np.arange(S), pick, np.arange(T - L, T)])
        idx = torch.from_numpy(idx_np).cuda()
        nsel = torch.full((B,), cap, dtype=torch.int32, device="cuda")
        rows = torch.zeros((B, cap), dtype=torch.int32, device="cuda")
        out = torch.zeros((B, NQ, D), dtype=torch.float32, device="cuda")
        ws = skv.workspace(st.desc)
        st.tier.resolve(idx, nsel, 0, rows)
        skv.attend(st.desc, st.c.q.cuda(), st.tier.resident(), rows, nsel, D ** -0.5, out, ws)
        st.tier.stats()
        go = out.cpu().numpy()
        for b in (0, 3):
            T = st.T[b]
            o = oracle.tier_attention(st.q_np[b], st.rec[b], st.rk[b], st.rv[b], st.rks[b],
                                      st.rvs[b], idx_np[b], T, S, L, D ** -0.5, NQ // H, D)
            err = float(np.max(np.abs(go[b] - o)))
            say("tier append full size seq", b, "err", err)
            assert err <= ATOL
    finally:
        st.tier.close()
