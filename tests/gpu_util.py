"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
on a generated case, run the oracle on the same bytes, compare."""

from __future__ import annotations

import sys
import time

import numpy as np
import pytest
import torch

import oracle
import synth

ATOL = 2e-3          # attention outputs: max abs error against the fp64 oracle


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import top_sparse_kv_amd as skv   # raises loudly if the library is missing
    skv.lib()
    return skv


def say(*a):
    print("[gpu-test %.1fs]" % time.monotonic(), *a, flush=True)
    sys.stdout.flush()


def np16(t: torch.Tensor) -> np.ndarray:
    """fp16 / bf16 tensor -> uint16 bit patterns (numpy, host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def token_desc_of(skv, c: synth.TokenCase):
    kvd = skv.SKV_KV_I8_ROWSCALE if c.kv_format == "i8" else skv.SKV_KV_F16
    return skv.token_desc(c.B, c.T_max, c.n_kv, c.n_q, c.D, rank=c.R, topk=c.k, n_sink=c.S,
                          n_tail=c.L, kv_dtype=kvd)


def block_desc_of(skv, c: synth.BlockCase):
    return skv.block_desc(c.B, c.T_max, c.n_kv, c.n_q, c.D, index_dim=c.index_dim, topk_blocks=c.k)


def to_dev(c, fields):
    return {f: (getattr(c, f).cuda() if getattr(c, f) is not None else None) for f in fields}


def run_token_gpu(skv, c: synth.TokenCase, sm_scale, *, fused=False, qs_in=None):
    """Runs qsketch/score/topk/attend on the GPU; returns host numpy results."""
    dev = to_dev(c, ["ctx_len", "q", "basis", "codes", "sk_scale", "k_cache", "v_cache",
                     "k_scale", "v_scale"])
    desc = token_desc_of(skv, c)
    cap = skv.select_capacity(desc)
    ws = skv.workspace(desc)
    qs = torch.zeros((c.B, c.n_kv * c.R), dtype=torch.int8, device="cuda")
    qsc = torch.zeros((c.B,), dtype=torch.float32, device="cuda")
    keys = torch.full((c.B, c.T_max), float("nan"), dtype=torch.float64, device="cuda")
    idx = torch.full((c.B, cap), -1, dtype=torch.int32, device="cuda")
    nsel = torch.zeros((c.B,), dtype=torch.int32, device="cuda")
    out = torch.zeros((c.B, c.n_q, c.D), dtype=torch.float32, device="cuda")
    kv = skv.kv_view(dev["k_cache"], dev["v_cache"], dev["k_scale"], dev["v_scale"])
    if fused:
        skv.step(desc, dev["ctx_len"], dev["q"], dev["basis"], qs, qsc, None, dev["codes"],
                 dev["sk_scale"], kv, idx, nsel, sm_scale, out, ws)
        # the fused step keeps no keys; score them separately for the key checks
        skv.score(desc, dev["ctx_len"], qs, dev["codes"], dev["sk_scale"], keys, ws)
    else:
        skv.qsketch(desc, dev["q"], dev["basis"], qs, qsc, ws)
        qs_use = qs if qs_in is None else torch.from_numpy(qs_in).cuda()
        skv.score(desc, dev["ctx_len"], qs_use, dev["codes"], dev["sk_scale"], keys, ws)
        skv.topk(desc, dev["ctx_len"], keys, idx, nsel, ws)
        skv.attend(desc, dev["q"], kv, idx, nsel, sm_scale, out, ws)
    flags = skv.check(ws)
    return dict(qs=qs.cpu().numpy(), qscale=qsc.cpu().numpy(), keys=keys.cpu().numpy(),
                idx=idx.cpu().numpy(), n_sel=nsel.cpu().numpy(), out=out.cpu().numpy().astype(np.float64),
                flags=flags)


def run_block_gpu(skv, c: synth.BlockCase, sm_scale, *, fused=False):
    dev = to_dev(c, ["ctx_len", "q", "qi", "kp", "k_cache", "v_cache"])
    desc = block_desc_of(skv, c)
    cap = skv.select_capacity(desc)
    ws = skv.workspace(desc)
    keys = torch.full((c.B, c.T_max // 4), float("nan"), dtype=torch.float64, device="cuda")
    idx = torch.full((c.B, cap), -1, dtype=torch.int32, device="cuda")
    nsel = torch.zeros((c.B,), dtype=torch.int32, device="cuda")
    out = torch.zeros((c.B, c.n_q, c.D), dtype=torch.float32, device="cuda")
    kv = skv.kv_view(dev["k_cache"], dev["v_cache"])
    if fused:
        skv.step(desc, dev["ctx_len"], dev["q"], None, None, None, dev["qi"], dev["kp"], None,
                 kv, idx, nsel, sm_scale, out, ws)
        skv.score(desc, dev["ctx_len"], dev["qi"], dev["kp"], None, keys, ws)
    else:
        skv.score(desc, dev["ctx_len"], dev["qi"], dev["kp"], None, keys, ws)
        skv.topk(desc, dev["ctx_len"], keys, idx, nsel, ws)
        skv.attend(desc, dev["q"], kv, idx, nsel, sm_scale, out, ws)
    flags = skv.check(ws)
    return dict(keys=keys.cpu().numpy(), idx=idx.cpu().numpy(), n_sel=nsel.cpu().numpy(),
                out=out.cpu().numpy().astype(np.float64), flags=flags)


def gather_rows(t: torch.Tensor, b: int, idx: np.ndarray) -> np.ndarray:
    """Rows idx of sequence b, copied to the host (plain torch indexing)."""
    if t is None:
        return None
    ii = torch.from_numpy(np.asarray(idx, dtype=np.int64)).to(t.device)
    return t[b].index_select(0, ii).cpu().numpy()


def oracle_token(c: synth.TokenCase, sm_scale, seqs=None):
    """Oracle A1..A4 on the case's bytes for the listed sequences."""
    seqs = list(range(c.B)) if seqs is None else list(seqs)
    q = c.q.cpu().numpy()
    basis = c.basis.cpu().numpy()
    qs, qscale = oracle.query_sketch(q, basis, c.group)
    codes = c.codes[seqs].cpu().numpy()
    sks = c.sk_scale[seqs].cpu().numpy()
    keys = np.full((c.B, c.T_max), np.nan)
    keys[seqs] = oracle.sketch_keys(qs[seqs], codes, sks, [c.lens[b] for b in seqs], c.S, c.k, c.L)
    idx, out = {}, {}
    fmt = c.kv_format
    for b in seqs:
        sel = oracle.select_tokens(keys[b], c.lens[b], c.S, c.k, c.L)
        idx[b] = sel
        kr, vr = gather_rows(c.k_cache, b, sel), gather_rows(c.v_cache, b, sel)
        ks = gather_rows(c.k_scale, b, sel) if c.k_scale is not None else None
        vs = gather_rows(c.v_scale, b, sel) if c.v_scale is not None else None
        if ks is not None:
            ks, vs = ks.view(np.float16), vs.view(np.float16)
        if fmt == "f16":
            kr, vr = kr.view(np.float16), vr.view(np.float16)
        loc = np.arange(sel.size)
        out[b] = oracle.sparse_attention(q[b], kr, vr, ks, vs, loc, sm_scale, c.group, fmt)
    return dict(qs=qs, qscale=qscale, keys=keys, idx=idx, out=out)


def oracle_block(c: synth.BlockCase, sm_scale, seqs=None):
    seqs = list(range(c.B)) if seqs is None else list(seqs)
    qi = np16(c.qi)
    kp = np16(c.kp[seqs])
    keys = np.full((c.B, c.T_max // 4), np.nan)
    keys[seqs] = oracle.pooled_keys(qi[seqs], kp, [c.lens[b] for b in seqs])
    q = np16(c.q)
    idx, out = {}, {}
    for b in seqs:
        sel = oracle.select_blocks(keys[b], c.lens[b], c.k)
        idx[b] = sel
        kr = gather_rows(c.k_cache.view(torch.int16), b, sel).view(np.uint16)
        vr = gather_rows(c.v_cache.view(torch.int16), b, sel).view(np.uint16)
        out[b] = oracle.sparse_attention(q[b], kr, vr, None, None, np.arange(sel.size), sm_scale,
                                         c.group, "bf16")
    return dict(keys=keys, idx=idx, out=out)


def compare_keys(gk, ok, b, lo, hi):
    a, e = gk[b, lo:hi], ok[b, lo:hi]
    bad = np.nonzero(~((a == e) | (np.isnan(a) & np.isnan(e))))[0]
    assert bad.size == 0, "seq %d: %d key mismatches, first at %d: gpu %r oracle %r" % (
        b, bad.size, lo + bad[0], a[bad[0]], e[bad[0]])


def compare_sel(g, o, b):
    n = int(g["n_sel"][b])
    got = g["idx"][b, :n]
    want = o["idx"][b]
    assert n == want.size, "seq %d: n_sel %d vs oracle %d" % (b, n, want.size)
    if not np.array_equal(got, want):
        diff = np.setdiff1d(want, got)
        raise AssertionError("seq %d: index sets differ (%d missing, e.g. %s)" % (b, diff.size, diff[:5]))


def compare_out(g, o, b, atol=ATOL):
    err = np.max(np.abs(g["out"][b] - o["out"][b])) if o["out"][b].size else 0.0
    assert err <= atol, "seq %d: max abs error %.3g > %.3g" % (b, err, atol)
    return err
