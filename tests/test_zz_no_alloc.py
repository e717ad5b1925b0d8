"""sparsekv_step_noalloc (the step in the library's own device scratch) against
sparsekv_step with a caller workspace, through the C ABI, on the same seeded
inputs.  Both run the same kernels, so every output must be identical bit for
bit: query sketch codes and scale, index lists and counts, attention output and
the device flag word.  The calls come in a row on one device, each smaller than
the one before, so a later call runs over what an earlier one left in the
scratch."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import block_desc_of, need_gpu, say, to_dev, token_desc_of


def _token_case(B, T, lens, seed):
    return synth.make_token_case(B, T, lens, n_kv=4, n_q=24, D=256, S=64, k=2048, L=1024,
                                 kv_format="i8", seed=seed)


def _block_case(B, T, lens, seed):
    return synth.make_block_case(B, T, lens, n_kv=2, n_q=16, D=256, k=512, seed=seed)


def _run_token(skv, c, sm, noalloc):
    dev = to_dev(c, ["ctx_len", "q", "basis", "codes", "sk_scale", "k_cache", "v_cache",
                     "k_scale", "v_scale"])
    desc = token_desc_of(skv, c)
    cap = skv.select_capacity(desc)
    qs = torch.full((c.B, c.n_kv * c.R), 77, dtype=torch.int8, device="cuda")
    qsc = torch.full((c.B,), -1.0, dtype=torch.float32, device="cuda")
    idx = torch.full((c.B, cap), -1, dtype=torch.int32, device="cuda")
    nsel = torch.full((c.B,), -1, dtype=torch.int32, device="cuda")
    out = torch.full((c.B, c.n_q, c.D), float("nan"), dtype=torch.float32, device="cuda")
    kv = skv.kv_view(dev["k_cache"], dev["v_cache"], dev["k_scale"], dev["v_scale"])
    if noalloc:
        flags = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        skv.step_noalloc(desc, dev["ctx_len"], dev["q"], dev["basis"], qs, qsc, None, dev["codes"],
                         dev["sk_scale"], kv, idx, nsel, sm, out, flags)
        f = int(flags.cpu().numpy().view(np.uint32)[0])
    else:
        ws = skv.workspace(desc)
        skv.step(desc, dev["ctx_len"], dev["q"], dev["basis"], qs, qsc, None, dev["codes"],
                 dev["sk_scale"], kv, idx, nsel, sm, out, ws)
        f = skv.check(ws)
    torch.cuda.synchronize()
    return dict(qs=qs.cpu().numpy(), qscale=qsc.cpu().numpy().view(np.uint32), idx=idx.cpu().numpy(),
                n_sel=nsel.cpu().numpy(), out=out.cpu().numpy().view(np.uint32), flags=f)


def _run_block(skv, c, sm, noalloc):
    dev = to_dev(c, ["ctx_len", "q", "qi", "kp", "k_cache", "v_cache"])
    desc = block_desc_of(skv, c)
    cap = skv.select_capacity(desc)
    idx = torch.full((c.B, cap), -1, dtype=torch.int32, device="cuda")
    nsel = torch.full((c.B,), -1, dtype=torch.int32, device="cuda")
    out = torch.full((c.B, c.n_q, c.D), float("nan"), dtype=torch.float32, device="cuda")
    kv = skv.kv_view(dev["k_cache"], dev["v_cache"])
    if noalloc:
        flags = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        skv.step_noalloc(desc, dev["ctx_len"], dev["q"], None, None, None, dev["qi"], dev["kp"], None,
                         kv, idx, nsel, sm, out, flags)
        f = int(flags.cpu().numpy().view(np.uint32)[0])
    else:
        ws = skv.workspace(desc)
        skv.step(desc, dev["ctx_len"], dev["q"], None, None, None, dev["qi"], dev["kp"], None,
                 kv, idx, nsel, sm, out, ws)
        f = skv.check(ws)
    torch.cuda.synchronize()
    return dict(idx=idx.cpu().numpy(), n_sel=nsel.cpu().numpy(), out=out.cpu().numpy().view(np.uint32),
                flags=f)


def _same(a, b, what):
    for key in a:
        if key == "flags":
            assert a[key] == b[key], "%s: flags 0x%x != 0x%x" % (what, a[key], b[key])
        else:
            assert np.array_equal(a[key], b[key]), "%s: %s differs" % (what, key)


@pytest.mark.gpu
def test_noalloc_step_matches_workspace_step():
    skv = need_gpu()
    sm = 256 ** -0.5
    # a full-length 8 x 250,000 batch first (33 MiB of the 64 MiB scratch), then
    # smaller ones that reuse what it left
    calls = [("token 8 x 250,000", lambda: _token_case(8, 250_000, None, 2001), _run_token),
             ("token ragged 3 x 40,960", lambda: _token_case(3, 40_960, [40_000, 17_001, 3_137], 2002),
              _run_token),
             ("token dense 2 x 3,136", lambda: _token_case(2, 3_136, [3_136, 1_000], 2003), _run_token),
             ("block 1 x 20,000", lambda: _block_case(1, 20_000, None, 2004), _run_block)]
    for what, make, run in calls:
        say("noalloc:", what)
        c = make()
        ref = run(skv, c, sm, noalloc=False)
        got = run(skv, c, sm, noalloc=True)
        _same(got, ref, what)
        again = run(skv, c, sm, noalloc=True)   # the same call twice in a row
        _same(again, ref, what + " (repeat)")
        say("noalloc:", what, "identical; n_sel", ref["n_sel"].tolist()[:4], "flags 0x%x" % ref["flags"])


def test_noalloc_rejects_a_layer_beyond_the_scratch():
    """Host-side check, no GPU needed: a layer whose workspace exceeds the
    scratch is refused before anything is launched."""
    import top_sparse_kv_amd as skv
    lib = skv.lib()
    assert lib.sparsekv_abi_version() >= 5
    big = skv.token_desc(32, 250_000, 4, 24, 256, topk=2048, n_sink=64, n_tail=1024)
    assert skv.workspace_size(big) > (64 << 20)
    kv = skv.KVView(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), 250_000)
    one = ctypes.c_void_p(256)
    st = lib.sparsekv_step_noalloc(ctypes.byref(big), one, one, one, one, one, None, one, one,
                                   ctypes.byref(kv), one, one, 0.0625, one, None, None)
    assert skv._lib.STATUS[st] == "SKV_ERR_WORKSPACE"
    assert b"scratch" in lib.sparsekv_last_error()
    small = skv.token_desc(8, 250_000, 4, 24, 256, topk=2048, n_sink=64, n_tail=1024)
    assert skv.workspace_size(small) <= (64 << 20)
    st = lib.sparsekv_step_noalloc(ctypes.byref(small), None, one, one, one, one, None, one, one,
                                   ctypes.byref(kv), one, one, 0.0625, one, None, None)
    assert skv._lib.STATUS[st] == "SKV_ERR_INVALID"   # NULL ctx_len, refused on the host
