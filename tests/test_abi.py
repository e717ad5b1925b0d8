"""C ABI checks that need no GPU: the library loads, exports every function
include/sparsekv.h declares, and rejects bad descriptors and arguments on the
host with the documented status before touching the device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparsekv.h")


@pytest.fixture(scope="module")
def skv():
    from top_sparse_kv_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from top_sparse_kv_amd import build
        build.build()
    import top_sparse_kv_amd as m
    m.lib()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparsekv_\w+)\s*\(", text)))


def test_header_declarations_are_exported(skv):
    from top_sparse_kv_amd import _lib
    names = declared_functions()
    assert len(names) >= 20
    lib = skv.lib()
    bound = {n for n, _, _ in _lib.SIGNATURES}
    for n in names:
        assert hasattr(lib, n), n
        assert n in bound, "binding lacks " + n


def declared_arity():
    """Parameter count of every function the header declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for name, params in re.findall(r"\b(sparsekv_\w+)\s*\(([^)]*)\)\s*;", text):
        params = params.strip()
        out[name] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_arity_matches_header(skv):
    from top_sparse_kv_amd import _lib
    arity = declared_arity()
    assert len(arity) == len(declared_functions())
    for name, _, args in _lib.SIGNATURES:
        assert arity[name] == len(args), (name, arity[name], len(args))


def test_struct_sizes_match_header(skv):
    # the C structs are plain int32 / pointer layouts; sizes pinned here
    assert ctypes.sizeof(skv.LayerDesc) == 15 * 4
    assert ctypes.sizeof(skv.KVView) == 5 * 8
    # skv_tier_desc: size, layer, ctx, n_slots, window, (pad) host pointer, policy,
    # page_tokens, pool_pages, (pad); skv_tier_stats: six int64
    assert ctypes.sizeof(skv.TierDesc) == 104
    assert ctypes.sizeof(skv.TierStats) == 6 * 8
    assert skv.abi_version() == 7


def test_capacity_and_workspace(skv):
    d2 = skv.token_desc(8, 250_000, 4, 24, 256, topk=2048, n_sink=64, n_tail=1024)
    d1 = skv.token_desc(1, 4096, 2, 8, 128, topk=256, n_sink=16, n_tail=128, kv_dtype=skv.SKV_KV_F16)
    d3 = skv.block_desc(1, 1_048_576, 2, 16, 256, topk_blocks=512)
    assert skv.select_capacity(d2) == 3136
    assert skv.select_capacity(d1) == 400
    assert skv.select_capacity(d3) == 2051
    for d in (d1, d2, d3):
        assert skv.workspace_size(d) > 0 and skv.workspace_size(d) % 256 == 0


BAD = [
    (dict(head_dim=192), 2),
    (dict(n_q_heads=25), 1),
    (dict(n_q_heads=4 * 17), 2),
    (dict(topk=0), 2),
    (dict(topk=5000), 2),
    (dict(batch=0), 1),
    (dict(max_ctx=0), 1),
    (dict(block=4), 1),
    (dict(rank=63), 2),
    (dict(n_sink=-1), 1),
    (dict(kv_dtype=2), 2),
    (dict(q_dtype=1), 2),
    (dict(index_mode=7), 1),
    (dict(struct_size=8), 1),
]


@pytest.mark.parametrize("change,status", BAD)
def test_bad_descriptor(skv, change, status):
    d = skv.token_desc(8, 250_000, 4, 24, 256, topk=2048, n_sink=64, n_tail=1024)
    for k, v in change.items():
        setattr(d, k, v)
    st = skv.lib().sparsekv_validate(ctypes.byref(d))
    assert st == status, (change, st, skv.lib().sparsekv_last_error())
    assert skv.lib().sparsekv_last_error()


def test_bad_block_descriptor(skv):
    d = skv.block_desc(1, 1 << 20, 2, 16, 256, topk_blocks=512)
    d.n_sink = 4
    assert skv.lib().sparsekv_validate(ctypes.byref(d)) == 2
    d = skv.block_desc(1, 1 << 20, 2, 16, 256, topk_blocks=512)
    d.kv_dtype = skv.SKV_KV_F16
    assert skv.lib().sparsekv_validate(ctypes.byref(d)) == 2
    d = skv.block_desc(1, 1 << 20, 2, 16, 256, index_dim=100, topk_blocks=512)
    assert skv.lib().sparsekv_validate(ctypes.byref(d)) == 2


def test_host_errors_before_any_device_work(skv):
    """NULL pointers and a missing / short workspace are rejected on the host."""
    lib = skv.lib()
    d = skv.token_desc(2, 1000, 4, 24, 256, topk=64, n_sink=4, n_tail=8)
    dummy = ctypes.c_void_p(0x1000)
    # workspace missing
    st = lib.sparsekv_score(ctypes.byref(d), dummy, dummy, dummy, dummy, dummy, None, 0, None)
    assert st == 3
    # workspace too small
    st = lib.sparsekv_topk(ctypes.byref(d), dummy, dummy, dummy, dummy, ctypes.c_void_p(0x100000), 16, None)
    assert st == 3
    # NULL keys
    need = skv.workspace_size(d)
    st = lib.sparsekv_topk(ctypes.byref(d), dummy, None, dummy, dummy, ctypes.c_void_p(0x100000), need, None)
    assert st == 1
    # NULL kv view
    st = lib.sparsekv_attend(ctypes.byref(d), dummy, None, dummy, dummy, 0.1, dummy,
                             ctypes.c_void_p(0x100000), need, None)
    assert st == 1
    # qsketch is token-mode only
    db = skv.block_desc(1, 4096, 2, 16, 256, topk_blocks=64)
    st = lib.sparsekv_qsketch(ctypes.byref(db), dummy, dummy, dummy, dummy, None, 0, None)
    assert st == 1
    # misaligned workspace
    st = lib.sparsekv_topk(ctypes.byref(d), dummy, dummy, dummy, dummy, ctypes.c_void_p(0x100010), need, None)
    assert st == 3


def test_tier_rejects_bad_descriptors(skv):
    lib = skv.lib()
    layer = skv.token_desc(2, 10_000, 4, 24, 256, topk=64, n_sink=4, n_tail=8)
    h = ctypes.c_void_p()
    for ctx, slots, window, status in ((0, 200, 1, 1), (20_000, 200, 1, 1), (10_000, 64, 1, 1),
                                        (10_000, 200, 0, 1)):
        td = skv.TierDesc(ctypes.sizeof(skv.TierDesc), layer, ctx, slots, window, None)
        assert lib.sparsekv_tier_create(ctypes.byref(td), ctypes.byref(h)) == status
    l2 = skv.token_desc(2, 10_000, 2, 8, 128, topk=64, n_sink=4, n_tail=8, kv_dtype=skv.SKV_KV_F16)
    td = skv.TierDesc(ctypes.sizeof(skv.TierDesc), l2, 10_000, 200, 1, None)
    assert lib.sparsekv_tier_create(ctypes.byref(td), ctypes.byref(h)) == 2


def test_status_strings(skv):
    lib = skv.lib()
    for s in range(8):
        assert lib.sparsekv_status_str(s)
    assert lib.sparsekv_status_str(99) == b"unknown status"


def test_contraction_path_switch(skv):
    """The measurement switch takes exactly its two values (no device work)."""
    lib = skv.lib()
    assert lib.sparsekv_set_contraction_path(2) == 1
    assert lib.sparsekv_set_contraction_path(-1) == 1
    assert lib.sparsekv_set_contraction_path(skv.SKV_PATH_VALU) == 0
    assert lib.sparsekv_set_contraction_path(skv.SKV_PATH_MFMA) == 0


def test_multi_query_host_checks(skv):
    """The multi-query step takes 1..16 query tokens per sequence in token mode
    (64, 128 or 256 sketch bytes per token); its workspace holds one virtual
    sequence per query; bad arguments are rejected on the host."""
    lib = skv.lib()
    d = skv.token_desc(8, 250_000, 4, 24, 256, topk=2048, n_sink=64, n_tail=1024)
    one = skv.workspace_size(d)
    assert skv.workspace_size_multi(d, 1) == one
    w8 = skv.workspace_size_multi(d, 8)
    assert w8 > 4 * one and w8 % 256 == 0
    n = skv._lib.c_sz()
    for m in (0, 17, -1):
        assert lib.sparsekv_workspace_size_multi(ctypes.byref(d), m, ctypes.byref(n)) == 2
    db = skv.block_desc(1, 4096, 2, 16, 256, topk_blocks=64)
    assert lib.sparsekv_workspace_size_multi(ctypes.byref(db), 4, ctypes.byref(n)) == 2
    d32 = skv.token_desc(2, 4096, 1, 8, 128, rank=64, topk=64, n_sink=4, n_tail=8,
                         kv_dtype=skv.SKV_KV_F16)   # 32 sketch bytes per token
    assert lib.sparsekv_workspace_size_multi(ctypes.byref(d32), 4, ctypes.byref(n)) == 2
    dummy = ctypes.c_void_p(0x1000)
    kv = skv.KVView(dummy, dummy, dummy, dummy, 250_000)
    args = [dummy] * 7   # ctx_len, q, basis, qs, qs_scale, index_keys, index_scale
    # workspace too small (sized for one query)
    st = lib.sparsekv_step_multi(ctypes.byref(d), 8, *args, ctypes.byref(kv), dummy, dummy, 0.1,
                                 dummy, ctypes.c_void_p(0x100000), one, None)
    assert st == 3
    # NULL query
    a2 = list(args)
    a2[1] = None
    st = lib.sparsekv_step_multi(ctypes.byref(d), 8, *a2, ctypes.byref(kv), dummy, dummy, 0.1,
                                 dummy, ctypes.c_void_p(0x100000), w8, None)
    assert st == 1


def test_tier_policy_checks(skv):
    """LRU tiers need topk <= n_slots <= the LDS slot table; an unknown policy is
    rejected; a descriptor that ends before the policy field means CLOCK."""
    lib = skv.lib()
    layer = skv.token_desc(2, 10_000, 4, 24, 256, topk=64, n_sink=4, n_tail=8)
    h = ctypes.c_void_p()
    td = skv.TierDesc(ctypes.sizeof(skv.TierDesc), layer, 10_000, 63, 1, None, skv.SKV_TIER_LRU)
    assert lib.sparsekv_tier_create(ctypes.byref(td), ctypes.byref(h)) == 1
    td = skv.TierDesc(ctypes.sizeof(skv.TierDesc), layer, 10_000, 200, 1, None, 7)
    assert lib.sparsekv_tier_create(ctypes.byref(td), ctypes.byref(h)) == 1
    td = skv.TierDesc(skv.TierDesc.policy.offset, layer, 10_000, 60, 1, None, skv.SKV_TIER_LRU)
    # read as CLOCK: 60 slots do not exceed window * topk = 64
    assert lib.sparsekv_tier_create(ctypes.byref(td), ctypes.byref(h)) == 1


def test_tier_page_checks(skv):
    """Page sizes must be 0 or a power of two in [16, 4096], a pool needs a
    page size; map / unmap / attend reject a NULL tier on the host."""
    lib = skv.lib()
    layer = skv.token_desc(2, 10_000, 4, 24, 256, topk=64, n_sink=4, n_tail=8)
    h = ctypes.c_void_p()
    for P, pool in ((48, 4), (8, 4), (8192, 1), (0, 4), (64, -1)):
        td = skv.TierDesc(ctypes.sizeof(skv.TierDesc), layer, 10_000, 200, 1, None, 0, P, pool)
        assert lib.sparsekv_tier_create(ctypes.byref(td), ctypes.byref(h)) == 1, (P, pool)
        assert b"page" in lib.sparsekv_last_error() or b"pool" in lib.sparsekv_last_error()
    assert lib.sparsekv_tier_map_page(None, 0, 0, 0, None, None, None, None, None) == 1
    assert lib.sparsekv_tier_unmap_page(None, 0, 0, None) == 1
    assert lib.sparsekv_tier_attend(None, None, None, None, 1.0, None, None, 0, None) == 1
    assert lib.sparsekv_tier_host_ptr(None) is None


def test_tier_append_null_checks(skv):
    """sparsekv_tier_append rejects a NULL tier or buffer before enqueueing anything."""
    lib = skv.lib()
    dummy = ctypes.c_void_p(0x1000)
    assert lib.sparsekv_tier_append(None, dummy, dummy, dummy, dummy, dummy, dummy, None) == 1
    assert lib.sparsekv_tier_append(dummy, None, dummy, dummy, dummy, dummy, dummy, None) == 1
    assert lib.sparsekv_tier_append(dummy, dummy, dummy, dummy, None, dummy, dummy, None) == 1


def test_tier_resolve_multi_and_attend_multi_checks(skv):
    """Host-side refusals, nothing enqueued: NULL arguments, a query count
    outside [1, 16], a workspace sized for one query token."""
    lib = skv.lib()
    dummy = ctypes.c_void_p(0x1000)
    assert lib.sparsekv_tier_resolve_multi(None, 4, dummy, dummy, 0, dummy, None) == 1
    assert lib.sparsekv_tier_resolve_multi(dummy, 4, None, dummy, 0, dummy, None) == 1
    for m in (0, 17):
        assert lib.sparsekv_tier_resolve_multi(dummy, m, dummy, dummy, 0, dummy, None) == 2
    d = skv.token_desc(4, 250_000, 4, 24, 256, topk=2048, n_sink=64, n_tail=1024)
    kv = skv.KVView(dummy, dummy, dummy, dummy, 250_000)
    one = skv.workspace_size(d)
    four = skv.workspace_size_multi(d, 4)
    st = lib.sparsekv_attend_multi(ctypes.byref(d), 4, dummy, ctypes.byref(kv), dummy, dummy, 0.1,
                                   dummy, ctypes.c_void_p(0x100000), one, None)
    assert st == 3 and four > one
    st = lib.sparsekv_attend_multi(ctypes.byref(d), 4, None, ctypes.byref(kv), dummy, dummy, 0.1,
                                   dummy, ctypes.c_void_p(0x100000), four, None)
    assert st == 1
    st = lib.sparsekv_attend_multi(ctypes.byref(d), 0, dummy, ctypes.byref(kv), dummy, dummy, 0.1,
                                   dummy, ctypes.c_void_p(0x100000), four, None)
    assert st == 2


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus above 1 exits with a message (no GPU needed)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_header_is_plain_c(tmp_path):
    """include/sparsekv.h compiles as strict C99 (plain pointers and sizes, no
    C++ or HIP types in the boundary), and as C++17."""
    import shutil
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = tmp_path / "use.c"
    src.write_text('#include "sparsekv.h"\n'
                   "int main(void) { return sparsekv_abi_version() == SPARSEKV_ABI_VERSION ? 0 : 1; }\n")
    for cc, std in (("gcc", "-std=c99"), ("g++", "-std=c++17")):
        if shutil.which(cc) is None:
            pytest.skip("%s not available" % cc)
        lang = ["-x", "c++"] if cc == "g++" else []
        r = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                            *lang, "-I", os.path.join(root, "include"), str(src)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_committed_traffic_summary(tmp_path):
    """The counter summary bench.py reads its `traffic` fields from is
    self-consistent: each kernel's bytes per launch are its FETCH_SIZE and
    WRITE_SIZE averages (KiB per dispatch) scaled by the calibration copy's
    factors, as the tables of the same file give them; a source hash that
    does not match the tree yields None (no GPU needed)."""
    import importlib.util
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    text = open(bench.TRAFFIC_FILE).read()

    def avg(kernel, counter):
        vals = [float(m.group(1)) for m in re.finditer(
            r"^\| [^|]*%s[^|]* \| \d+ \| %s \| ([0-9.e+]+) \|$" % (re.escape(kernel), counter), text, re.M)]
        assert len(vals) == 1, (kernel, counter, vals)
        return vals[0]

    copy = "bitwise_not_kernel"
    f_scale = 1048576.0 / avg(copy, "FETCH_SIZE")
    w_scale = 1048576.0 / avg(copy, "WRITE_SIZE")
    for prefix, kernel in (("", "score_kernel<skv::SketchSrc<8>, true>"),
                           ("attend_", "attend_kernel<0, 256, 8, true>")):
        want = 1024 * (avg(kernel, "FETCH_SIZE") * f_scale + avg(kernel, "WRITE_SIZE") * w_scale)
        got = int(re.search(r"^%straffic_bytes_per_launch: (\d+)$" % prefix, text, re.M).group(1))
        assert abs(got - want) <= 2, (kernel, got, want)
    stale = tmp_path / "other.hip"
    stale.write_text("// not the kernel's source\n")
    assert bench.committed_traffic("attend_", [str(stale)]) is None
    assert bench.committed_traffic("", [str(stale)]) is None


def test_committed_tier_io_summary():
    """The host-tier counter summary is self-consistent: per line, the IO read
    counter per dispatch x dispatches x the calibrated bytes per count gives
    the host bytes counted, their ratio to the algorithmic host bytes is the
    ratio in the table, and that ratio is the io_ratio bench.py reads (no GPU
    needed)."""
    import importlib.util
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    text = open(bench.TIER_IO_FILE).read()
    per_count = float(re.search(r"so one\s+count = ([0-9.]+) B", text).group(1))
    num = lambda x: float(x.replace(",", ""))
    rows = re.findall(r"^\| (cfg5\w*) \| [^|]+ \| (\d+) \| ([0-9,.]+) \| ([0-9,]+) \| ([0-9,]+) \| ([0-9.]+) \|$",
                      text, re.M)
    assert {r[0] for r in rows} == {"cfg5", "cfg5r"}
    for name, disp, per, counted, alg, ratio in rows:
        assert abs(num(per) * int(disp) * per_count - num(counted)) <= 1e-5 * num(counted), name
        assert abs(num(counted) / num(alg) - float(ratio)) < 1e-4, name
        got = float(re.search(r"^io_ratio_%s: ([0-9.]+)$" % name, text, re.M).group(1))
        assert got == float(ratio), name
