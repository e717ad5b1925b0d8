"""Benchmark of the sparse-KV decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config cfg2]

A step is one layer-step: score (query sketch + sketch scan), select and
attend for the whole batch of one attention layer, through the C ABI
(sparsekv_step).  The default workload is 8 sequences x 250,000 tokens, 4 KV
heads x 24 query heads, head_dim 256, int4 rank-64 sketch, int8 K/V, keep
top-2048 + 64 sinks + 1024 tail.  Layers rotate over distinct buffers so the
scanned bytes come from HBM, not the 256 MB Infinity Cache.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import top_sparse_kv_amd as skv  # noqa: E402

METRIC = "sparse decode layer-steps/s at 250K ctx; achieved HBM GB/s vs MI355X peak"
PEAK_HBM_GBS = 8000.0
CALIB_BYTES = 1 << 30          # plain streaming kernel used to scale FETCH_SIZE / WRITE_SIZE
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_collect_cfg2_traffic.md")
SCORE_SRC = [os.path.join(ROOT, "top_sparse_kv_amd", "csrc", f) for f in ("score.hip", "keys_common.h")]
ATTEND_SRC = [os.path.join(ROOT, "top_sparse_kv_amd", "csrc", f) for f in ("attend.hip", "skv_internal.h")]


def log(*a):
    print("[bench %.1fs]" % (time.monotonic() - T0), *a, file=sys.stderr, flush=True)


T0 = time.monotonic()

CONFIGS = {
    "cfg2": dict(kind="token", B=8, T=250_000, n_kv=4, n_q=24, D=256, S=64, k=2048, L=1024,
                 kv="i8", layers=8, seed=1002, mb=2,
                 workload="8 seq x 250,000 tokens; 4 KV x 24 q heads, head_dim 256; int4 rank-64 "
                          "sketch; int8 K/V + fp16 row scales; top-2048 + 64 sinks + 1024 tail"),
    "cfg2k": dict(kind="token", B=8, T=250_000, n_kv=4, n_q=24, D=256, S=64, k=4096, L=1024, kv="i8",
                  layers=8, seed=1002, mb=2,
                  workload="8 seq x 250,000 tokens; cfg2 layer shape with the largest budget, top-4096 "
                           "+ 64 sinks + 1024 tail (5,184 rows per sequence)"),
    "cfg2kl": dict(kind="token", B=1, T=2_097_152, n_kv=4, n_q=24, D=256, S=64, k=4096, L=1024, kv="i8",
                   layers=2, seed=73,
                   workload="1 seq x 2,097,152 tokens (the largest context) with the largest budget, "
                            "top-4096 + 64 sinks + 1024 tail; cfg2 layer shape"),
    "cfg4a": dict(kind="token", B=32, T=131_072, n_kv=4, n_q=24, D=256, S=64, k=2048, L=1024,
                  kv="i8", layers=4, seed=1004, mb=2,
                  workload="32 seq x 131,072 tokens; cfg2 layer shape"),
    "cfg4b": dict(kind="token", B=32, T=250_000, n_kv=4, n_q=24, D=256, S=64, k=2048, L=1024,
                  kv="i8", layers=2, seed=1014, mixed=(2048, 250_000), mb=2,
                  workload="32 seq, lengths uniform in 2,048..250,000 (seeded); cfg2 layer shape"),
    "cfg2m": dict(kind="token", B=8, T=250_000, n_kv=4, n_q=24, D=256, S=64, k=2048, L=1024,
                  kv="i8", layers=8, seed=1002, M=8,
                  workload="8 seq x 250,000 tokens, 8 query tokens each (current + 7 drafted, "
                           "one pick per query at its causal context); cfg2 layer shape"),
    "cfg3p": dict(kind="prefill", T=1_048_576, P=4096, n_kv=2, n_q=16, D=256, k=512,
                  chunk_mib=256, seed=1003,
                  workload="prefill of 4096 tokens at a 1,048,576-token history, one QSA layer "
                           "(2 KV x 16 q heads, head_dim 256, bf16 K/V in pinned host memory); "
                           "512 picked blocks per query; 256 MiB device working buffer"),
    "cfg5l": dict(kind="tier", B=4, T=250_000, n_kv=4, n_q=24, D=256, S=64, k=2048, L=1024,
                  kv="i8", layers=1, seed=1005, warm_steps=64, steps=256, policy="lru", slots=4096,
                  workload="4 seq x 250,000 tokens; cfg2 layer shape; int4 host-RAM K/V records read "
                           "zero-copy, LRU hot buffer of 2 x top-k = 4,096 slots, drifting-locality "
                           "picks"),
    "cfg5c": dict(kind="tier", B=4, T=250_000, n_kv=4, n_q=24, D=256, S=64, k=2048, L=1024,
                  kv="i8", layers=1, seed=1005, warm_steps=64, steps=256, slots=4096,
                  workload="4 seq x 250,000 tokens; cfg2 layer shape; int4 host-RAM K/V records read "
                           "zero-copy, windowed-CLOCK hot buffer of 4,096 slots (the LRU line's "
                           "capacity), drifting-locality picks"),
    "cfg2a": dict(kind="append", B=8, T=250_000, n_kv=4, n_q=24, D=256, S=64, k=2048, L=1024,
                  kv="i8", layers=1, seed=1002,
                  workload="decode-step append for 8 seq x 250,000 tokens (cfg2 layer shape): the "
                           "new token's int8 K/V rows + scales and its int4 key sketch"),
    "cfg5a": dict(kind="tier_append", B=4, T=250_000, n_kv=4, n_q=24, D=256, S=64, k=2048, L=1024,
                  kv="i8", layers=1, seed=1005,
                  workload="decode-step append for the host tier, 4 seq x 250,000 tokens (cfg5 "
                           "shape): the new token's int4 host record written zero-copy, its int8 "
                           "rows into the tail ring, its int4 key sketch"),
    "cfg5m": dict(kind="tier", B=4, T=250_000, n_kv=4, n_q=24, D=256, S=64, k=2048, L=1024,
                  kv="i8", layers=1, seed=1005, warm_steps=64, steps=256, M=4, share=0.9,
                  workload="4 seq x 250,000 tokens, 4 query tokens each (current + 3 drafted, "
                           "90% of each draft's picks shared with the current token's); cfg2 layer "
                           "shape; int4 host-RAM K/V records read zero-copy, 2.5% hot slots "
                           "(windowed CLOCK) holding every query's rows, drifting-locality picks"),
    "cfg5": dict(kind="tier", B=4, T=250_000, n_kv=4, n_q=24, D=256, S=64, k=2048, L=1024,
                 kv="i8", layers=1, seed=1005, warm_steps=64, steps=256,
                 workload="4 seq x 250,000 tokens; cfg2 layer shape; int4 host-RAM K/V records read "
                          "zero-copy, 2.5% hot slots (windowed CLOCK), drifting-locality picks"),
    "cfg5r": dict(kind="tier", B=4, T=250_000, n_kv=4, n_q=24, D=256, S=64, k=2048, L=1024,
                  kv="i8", layers=1, seed=1005, warm_steps=64, steps=256, policy="lru", slots=4096,
                  page_tokens=64, pool_pages=1024,
                  workload="4 seq x 250,000 tokens; cfg2 layer shape; mixed residency: pages of 64 "
                           "tokens, the 1,024 most recent middle pages of each sequence's 3,907 "
                           "resident on the GPU and read in place, "
                           "the rest int4 host-RAM records read zero-copy through an LRU hot buffer "
                           "of 4,096 slots; drifting-locality picks"),
    "cfg3": dict(kind="block", B=1, T=1_048_576, n_kv=2, n_q=16, D=256, k=512, layers=12,
                 seed=1003,
                 workload="1 seq x 1,048,576 tokens; 12 QSA layers; 2 KV x 16 q heads, head_dim "
                          "256, bf16 K/V; 128-d bf16 pooled key per 4-token block; top-512 blocks"),
}


class Layer:
    """Device buffers of one layer plus the output buffers of its step."""

    def __init__(self, cfg, li):
        self.cfg = cfg
        seed = cfg["seed"] + 7919 * li
        if cfg["kind"] == "token":
            lens = None
            if "mixed" in cfg:
                lens = synth.gen.mixed_lengths(cfg["B"], cfg["mixed"][0], cfg["mixed"][1], seed=cfg["seed"])
            c = synth.make_token_case(cfg["B"], cfg["T"], lens, n_kv=cfg["n_kv"], n_q=cfg["n_q"],
                                      D=cfg["D"], S=cfg["S"], k=cfg["k"], L=cfg["L"],
                                      kv_format=cfg["kv"], seed=seed, device="cuda")
            self.desc = skv.token_desc(c.B, c.T_max, c.n_kv, c.n_q, c.D, topk=c.k, n_sink=c.S,
                                       n_tail=c.L,
                                       kv_dtype=skv.SKV_KV_I8_ROWSCALE if cfg["kv"] == "i8" else skv.SKV_KV_F16)
            self.q, self.basis = c.q, c.basis
            self.ikeys, self.iscale, self.iq = c.codes, c.sk_scale, None
            self.kv = skv.kv_view(c.k_cache, c.v_cache, c.k_scale, c.v_scale)
            self.qs = torch.zeros((c.B, c.n_kv * c.R), dtype=torch.int8, device="cuda")
            self.qsc = torch.zeros((c.B,), dtype=torch.float32, device="cuda")
            self.keys = torch.zeros((c.B, c.T_max), dtype=torch.float64, device="cuda")
        else:
            c = synth.make_block_case(cfg["B"], cfg["T"], n_kv=cfg["n_kv"], n_q=cfg["n_q"],
                                      D=cfg["D"], k=cfg["k"], seed=seed, device="cuda")
            self.desc = skv.block_desc(c.B, c.T_max, c.n_kv, c.n_q, c.D, topk_blocks=c.k)
            self.q, self.basis = c.q, None
            self.ikeys, self.iscale, self.iq = c.kp, None, c.qi
            self.kv = skv.kv_view(c.k_cache, c.v_cache)
            self.qs = self.qsc = None
            self.keys = torch.zeros((c.B, c.T_max // 4), dtype=torch.float64, device="cuda")
        self.case = c
        self.ctx = c.ctx_len
        cap = skv.select_capacity(self.desc)
        self.M = cfg.get("M", 0)
        if self.M:
            # several query tokens per sequence (sparsekv_step_multi)
            M, nq = self.M, c.n_kv * c.R
            self.mq = synth.multi_queries(c.B, M, c.n_q, c.D, seed, device="cuda")
            self.mqs = torch.zeros((c.B, M, nq), dtype=torch.int8, device="cuda")
            self.mqsc = torch.zeros((c.B, M), dtype=torch.float32, device="cuda")
            self.midx = torch.zeros((c.B, M, cap), dtype=torch.int32, device="cuda")
            self.mnsel = torch.zeros((c.B, M), dtype=torch.int32, device="cuda")
            self.mout = torch.zeros((c.B, M, c.n_q, c.D), dtype=torch.float32, device="cuda")
        self.idx = torch.zeros((c.B, cap), dtype=torch.int32, device="cuda")
        self.nsel = torch.zeros((c.B,), dtype=torch.int32, device="cuda")
        self.out = torch.zeros((c.B, c.n_q, c.D), dtype=torch.float32, device="cuda")
        self.sm = c.D ** -0.5

    def split(self, m):
        """The batch as m micro-batches of B/m sequences: per micro-batch, the
        same call on views of this layer's buffers (sequences are independent,
        so a micro-batch's results are those of its sequences in the whole
        batch).  Each micro-batch runs on its own stream with its own
        workspace."""
        c, per = self.case, self.case.B // m
        self.groups = []
        for g in range(m):
            sl = slice(g * per, (g + 1) * per)
            kv = skv.kv_view(c.k_cache[sl], c.v_cache[sl], c.k_scale[sl], c.v_scale[sl])
            if self.M:
                desc = skv.token_desc(per, c.T_max, c.n_kv, c.n_q, c.D, topk=c.k, n_sink=c.S,
                                      n_tail=c.L, kv_dtype=self.desc.kv_dtype)
                a = (desc, self.M, self.ctx[sl], self.mq[sl], self.basis, self.mqs[sl],
                     self.mqsc[sl], self.ikeys[sl], self.iscale[sl], kv, self.midx[sl],
                     self.mnsel[sl], self.sm, self.mout[sl])
                self.groups.append((skv.step_multi, a))
            else:
                desc = skv.token_desc(per, c.T_max, c.n_kv, c.n_q, c.D, topk=c.k, n_sink=c.S,
                                      n_tail=c.L, kv_dtype=self.desc.kv_dtype)
                a = (desc, self.ctx[sl], self.q[sl], self.basis, self.qs[sl], self.qsc[sl], None,
                     self.ikeys[sl], self.iscale[sl], kv, self.idx[sl], self.nsel[sl], self.sm,
                     self.out[sl])
                self.groups.append((skv.step, a))
        return self.groups

    def step_groups(self, wss, streams):
        for (fn, a), w, st in zip(self.groups, wss, streams):
            fn(*a, w, stream=st)

    def step(self, ws):
        if self.M:
            skv.step_multi(self.desc, self.M, self.ctx, self.mq, self.basis, self.mqs, self.mqsc,
                           self.ikeys, self.iscale, self.kv, self.midx, self.mnsel, self.sm,
                           self.mout, ws)
            return
        skv.step(self.desc, self.ctx, self.q, self.basis, self.qs, self.qsc, self.iq, self.ikeys,
                 self.iscale, self.kv, self.idx, self.nsel, self.sm, self.out, ws)

    def union_rows(self):
        """Distinct (sequence, row) pairs the last multi-query step attended:
        the rows a step must gather at least once."""
        n = self.mnsel.cpu().numpy()
        idx = self.midx.cpu().numpy()
        return sum(len(np.unique(np.concatenate([idx[b, j, :n[b, j]] for j in range(self.M)])))
                   for b in range(self.case.B))

    def qsketch(self, ws):
        skv.qsketch(self.desc, self.q, self.basis, self.qs, self.qsc, ws)

    def score(self, ws):
        iq = self.qs if self.iq is None else self.iq
        skv.score(self.desc, self.ctx, iq, self.ikeys, self.iscale, self.keys, ws)

    def topk(self, ws):
        skv.topk(self.desc, self.ctx, self.keys, self.idx, self.nsel, ws)

    def score_topk(self, ws):
        iq = self.qs if self.iq is None else self.iq
        skv.score_topk(self.desc, self.ctx, iq, self.ikeys, self.iscale, self.idx, self.nsel, ws)

    def attend(self, ws):
        skv.attend(self.desc, self.q, self.kv, self.idx, self.nsel, self.sm, self.out, ws)


def algorithmic_bytes(cfg, lens=None):
    """Bytes the method must move per layer-step (what each stage reads/writes
    at minimum): the scan, the gathered K/V rows (+ row scales), q, out.  With
    per-sequence lengths, a sequence at or below the dense switch reads no
    sketch and gathers all of its rows."""
    B, D, n_kv, n_q = cfg["B"], cfg["D"], cfg["n_kv"], cfg["n_q"]
    if cfg["kind"] == "token":
        lens = [cfg["T"]] * B if lens is None else [int(x) for x in lens]
        cap = cfg["S"] + cfg["k"] + cfg["L"]
        scan = sum((T - cfg["S"] - cfg["L"]) * (n_kv * 64 // 2 + 2) for T in lens if T > cap)
        eb, sb = (1, 2) if cfg["kv"] == "i8" else (2, 0)
        gather = sum(min(T, cap) for T in lens) * n_kv * (D * eb + sb) * 2
        basis = n_kv * D * 64 * 4
    else:
        scan = B * (cfg["T"] // 4) * 128 * 2
        n_sel = 4 * cfg["k"]
        gather = B * n_sel * n_kv * D * 2 * 2
        basis = 0
    qbytes = B * n_q * D * 2
    out = B * n_q * D * 4
    return dict(scan=scan, gather=gather, other=qbytes + out + basis,
                total=scan + gather + qbytes + out + basis)


def algorithmic_bytes_multi(cfg, union_rows):
    """Multi-query step: the sketch is scanned once for all queries; the K/V
    rows attended by any query of a sequence are gathered at least once."""
    B, D, n_kv, n_q, M = cfg["B"], cfg["D"], cfg["n_kv"], cfg["n_q"], cfg["M"]
    scan = B * (cfg["T"] - cfg["S"] - cfg["L"]) * (n_kv * 64 // 2 + 2)
    gather = union_rows * n_kv * (D + 2) * 2
    other = B * M * n_q * D * (2 + 4) + n_kv * D * 64 * 4
    return dict(scan=scan, gather=gather, other=other, total=scan + gather + other)


def time_loop_groups(layers, wss, streams, n):
    """n layer-steps, each as the layer's micro-batches on their streams (each
    stream runs its micro-batch's layer-steps in order); the streams fork from
    and join back to the current stream inside the timed region."""
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for s in streams:
        s.wait_event(e0)
    for i in range(n):
        layers[i % len(layers)].step_groups(wss, streams)
    for s in streams:
        st.wait_stream(s)
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / 1e3   # seconds


def time_loop(fn, layers, ws, n):
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for i in range(n):
        fn(layers[i % len(layers)], ws)
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / 1e3   # seconds


def source_hash(paths):
    """First 16 hex digits of the sha256 of the concatenated source files."""
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(prefix="", src=None):
    """HBM bytes per launch of a kernel from the committed counter summary
    (the score stream's fields, or those named with prefix), or None when
    there is none or the kernel's sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            fields = dict(ln.split(":", 1) for ln in f.read().splitlines()
                          if ln.startswith((prefix + "traffic_bytes_per_launch:",
                                            prefix + ("src_sha256_16:" if prefix else "score_src_sha256_16:"))))
    except OSError:
        return None
    key = prefix + ("src_sha256_16" if prefix else "score_src_sha256_16")
    if fields.get(key, "").strip() != source_hash(src or SCORE_SRC):
        return None
    try:
        return int(float(fields[prefix + "traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


TIER_IO_FILE = os.path.join(ROOT, "profiles", "tier_resolve_cfg5_pcie_traffic.md")
TIER_SRC = [os.path.join(ROOT, "top_sparse_kv_amd", "csrc", "tier.hip")]


def committed_io_ratio(config: str):
    """Host (PCIe) bytes the fused tier resolver reads per algorithmic host
    byte, from the committed counter summary of this line, or None when there
    is none or the kernel source changed since it was taken."""
    try:
        with open(TIER_IO_FILE) as f:
            fields = dict(ln.split(":", 1) for ln in f.read().splitlines()
                          if ln.startswith(("io_ratio_", "tier_src_sha256_16:")))
    except OSError:
        return None
    if fields.get("tier_src_sha256_16", "").strip() != source_hash(TIER_SRC):
        return None
    try:
        return float(fields["io_ratio_" + config])
    except (KeyError, ValueError):
        return None


def rocprof_summary(path, out):
    """Writes a short text summary of a rocprofv3 csv: kernel stats (average
    duration per library kernel) or counter collection (average value per
    dispatch of each counter for the library kernels and the copy used for
    calibration)."""
    import collections
    import csv
    lines = []
    if path.endswith("kernel_trace.csv"):
        # per kernel and grid shape (a micro-batch's launches have their own
        # grid), from the individual dispatches
        groups = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            nm = r["Kernel_Name"]
            if "skv" not in nm:
                continue
            nm = nm.replace("(anonymous namespace)::", "").split("(")[0]
            gx = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
            gy = int(r["Grid_Size_Y"]) // max(1, int(r["Workgroup_Size_Y"]))
            groups[(nm, "%d x %d" % (gx, gy))].append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines.append("| kernel | workgroups | calls | avg us | min us | max us |")
        lines.append("|---|---|---|---|---|---|")
        for (nm, grid), ts in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            lines.append("| %s | %s | %d | %.2f | %.2f | %.2f |" % (
                nm, grid, len(ts), sum(ts) / len(ts), min(ts), max(ts)))
    elif path.endswith("kernel_stats.csv"):
        lines.append("| kernel | calls | avg us | min us | max us |")
        lines.append("|---|---|---|---|---|")
        for r in csv.DictReader(open(path)):
            if "skv" in r["Name"]:
                nm = r["Name"].replace("(anonymous namespace)::", "").split("(")[0]
                lines.append("| %s | %s | %.2f | %.2f | %.2f |" % (
                    nm, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                    float(r["MaxNs"]) / 1e3))
    else:
        agg = collections.defaultdict(lambda: collections.defaultdict(float))
        disp = collections.defaultdict(set)
        for r in csv.DictReader(open(path)):
            nm = r.get("Kernel_Name", "")
            if "skv" not in nm and "bitwise_not" not in nm:
                continue
            key = nm.replace("(anonymous namespace)::", "").split("(")[0][-70:]
            agg[key][r["Counter_Name"]] += float(r["Counter_Value"])
            disp[key].add(r.get("Dispatch_Id", ""))
        lines.append("| kernel | dispatches | counter | average per dispatch |")
        lines.append("|---|---|---|---|")
        for key, cs in agg.items():
            n = max(1, len(disp[key]))
            for c, v in sorted(cs.items()):
                lines.append("| %s | %d | %s | %.6g |" % (key, n, c, v / n))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores() -> int:
    """CPUs this process may run on (the box's share), capped at 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def read_ceiling(buf: torch.Tensor, nbytes: int, reps: int = 20):
    """The library's plain streaming read (sparsekv_read_bytes) over nbytes of
    a device buffer, best of a few grid sizes: the rate a kernel that only
    reads those bytes reaches on this GPU, each launch timed by its own
    events."""
    nb = min(nbytes, buf.numel() * buf.element_size()) // 16 * 16
    best = None
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    for n_wg in (2048, 4096, 8192):
        for _ in range(3):
            skv.read_bytes(buf.data_ptr(), nb, sink, n_wg)
        skv.timer_enable(True)
        for _ in range(reps):
            skv.read_bytes(buf.data_ptr(), nb, sink, n_wg)
        ms, n = skv.timer_read()
        skv.timer_enable(False)
        us = ms * 1e3 / max(1, n)
        if best is None or us < best["avg_launch_us"]:
            best = {"bytes": nb, "n_wg": n_wg, "avg_launch_us": round(us, 2),
                    "GBps": round(nb / us / 1e3, 1), "frac": round(nb / us / 1e3 / PEAK_HBM_GBS, 4),
                    "launches_timed": n}
    return best


def _hip_runtime():
    """The HIP runtime library this process already uses (torch loaded it)."""
    import ctypes
    with open("/proc/self/maps") as f:
        for ln in f:
            path = ln.split()[-1]
            if "libamdhip64.so" in path and os.path.exists(path):
                return ctypes.CDLL(path)
    return None


def zero_copy_read(mib: int, reps: int = 20):
    """The library's plain streaming read over `mib` MiB of pinned, device-mapped
    host memory (hipHostMalloc, its device address from
    hipHostGetDevicePointer): the rate a kernel that only reads host memory
    reaches over this GPU's link; also the known-size read the IO counters are
    calibrated on."""
    import ctypes
    hip = _hip_runtime()
    if hip is None:
        return None
    nb = mib << 20
    hptr, dptr = ctypes.c_void_p(), ctypes.c_void_p()
    if hip.hipHostMalloc(ctypes.byref(hptr), ctypes.c_size_t(nb), ctypes.c_uint(0x1 | 0x2)) != 0:
        return None
    try:
        ctypes.memset(hptr, 1, nb)
        if hip.hipHostGetDevicePointer(ctypes.byref(dptr), hptr, ctypes.c_uint(0)) != 0 or not dptr.value:
            return None
        sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
        for _ in range(3):
            skv.read_bytes(dptr.value, nb, sink, 1024)
        skv.timer_enable(True)
        for _ in range(reps):
            skv.read_bytes(dptr.value, nb, sink, 1024)
        ms, n = skv.timer_read()
        skv.timer_enable(False)
        torch.cuda.synchronize()
        us = ms * 1e3 / max(1, n)
        return {"bytes": nb, "n_wg": 1024, "avg_launch_us": round(us, 2), "GBps": round(nb / us / 1e3, 2),
                "launches_timed": n}
    finally:
        torch.cuda.synchronize()
        hip.hipHostFree(hptr)


def _oracle_seq_worker(a):
    """One process of the all-core oracle run: `reps` layer-steps of one
    sequence (query sketch, exact keys, selection, attention over its gathered
    rows), inputs memory-mapped from files the parent wrote."""
    d, b, T, S, k, L, group, sm, reps = a
    import oracle
    from threadpoolctl import threadpool_limits
    ld = lambda name: np.load(os.path.join(d, "%s_%d.npy" % (name, b)), mmap_mode="r")
    q, codes, sks = ld("q"), ld("codes"), ld("sks")
    basis = np.load(os.path.join(d, "basis.npy"))
    kr, vr, ks, vs = ld("kr"), ld("vr"), ld("ks"), ld("vs")
    with threadpool_limits(limits=1):
        t = time.perf_counter()
        for _ in range(reps):
            qs, _ = oracle.query_sketch(q, basis, group)
            keys = oracle.sketch_keys(qs, codes, sks, [T], S, k, L)
            sel = oracle.select_tokens(keys[0], T, S, k, L)
            oracle.sparse_attention(q[0], kr, vr, ks, vs, np.arange(sel.size), sm, group, "i8")
        return time.perf_counter() - t


def cpu_baseline_all_cores(layer: Layer, cfg, seq_step_s: float, min_seconds=10.0):
    """The same oracle layer-step with its sequences spread over the host's
    cores (one process per sequence, each limited to one BLAS thread); inputs
    are written once to memory-mapped files, outside the timed region."""
    import multiprocessing as mp
    import shutil
    import tempfile
    import oracle
    c = layer.case
    n = min(c.B, host_cores())
    if n < 2 or cfg.get("M") or cfg["kind"] != "token":
        return None
    d = tempfile.mkdtemp(prefix="skv_oracle_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        q = c.q.cpu().numpy()
        basis = c.basis.cpu().numpy()
        np.save(os.path.join(d, "basis.npy"), basis)
        qs, _ = oracle.query_sketch(q, basis, c.group)
        keys = oracle.sketch_keys(qs, c.codes.cpu().numpy(), c.sk_scale.cpu().numpy(), c.lens, c.S, c.k, c.L)
        for b in range(c.B):
            sel = oracle.select_tokens(keys[b], c.lens[b], c.S, c.k, c.L)
            ii = torch.from_numpy(sel).cuda()
            for name, t in (("kr", c.k_cache), ("vr", c.v_cache), ("ks", c.k_scale), ("vs", c.v_scale)):
                np.save(os.path.join(d, "%s_%d.npy" % (name, b)), t[b].index_select(0, ii).cpu().numpy())
            np.save(os.path.join(d, "q_%d.npy" % b), q[b:b + 1])
            np.save(os.path.join(d, "codes_%d.npy" % b), c.codes[b:b + 1].cpu().numpy())
            np.save(os.path.join(d, "sks_%d.npy" % b), c.sk_scale[b:b + 1].cpu().numpy())
        # repetitions so that the parallel run takes about min_seconds
        reps = max(1, int(min_seconds / max(1e-3, seq_step_s * c.B / n)))
        reps = min(reps, 200)
        args = [(d, b, c.lens[b], c.S, c.k, c.L, c.group, layer.sm, reps) for b in range(c.B)]
        with mp.get_context("spawn").Pool(n) as pool:
            pool.map(_oracle_seq_worker, [(d, b, c.lens[b], c.S, c.k, c.L, c.group, layer.sm, 1)
                                          for b in range(n)])   # start-up outside the timing
            t = time.perf_counter()
            pool.map(_oracle_seq_worker, args, chunksize=1)
            wall = time.perf_counter() - t
        return dict(value=reps / wall, unit="layer-steps/s", cores=n, kind="oracle",
                    sample="%d repetitions of one full layer-step of layer 0 (%d sequences x %d tokens), "
                           "one process per sequence on %d cores" % (reps, c.B, c.T_max, n),
                    seconds=wall)
    finally:
        shutil.rmtree(d, ignore_errors=True)


def cpu_baseline(layer: Layer, cfg):
    """The CPU oracle timed on one host core (BLAS pools limited to one thread)
    on one full layer-step of layer 0 (all sequences of the batch): query
    sketch, exact keys, selection and attention.  Data movement to the host is
    not timed."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        return _cpu_baseline(layer, cfg)


def _cpu_baseline(layer: Layer, cfg, min_seconds=10.0, max_reps=500):
    """Repeats the oracle's layer-step until about min_seconds of timed CPU
    work have accumulated; the gathered K/V rows are moved to the host once,
    outside the timed sections."""
    import oracle
    c = layer.case
    t_total, reps, rows = 0.0, 0, None
    if cfg.get("M"):
        # one sequence (of the batch) x M query tokens per repetition
        M, b = cfg["M"], 0
        host = [x[b:b + 1].cpu().numpy() for x in (c.codes, c.sk_scale, c.k_cache, c.v_cache,
                                                     c.k_scale, c.v_scale)]
        qm = layer.mq[b:b + 1].cpu().numpy()
        basis = c.basis.cpu().numpy()
        while reps < max_reps and (reps == 0 or t_total < min_seconds):
            t = time.perf_counter()
            oracle.multiquery.token_step_multi(qm, basis, *host, [c.lens[b]], M=M, S=c.S,
                                               k_top=c.k, L=c.L, group=c.group, sm_scale=layer.sm,
                                               fmt="i8")
            t_total += time.perf_counter() - t
            reps += 1
        return dict(value=reps / t_total / c.B, unit="layer-steps/s", cores=1, kind="oracle",
                    sample="%d repetitions of sequence 0 of layer 0 (%d query tokens x %d tokens); "
                           "value scaled to the %d-sequence batch" % (reps, M, c.T_max, c.B),
                    seconds=t_total)
    if cfg["kind"] == "token":
        q = c.q.cpu().numpy()
        basis = c.basis.cpu().numpy()
        codes = c.codes.cpu().numpy()
        sks = c.sk_scale.cpu().numpy()
        while reps < max_reps and (reps == 0 or t_total < min_seconds):
            t = time.perf_counter()
            qs, _ = oracle.query_sketch(q, basis, c.group)
            keys = oracle.sketch_keys(qs, codes, sks, c.lens, c.S, c.k, c.L)
            sels = [oracle.select_tokens(keys[b], c.lens[b], c.S, c.k, c.L) for b in range(c.B)]
            t_total += time.perf_counter() - t
            if rows is None:
                rows = []
                for b in range(c.B):
                    ii = torch.from_numpy(sels[b]).cuda()
                    rows.append([x[b].index_select(0, ii).cpu().numpy()
                                 for x in (c.k_cache, c.v_cache, c.k_scale, c.v_scale)])
            t = time.perf_counter()
            for b in range(c.B):
                kr, vr, ks, vs = rows[b]
                oracle.sparse_attention(q[b], kr, vr, ks, vs, np.arange(sels[b].size), layer.sm,
                                        c.group, "i8")
            t_total += time.perf_counter() - t
            reps += 1
        sample = "%d repetitions of one full layer-step of layer 0: %d sequences x %d tokens" % (
            reps, c.B, c.T_max)
    else:
        def bits(x):
            return x.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        qi, kp, q = bits(c.qi), bits(c.kp), bits(c.q)
        while reps < max_reps and (reps == 0 or t_total < min_seconds):
            t = time.perf_counter()
            keys = oracle.pooled_keys(qi, kp, c.lens)
            sel = oracle.select_blocks(keys[0], c.lens[0], c.k)
            t_total += time.perf_counter() - t
            if rows is None:
                ii = torch.from_numpy(sel).cuda()
                rows = (bits(c.k_cache[0].index_select(0, ii)), bits(c.v_cache[0].index_select(0, ii)))
            t = time.perf_counter()
            oracle.sparse_attention(q[0], rows[0], rows[1], None, None, np.arange(sel.size), layer.sm,
                                    c.group, "bf16")
            t_total += time.perf_counter() - t
            reps += 1
        sample = "%d repetitions of one full layer-step of layer 0 (1 sequence x %d tokens)" % (
            reps, c.T_max)
    return dict(value=reps / t_total, unit="layer-steps/s", cores=1, kind="oracle", sample=sample,
                seconds=t_total)


PCIE5_X16_GBS = 64.0   # PCIe 5.0 x16, one direction (nominal)


def bench_append(cfg, args):
    """The decode-step append alone: every sequence's new token written at
    ctx_len - 2000 (inside the cache), timed by the kernel's own dispatches."""
    L0 = Layer(dict(cfg, kind="token"), 0)
    c0 = L0.case
    ws = skv.workspace(L0.desc)
    g = torch.Generator(device="cuda").manual_seed(7)
    k_new = torch.randn((c0.B, c0.n_kv, c0.D), generator=g, device="cuda").to(torch.float16)
    v_new = torch.randn((c0.B, c0.n_kv, c0.D), generator=g, device="cuda").to(torch.float16)
    ctx_a = (L0.ctx - 2000).clamp(min=0).to(torch.int32).contiguous()

    def call(layer, ws_):
        skv.append(layer.desc, ctx_a, k_new, v_new, layer.basis, layer.kv, layer.ikeys,
                   layer.iscale, ws_)
    for _ in range(max(5, args.warmup)):
        call(L0, ws)
    secs = time_loop(call, [L0], ws, args.steps)
    skv.timer_enable(True)
    time_loop(call, [L0], ws, args.steps)
    a_ms, a_n = skv.timer_read()
    skv.timer_enable(False)
    skv.check(ws)
    B, H, D = c0.B, c0.n_kv, c0.D
    # what one call must move: the new rows (fp16) and the basis in; int8 rows,
    # row scales, sketch codes and scale out; ctx_len in and out
    alg = B * H * D * 2 * 2 + H * D * 64 * 4 + B * (H * D * 2 + H * 2 * 2 + H * 32 + 2) + B * 8
    a_s = a_ms / 1e3 / max(1, a_n)
    res = {
        "metric": METRIC + " (append: calls/s)", "value": round(args.steps / secs, 2),
        "unit": "appends/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1e3 * secs / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": cfg["workload"], "name": args.config, "batch": B, "ctx": cfg["T"]},
        "roofline": {"kernel": "append", "bound": "hbm", "achieved": round(alg / a_s / 1e9, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(alg / a_s / 1e9 / PEAK_HBM_GBS, 5), "traffic": None,
                     "bytes_per_launch": alg, "avg_launch_us": round(a_s * 1e6, 2),
                     "launches_timed": a_n,
                     "note": "one workgroup per sequence: launch- and latency-bound"},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        import oracle
        from threadpoolctl import threadpool_limits
        caches = {"codes": c0.codes[:, -2100:].cpu().numpy().copy(),
                  "sk_scale": c0.sk_scale[:, -2100:].cpu().numpy().copy(),
                  "k": c0.k_cache[:, -2100:].cpu().numpy().copy(),
                  "v": c0.v_cache[:, -2100:].cpu().numpy().copy(),
                  "k_scale": c0.k_scale[:, -2100:].cpu().numpy().copy(),
                  "v_scale": c0.v_scale[:, -2100:].cpu().numpy().copy()}
        kn, vn, basis = k_new.cpu().numpy(), v_new.cpu().numpy(), c0.basis.cpu().numpy()
        ctx0 = np.full(B, 100, dtype=np.int32)   # rows inside the host copy of the last 2100 rows
        t_total, reps = 0.0, 0
        with threadpool_limits(limits=1):
            while reps < 5000 and (reps == 0 or t_total < 10.0):
                t0 = time.perf_counter()
                oracle.append.append_tokens(ctx0, kn, vn, basis, caches, 2100)
                t_total += time.perf_counter() - t0
                reps += 1
        res["cpu_baseline"] = {"value": round(reps / t_total, 3), "unit": "appends/s", "cores": 1,
                               "kind": "oracle",
                               "sample": "%d appends of all %d sequences into a host copy of the "
                                         "caches' last rows" % (reps, B),
                               "seconds": round(t_total, 3)}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def bench_tier_append(cfg, args):
    """The decode-step append of the host tier alone: every sequence's new
    token goes into its host record (zero-copy), the tail ring and the key
    sketch; timed by the kernel's own dispatches and by the host clock."""
    B, T, H, D, S, L, k = cfg["B"], cfg["T"], cfg["n_kv"], cfg["D"], cfg["S"], cfg["k"], cfg["L"]
    R = 64
    n_calls = max(5, args.warmup) + 2 * args.steps
    cap = T + n_calls
    log("generating the host-tier case")
    c = synth.make_tier_case(B, T, n_kv=H, n_q=cfg["n_q"], D=D, S=S, k=k, L=L, seed=cfg["seed"],
                             device="cuda")
    desc = skv.token_desc(B, cap, H, cfg["n_q"], D, topk=k, n_sink=S, n_tail=L)
    tier = skv.Tier(desc, T, c.n_slots, 1)
    try:
        tier.host_records()[:, :T] = c.records.cpu().numpy()
        tier.load_resident(c.res_k, c.res_v, c.res_ks, c.res_vs)
        basis = synth.orthonormal_basis(H, D, R, cfg["seed"]).cuda()
        codes = torch.zeros((B, cap, H * R // 2), dtype=torch.uint8, device="cuda")
        sksc = torch.zeros((B, cap), dtype=torch.float16, device="cuda")
        ctx = torch.full((B,), T, dtype=torch.int32, device="cuda")
        g = torch.Generator(device="cuda").manual_seed(7)
        k_new = torch.randn((B, H, D), generator=g, device="cuda").to(torch.float16)
        v_new = torch.randn((B, H, D), generator=g, device="cuda").to(torch.float16)

        def call(_layer, _ws):
            tier.append(ctx, k_new, v_new, basis, codes, sksc)
        for _ in range(max(5, args.warmup)):
            call(None, None)
        secs = time_loop(call, [None], None, args.steps)
        skv.timer_enable(True)
        time_loop(call, [None], None, args.steps)
        a_ms, a_n = skv.timer_read()
        skv.timer_enable(False)
        tier.stats()                              # raises on any tier flag
        assert int(ctx[0].item()) == T + n_calls
    finally:
        tier.close()
    rec = 2 * (D // 2 + 2 * (D // 64))
    host_bytes = B * H * rec
    # what one call must move: the new rows (fp16) and the basis in; int8 rows,
    # row scales, sketch codes and scale to the GPU, the records to host memory
    dev_bytes = B * H * D * 2 * 2 + H * D * R * 4 + B * (H * D * 2 + H * 2 * 2 + H * R // 2 + 2) + B * 8
    a_s = a_ms / 1e3 / max(1, a_n)
    res = {
        "metric": METRIC + " (tier append: calls/s)", "value": round(args.steps / secs, 2),
        "unit": "appends/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1e3 * secs / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": cfg["workload"], "name": args.config, "batch": B, "ctx": T},
        "roofline": {"kernel": "tier_append", "bound": "hbm",
                     "achieved": round((dev_bytes + host_bytes) / a_s / 1e9, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round((dev_bytes + host_bytes) / a_s / 1e9 / PEAK_HBM_GBS, 5),
                     "traffic": None, "bytes_per_launch": dev_bytes + host_bytes,
                     "host_bytes_per_launch": host_bytes, "avg_launch_us": round(a_s * 1e6, 2),
                     "launches_timed": a_n,
                     "note": "one workgroup per sequence: launch- and latency-bound"},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        import oracle
        from threadpoolctl import threadpool_limits
        rb = rec
        rec_np = np.zeros((B, 64, H, rb), dtype=np.uint8)          # the rows an append writes
        rk, rv = c.res_k.cpu().numpy(), c.res_v.cpu().numpy()
        rks, rvs = c.res_ks.cpu().numpy(), c.res_vs.cpu().numpy()
        kn, vn, bas = k_new.cpu().numpy(), v_new.cpu().numpy(), basis.cpu().numpy()
        t_total, reps = 0.0, 0
        with threadpool_limits(limits=1):
            while reps < 5000 and (reps == 0 or t_total < 10.0):
                t0 = time.perf_counter()
                for b in range(B):
                    oracle.append.key_sketch(kn[b], bas)
                    oracle.append.tier_append_token(reps % 64, rec_np[b], rk[b], rv[b], rks[b],
                                                    rvs[b], S, L, kn[b], vn[b])
                t_total += time.perf_counter() - t0
                reps += 1
        res["cpu_baseline"] = {"value": round(reps / t_total, 3), "unit": "appends/s", "cores": 1,
                               "kind": "oracle",
                               "sample": "%d appends of all %d sequences (record, tail, sketch) "
                                         "into host copies" % (reps, B),
                               "seconds": round(t_total, 3)}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def bench_prefill(cfg, args):
    """Prefill attention over host-resident K/V: one call streams the history
    once through the working buffer and attends every prefill query's picks
    (seeded uniform block picks stand in for the indexer's selection)."""
    T, P, n_kv, n_q, D, kb = cfg["T"], cfg["P"], cfg["n_kv"], cfg["n_q"], cfg["D"], cfg["k"]
    log("generating %d x %d x %d bf16 K and V in pinned host memory" % (T, n_kv, D))
    host = []
    for tid in (1, 2):
        t = torch.empty((T, n_kv, D), dtype=torch.bfloat16, pin_memory=True)
        g = torch.Generator(device="cuda").manual_seed(cfg["seed"] * 10 + tid)
        step = 1 << 18
        for a in range(0, T, step):
            t[a:a + step].copy_(torch.randn((min(step, T - a), n_kv, D), generator=g, device="cuda")
                                .to(torch.bfloat16))
        host.append(t)
    g = torch.Generator(device="cuda").manual_seed(cfg["seed"] * 10 + 3)
    q = torch.randn((P, n_q, D), generator=g, device="cuda").to(torch.bfloat16)
    idx_np, nsel_np = synth.prefill_picks(P, T, kb, cfg["seed"])
    idx, nsel = torch.from_numpy(idx_np).cuda(), torch.from_numpy(nsel_np).cuda()
    desc = skv.block_desc(1, T, n_kv, n_q, D, topk_blocks=kb)
    chunk_mib = args.chunk_mib or cfg["chunk_mib"]
    buf = torch.empty((chunk_mib << 20,), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((skv.prefill_workspace_size(desc, P),), dtype=torch.uint8, device="cuda")
    out = torch.zeros((P, n_q, D), dtype=torch.float32, device="cuda")
    sm = D ** -0.5

    def call():
        skv.prefill_attend(desc, q, idx, nsel, host[0], host[1], buf, sm, out, ws)

    for _ in range(max(1, args.warmup)):
        call()
    skv.check(ws)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(args.steps):
        call()
    e1.record(st)
    e1.synchronize()
    secs = e0.elapsed_time(e1) / 1e3
    skv.check(ws)
    # a plain pinned host-to-device copy of the same bytes, for reference
    dev = torch.empty((T, n_kv, D), dtype=torch.bfloat16, device="cuda")
    for _ in range(2):
        dev.copy_(host[0], non_blocking=True)
        dev.copy_(host[1], non_blocking=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(3):
        dev.copy_(host[0], non_blocking=True)
        dev.copy_(host[1], non_blocking=True)
    e1.record(st)
    e1.synchronize()
    copy_s = e0.elapsed_time(e1) / 1e3 / 3
    host_bytes = 2 * T * n_kv * D * 2
    per = secs / args.steps
    naive = int(nsel_np.astype(np.int64).sum()) * n_kv * D * 2 * 2
    res = {
        "metric": METRIC + " (prefill: layer-chunks/s)",
        "value": round(1.0 / per, 3),
        "unit": "layer-chunks/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(per * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg["workload"], "name": args.config, "history": T,
                   "prefill_tokens": P, "buffer_mib": chunk_mib},
        "prefill_tokens_per_s": round(P / per, 1),
        "host_bytes_per_call": host_bytes,
        "per_token_fetch_bytes": naive,
        "roofline": {"kernel": "prefill (host-to-device chunk copies)", "bound": "pcie",
                     "achieved": round(host_bytes / per / 1e9, 2), "peak": PCIE5_X16_GBS,
                     "unit": "GB/s", "frac": round(host_bytes / per / 1e9 / PCIE5_X16_GBS, 4),
                     "traffic": None, "plain_copy_GBps": round(host_bytes / copy_s / 1e9, 2)},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        import oracle
        from threadpoolctl import threadpool_limits
        kk, vv = (h.view(torch.int16).numpy().view(np.uint16) for h in host)
        qq = q.cpu().view(torch.int16).numpy().view(np.uint16)
        t_total, reps, n = 0.0, 0, 64
        with threadpool_limits(limits=1):
            while reps < 20 and (reps == 0 or t_total < 10.0):
                qs = list(range((reps * n) % P, (reps * n) % P + n))
                lists = [idx_np[p, :nsel_np[p]].astype(np.int64) for p in qs]
                t0 = time.perf_counter()
                oracle.prefill.prefill_attention(qq[qs], kk, vv, lists, sm, n_q // n_kv, "bf16")
                t_total += time.perf_counter() - t0
                reps += 1
        res["cpu_baseline"] = {"value": round(reps * n / t_total / P, 5), "unit": "layer-chunks/s",
                               "cores": 1, "kind": "oracle",
                               "sample": "%d batches of %d of the %d prefill queries (rows read from "
                                         "host memory); value scaled to all %d" % (reps, n, P, P),
                               "seconds": round(t_total, 3)}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def bench_tier(cfg, args):
    """Host-tier layer-step: the hot-buffer resolve (hits, windowed-CLOCK
    victims, zero-copy int4 fetch and dequantisation of the misses) followed by
    attention over the resolved rows, with picks from the seeded
    drifting-locality schedule in place of the indexer's selection."""
    B, T, S, L, k = cfg["B"], cfg["T"], cfg["S"], cfg["L"], cfg["k"]
    warm = args.warmup if args.warmup_given else cfg["warm_steps"]
    steps = args.steps if args.steps_given else cfg["steps"]
    M = cfg.get("M", 1)
    log("generating the host-tier case")
    c = synth.make_tier_case(B, T, n_kv=cfg["n_kv"], n_q=cfg["n_q"], D=cfg["D"], S=S, k=k, L=L,
                             seed=cfg["seed"], device="cuda")
    # M query tokens: the last M positions; picks below the first one's middle end
    T1 = T - M + 1
    picks = synth.drift_picks(B, T1, S, L, k, warm + steps, seed=cfg["seed"],
                              window=min(65536, (T1 - S - L) // 2), sigma_c=256.0)
    mpicks = synth.draft_picks(picks, M, cfg["share"], cfg["seed"]) if M > 1 else picks[:, :, None]
    desc = skv.token_desc(B, T, cfg["n_kv"], cfg["n_q"], cfg["D"], topk=k, n_sink=S, n_tail=L)
    n_slots = cfg.get("slots", c.n_slots)
    lru = cfg.get("policy") == "lru"
    P, pool = cfg.get("page_tokens", 0), cfg.get("pool_pages", 0)
    tier = skv.Tier(desc, T, n_slots, 1, policy=skv.SKV_TIER_LRU if lru else skv.SKV_TIER_CLOCK,
                    page_tokens=P, pool_pages=pool)
    mapped = []
    try:
        tier.host_records()[:] = c.records.cpu().numpy()
        tier.load_resident(c.res_k, c.res_v, c.res_ks, c.res_vs)
        res = tier.resident()
        if pool:
            # mixed residency: the most recent middle pages of every sequence
            # stay on the GPU (their int8 rows copied into the pool), the rest
            # are placeholders read through the hot buffer
            last = (T - L) // P - 1
            mapped = list(range(last - pool + 1, last + 1))
            log("mapping %d pages per sequence" % len(mapped))
            for b in range(B):
                for j0 in range(0, len(mapped), 128):
                    part = mapped[j0:j0 + 128]
                    rk, rks, rv, rvs = synth.tier_page_rows(B, T, n_kv=cfg["n_kv"], D=cfg["D"], seed=cfg["seed"],
                                                            page_tokens=P, pages=[(b, g) for g in part],
                                                            device="cuda")
                    for j, g in enumerate(part):
                        tier.map_page(b, g, j0 + j, rk[j], rv[j], rks[j], rvs[j])
                    torch.cuda.synchronize()
        cap = skv.select_capacity(desc)
        nst = warm + steps
        if M == 1:
            idx_all = torch.from_numpy(np.concatenate([
                np.broadcast_to(np.arange(S, dtype=np.int32), (nst, B, S)), picks,
                np.broadcast_to(np.arange(T - L, T, dtype=np.int32), (nst, B, L))], axis=2).copy()).cuda()
            ws = skv.workspace(desc)
            rows = torch.zeros((B, cap), dtype=torch.int32, device="cuda")
            nsel = torch.full((B,), cap, dtype=torch.int32, device="cuda")
            out = torch.zeros((B, cfg["n_q"], cfg["D"]), dtype=torch.float32, device="cuda")
            q = c.q.contiguous()
        else:
            tails = np.stack([np.arange(T1 + j - L, T1 + j, dtype=np.int32) for j in range(M)])
            idx_all = torch.from_numpy(np.concatenate([
                np.broadcast_to(np.arange(S, dtype=np.int32), (nst, B, M, S)), mpicks,
                np.broadcast_to(tails, (nst, B, M, L))], axis=3).copy()).cuda()
            ws = skv.workspace_multi(desc, M)
            rows = torch.zeros((B, M, cap), dtype=torch.int32, device="cuda")
            nsel = torch.full((B, M), cap, dtype=torch.int32, device="cuda")
            out = torch.zeros((B, M, cfg["n_q"], cfg["D"]), dtype=torch.float32, device="cuda")
            q = synth.multi_queries(B, M, cfg["n_q"], cfg["D"], cfg["seed"], device="cuda")
        sm = cfg["D"] ** -0.5

        def resolve(s_):
            if M == 1:
                tier.resolve(idx_all[s_], nsel, s_, rows)
            else:
                tier.resolve_multi(M, idx_all[s_], nsel, s_, rows)

        def attend():
            if M == 1:
                tier.attend(q, rows, nsel, sm, out, ws)
            else:
                skv.attend_multi(desc, M, q, res, rows, nsel, sm, out, ws)
        log("warmup", warm)
        for s_ in range(warm):
            resolve(s_)
            attend()
        st0 = tier.stats()
        log("timing %d layer-steps" % steps)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s_ in range(warm, warm + steps):
            resolve(s_)
            attend()
        e1.record()
        e1.synchronize()
        secs = e0.elapsed_time(e1) / 1e3
        st1 = tier.stats()
        # host bytes of every resolver dispatch in this process (the counter
        # pass over this command sees all of them)
        all_bytes, all_calls = st1.host_bytes, st1.steps
        # the resolve alone, on a replay of the same picks from a reset buffer
        tier.reset()
        for s_ in range(warm):
            resolve(s_)
        torch.cuda.synchronize()
        e0.record()
        for s_ in range(warm, warm + steps):
            resolve(s_)
        e1.record()
        e1.synchronize()
        rsecs = e0.elapsed_time(e1) / 1e3
        st2 = tier.stats()
        all_bytes += st2.host_bytes
        all_calls += st2.steps
        # the fused resolver (resolve + zero-copy fetch), timed by its own
        # dispatches (a third replay of the same picks: the same misses)
        tier.reset()
        for s_ in range(warm):
            resolve(s_)
        skv.timer_enable(True)
        for s_ in range(warm, warm + steps):
            resolve(s_)
        f_ms, f_n = skv.timer_read()
        skv.timer_enable(False)
        st3 = tier.stats()
        all_bytes += st3.host_bytes
        all_calls += st3.steps
        assert skv.check(ws) == 0
        zc = zero_copy_read(64)
        cpu = None
        if not args.no_cpu_baseline:
            log("cpu baseline (oracle)")
            cpu = _tier_cpu_baseline(cfg, c, mpicks, warm, tier.host_records()[0], lru, n_slots,
                                     q[0].cpu().numpy() if M > 1 else None, pages=mapped)
            cpu["cpu_model"] = cpu_model()
    finally:
        tier.close()
    hits, misses = st1.hits - st0.hits, st1.misses - st0.misses
    in_place = st1.in_place - st0.in_place
    hbytes = st1.host_bytes - st0.host_bytes
    res_line = {
        "metric": METRIC,
        "value": round(steps / secs, 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(1e3 * secs / steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": dict({"workload": cfg["workload"], "name": args.config, "batch": B, "ctx": T,
                        "hot_slots_per_seq": n_slots, "policy": "lru" if lru else "windowed-clock"},
                       **({"page_tokens": P, "resident_pages_per_seq": pool} if pool else {}),
                       **({"query_tokens_per_seq": M} if M > 1 else {})),
        "tier": {"miss_rate": round(misses / max(1, hits + misses), 4), "hits": hits, "misses": misses,
                 "in_place": in_place,
                 "host_bytes_per_step": round(hbytes / steps),
                 "pcie_GBps_over_step": round(hbytes / secs / 1e9, 2),
                 "resolve_us": round(rsecs / steps * 1e6, 2),
                 "pcie_GBps_during_resolve": round(hbytes / rsecs / 1e9, 2),
                 "pcie_peak_GBps": 64.0,
                 "zero_copy_read": zc,
                 "host_bytes_all_resolves": int(all_bytes), "resolve_calls": int(all_calls)},
        "roofline": None,
        "cpu_baseline": cpu,
    }
    if M > 1:
        res_line["query_tokens_per_s"] = round(steps / secs * B * M, 1)
    if f_n:
        f_s = f_ms / 1e3 / f_n
        per = hbytes / steps
        io = committed_io_ratio(args.config)
        res_line["roofline"] = {"kernel": "tier_resolve (resolve + zero-copy fetch, one kernel)", "bound": "pcie",
                                "achieved": round(per / f_s / 1e9, 2), "peak": PCIE5_X16_GBS,
                                "unit": "GB/s", "frac": round(per / f_s / 1e9 / PCIE5_X16_GBS, 4),
                                "traffic": round(io * per) if io else None, "bytes_per_launch": round(per),
                                "avg_launch_us": round(f_s * 1e6, 2), "launches_timed": f_n}
    print(json.dumps(res_line), flush=True)


def _tier_cpu_baseline(cfg, c, lists, warm, records_b, lru, n_slots, qm=None, min_seconds=10.0,
                       pages=()):
    """The oracle's host-tier layer-step on sequence 0 (hot-buffer resolve with
    its policy, then attention over the resident rows and the fetched host
    records; with several query tokens each query's list and attention),
    after the same warm-up; scaled to the whole batch.  lists: middle picks
    [n_steps][B][M][k]; qm: fp16 [M][H_q][D] queries of sequence 0 (M > 1)."""
    import oracle
    from threadpoolctl import threadpool_limits
    B, T, S, L = cfg["B"], cfg["T"], cfg["S"], cfg["L"]
    M = lists.shape[2]
    T1 = T - M + 1
    tier = oracle.residency.LruTier(n_slots, T) if lru else oracle.ClockTier(n_slots, T, window=1)
    paged = None
    if pages:
        # sequence 0's mapped pages: the page table and the int8 rows they hold
        P = cfg["page_tokens"]
        paged = oracle.residency.PagedTier(tier, P, (T + P - 1) // P)
        k8 = np.zeros((T, cfg["n_kv"], cfg["D"]), np.int8)
        v8 = np.zeros_like(k8)
        ks8 = np.zeros((T, cfg["n_kv"]), np.float16)
        vs8 = np.zeros_like(ks8)
        rk, rks, rv, rvs = synth.tier_page_rows(cfg["B"], T, n_kv=cfg["n_kv"], D=cfg["D"], seed=cfg["seed"],
                                                page_tokens=P, pages=[(0, g) for g in pages], device="cuda")
        for j, g in enumerate(pages):
            paged.map_page(g, j)
            m = min(P, T - g * P)
            k8[g * P:g * P + m], v8[g * P:g * P + m] = rk[j, :m].cpu().numpy(), rv[j, :m].cpu().numpy()
            ks8[g * P:g * P + m], vs8[g * P:g * P + m] = rks[j, :m].cpu().numpy(), rvs[j, :m].cpu().numpy()
        for arr, x in zip((k8, v8, ks8, vs8), (c.res_k[0], c.res_v[0], c.res_ks[0], c.res_vs[0])):
            x = x.cpu().numpy()
            arr[:S] = x[:S]
            arr[T - L:] = x[S:]

    def full(s_, j):
        return np.concatenate([np.arange(S), lists[s_, 0, j], np.arange(T1 + j - L, T1 + j)])
    for s_ in range(warm):
        if paged is not None:
            paged.step(lists[s_, 0, 0], s_)
        else:
            oracle.multiquery.tier_resolve_lists(tier, [full(s_, j) for j in range(M)], T, S, L, s_)
    qs = [c.q[0].cpu().numpy()] if M == 1 else [qm[j] for j in range(M)]
    rk, rv = c.res_k[0].cpu().numpy(), c.res_v[0].cpu().numpy()
    rks, rvs = c.res_ks[0].cpu().numpy(), c.res_vs[0].cpu().numpy()
    sm = cfg["D"] ** -0.5
    t_total, reps = 0.0, 0
    with threadpool_limits(limits=1):
        while reps < 400 and (reps == 0 or t_total < min_seconds) and warm + reps < lists.shape[0]:
            s_ = warm + reps
            idx = [full(s_, j) for j in range(M)]
            t0 = time.perf_counter()
            if paged is not None:
                paged.step(lists[s_, 0, 0], s_)
                oracle.paged_tier_attention(qs[0], records_b, k8, v8, ks8, vs8, idx[0], T, S, L, paged.block,
                                            paged.P, sm, cfg["n_q"] // cfg["n_kv"], cfg["D"])
            else:
                oracle.multiquery.tier_resolve_lists(tier, idx, T, S, L, s_)
                for j in range(M):
                    oracle.tier_attention(qs[j], records_b, rk, rv, rks, rvs, idx[j], T, S, L, sm,
                                          cfg["n_q"] // cfg["n_kv"], cfg["D"])
            t_total += time.perf_counter() - t0
            reps += 1
    return {"value": round(reps / t_total / B, 4), "unit": "layer-steps/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d steps of sequence 0 (resolve + attention%s), scaled to the %d-sequence batch"
                      % (reps, "" if M == 1 else " of its %d query tokens" % M, B),
            "seconds": round(t_total, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", default="cfg2", choices=sorted(CONFIGS))
    ap.add_argument("--layers", type=int, default=0, help="rotating layer buffers (0 = config default)")
    ap.add_argument("--micro-batches", type=int, default=0,
                    help="token configs: run the batch as this many micro-batches on as many streams "
                         "(0 = config default, 1 = one call per layer-step on one stream)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chunk-mib", type=int, default=0,
                    help="prefill: device working buffer in MiB (0 = config default)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB read + 1 GiB write stream (counter calibration)")
    ap.add_argument("--rocprof-summary", metavar="CSV",
                    help="summarise a rocprofv3 csv into --out and exit")
    ap.add_argument("--out", default=None)
    ap.add_argument("--contraction-path", choices=["mfma", "valu"], default="mfma",
                    help="kernel of single-query int8 attention: matrix cores (default) or the "
                         "fp32 vector-ALU kernel kept to measure what the matrix cores bring")
    args = ap.parse_args()
    if args.rocprof_summary:
        rocprof_summary(args.rocprof_summary, args.out or "/dev/stdout")
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = CONFIGS[args.config]
    if args.contraction_path == "valu":
        skv.set_contraction_path(skv.SKV_PATH_VALU)
    if cfg["kind"] == "prefill":
        bench_prefill(cfg, args)
        return
    if cfg["kind"] == "tier_append":
        bench_tier_append(cfg, args)
        return
    if cfg["kind"] == "append":
        bench_append(cfg, args)
        return
    if cfg["kind"] == "tier":
        args.warmup_given = "--warmup" in sys.argv
        args.steps_given = "--steps" in sys.argv
        bench_tier(cfg, args)
        return
    n_layers = args.layers or cfg["layers"]
    log("generating %d layers of %s" % (n_layers, args.config))
    layers = [Layer(cfg, li) for li in range(n_layers)]
    torch.cuda.synchronize()
    multi = cfg.get("M", 0)
    ws = skv.workspace_multi(layers[0].desc, multi) if multi else skv.workspace(layers[0].desc)
    log("warmup", args.warmup)
    for i in range(args.warmup):
        layers[i % n_layers].step(ws)
    skv.check(ws)
    mb = args.micro_batches or cfg.get("mb", 1)
    if mb > 1 and (cfg["kind"] != "token" or cfg["B"] % mb):
        sys.exit("--micro-batches %d: needs a token-mode batch divisible by it" % mb)
    single = None
    if mb > 1:
        # the batch as mb micro-batches on mb streams: while one micro-batch
        # runs its latency-bound select and attention, another streams its
        # sketch; each stream keeps its own micro-batch's layer-steps in order
        streams = [torch.cuda.Stream() for _ in range(mb)]
        for L in layers:
            L.split(mb)
        wss = [skv.workspace_multi(a[0], multi) if multi else skv.workspace(a[0])
               for _, a in layers[0].groups]
        time_loop_groups(layers, wss, streams, args.warmup)
        log("timing %d layer-steps as %d micro-batches of %d sequences"
            % (args.steps, mb, cfg["B"] // mb))
        secs = time_loop_groups(layers, wss, streams, args.steps)
        step_flags = 0
        for w in wss:
            step_flags |= skv.check(w)
        log("timing %d layer-steps as one call each on one stream" % args.steps)
        s1 = time_loop(Layer.step, layers, ws, args.steps)
        step_flags |= skv.check(ws)
        single = {"value": round(args.steps / s1, 2), "ms_per_step": round(1e3 * s1 / args.steps, 5)}
    else:
        log("timing %d layer-steps" % args.steps)
        secs = time_loop(Layer.step, layers, ws, args.steps)
        step_flags = skv.check(ws)   # SKV_FLAG_TOPK_SLOW: some select ran the exact slow path
    # the dominant kernel, in the same step loop: its dispatches record events
    skv.timer_enable(True)
    time_loop(Layer.step, layers, ws, max(50, args.steps // 2))
    score_ms, score_n = skv.timer_read()
    skv.timer_enable(False)
    # the attention kernel (gather + softmax tiles), same step loop
    skv.timer_enable(skv.SKV_TIMER_ATTEND)
    att_steps = max(50, args.steps // 2)
    time_loop(Layer.step, layers, ws, att_steps)
    att_ms, att_n = skv.timer_read()
    skv.timer_enable(False)
    # the same launches on the other units (matrix cores vs vector ALUs): what
    # the matrix cores bring to the contraction each path puts on them (one
    # query: the attention kernel; several: the sketch score)
    alt = None
    if cfg["kind"] == "token" and (multi or cfg["kv"] == "i8"):
        other = skv.SKV_PATH_MFMA if args.contraction_path == "valu" else skv.SKV_PATH_VALU
        skv.set_contraction_path(other)
        time_loop(Layer.step, layers, ws, 5)
        skv.timer_enable(skv.SKV_TIMER_STREAM if multi else skv.SKV_TIMER_ATTEND)
        time_loop(Layer.step, layers, ws, att_steps)
        alt_ms, alt_n = skv.timer_read()
        skv.timer_enable(False)
        skv.set_contraction_path(skv.SKV_PATH_VALU if args.contraction_path == "valu" else skv.SKV_PATH_MFMA)
        alt = ("mfma" if other == skv.SKV_PATH_MFMA else "valu", alt_ms / 1e3 / max(1, alt_n))
    nk = max(50, args.steps // 2)
    kt = {}
    for name in [] if multi else (["qsketch"] if cfg["kind"] == "token" else []) + [
            "score", "score_topk", "topk", "attend"]:
        fn = getattr(Layer, name)
        for i in range(5):
            fn(layers[i % n_layers], ws)
        kt[name] = time_loop(fn, layers, ws, nk) / nk
    skv.check(ws)
    if cfg["kind"] == "token" and not multi:
        # the decode-step append (new token's K/V rows and key sketch), written
        # 2000 rows before the end so every call lands inside the cache; runs
        # after the step timings because it overwrites cache rows
        L0 = layers[0]
        c0 = L0.case
        g = torch.Generator(device="cuda").manual_seed(7)
        k_new = torch.randn((c0.B, c0.n_kv, c0.D), generator=g, device="cuda").to(torch.float16)
        v_new = torch.randn((c0.B, c0.n_kv, c0.D), generator=g, device="cuda").to(torch.float16)
        ctx_a = (L0.ctx - 2000).clamp(min=0).to(torch.int32).contiguous()

        def append_call(layer, ws_):
            skv.append(layer.desc, ctx_a, k_new, v_new, layer.basis, layer.kv, layer.ikeys,
                       layer.iscale, ws_)
        for _ in range(5):
            append_call(L0, ws)
        kt["append"] = time_loop(append_call, [L0], ws, nk) / nk
        skv.check(ws)
    if multi:
        layers[0].step(ws)
        ab = algorithmic_bytes_multi(cfg, layers[0].union_rows())
    else:
        ab = algorithmic_bytes(cfg, layers[0].case.lens if cfg["kind"] == "token" else None)
    value = args.steps / secs
    # the dominant kernel of the step: the fused score-and-collect stream
    score_s = score_ms / 1e3 / max(1, score_n)
    traffic = committed_traffic() if args.config == "cfg2" else None
    roof = dict(kernel=("score_collect_multi" + (" (vector ALU)" if args.contraction_path == "valu" else ""))
                if multi else "score_collect", bound="hbm",
                achieved=round(ab["scan"] / score_s / 1e9, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                frac=round(ab["scan"] / score_s / 1e9 / PEAK_HBM_GBS, 4), traffic=traffic,
                bytes_per_launch=ab["scan"], avg_launch_us=round(score_s * 1e6, 2),
                launches_timed=score_n)
    # the attention kernel: the K/V rows (+ row scales) it must gather at
    # least once (with several queries, the union of a sequence's picks) and
    # the query rows it reads
    att_s = att_ms / 1e3 / att_steps   # one attention launch per step
    att_bytes = ab["gather"] + cfg["B"] * max(1, multi) * cfg["n_q"] * cfg["D"] * 2
    att = dict(kernel="attend" if args.contraction_path == "mfma" or multi else "attend (vector ALU)", bound="hbm",
               achieved=round(att_bytes / att_s / 1e9, 1),
               peak=PEAK_HBM_GBS, unit="GB/s",
               frac=round(att_bytes / att_s / 1e9 / PEAK_HBM_GBS, 4),
               traffic=committed_traffic("attend_", ATTEND_SRC)
               if args.config == "cfg2" and args.contraction_path == "mfma" else None,
               bytes_per_launch=att_bytes, avg_launch_us=round(att_s * 1e6, 2),
               launches_timed=att_n, launches_per_step=round(att_n / att_steps, 2))
    if alt:
        d, nb = (roof, ab["scan"]) if multi else (att, att_bytes)
        d["other_path"] = {"path": alt[0], "avg_launch_us": round(alt[1] * 1e6, 2),
                           "achieved": round(nb / alt[1] / 1e9, 1)}
    if multi and att_s > score_s:
        # several queries: the per-query gathers outweigh the one shared scan
        roof, att = att, roof
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * secs / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if cfg["kind"] == "token" else "bf16",
        "data": "synthetic",
        "config": dict({"workload": cfg["workload"], "name": args.config, "batch": cfg["B"],
                        "ctx": cfg["T"], "rotating_layers": n_layers},
                       **({"contraction_path": "valu"} if args.contraction_path == "valu" else {}),
                       **({"micro_batches": mb, "schedule": "%d micro-batches of %d sequences on %d "
                           "streams" % (mb, cfg["B"] // mb, mb)} if mb > 1 else {}),
                       **({"query_tokens_per_seq": multi} if multi else {})),
        "step_hbm": {"algorithmic_bytes": ab["total"], "achieved_GBps": round(ab["total"] * value / 1e9, 1),
                     "frac_of_peak": round(ab["total"] * value / 1e9 / PEAK_HBM_GBS, 4)},
        "kernels_us": {k: round(v * 1e6, 2) for k, v in kt.items()},
        "select_slow_path": bool(step_flags & skv.SKV_FLAG_TOPK_SLOW),
        "roofline": roof,
        "other_kernel": att,
        # each layer-step covers every sequence of the batch once
        "sequence_layer_steps_per_s": round(value * cfg["B"], 1),
    }
    if single:
        # the same layer-steps issued as one call per step on one stream
        res["single_stream"] = single
    if multi:
        res["query_tokens_per_s"] = round(value * cfg["B"] * multi, 1)
        res["step_hbm"]["union_rows"] = int(ab["gather"] // (cfg["n_kv"] * (cfg["D"] + 2) * 2))
    if args.calib_copy:
        # a plain stream of known size (reads CALIB_BYTES, writes CALIB_BYTES);
        # bitwise_not is used nowhere else, so its counter rows are unambiguous
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        res["calib_copy_bytes"] = CALIB_BYTES
    if not multi:
        # the plain-read ceiling of the scan's bytes (a device buffer of layer 0)
        rc = read_ceiling(layers[0].case.k_cache, ab["scan"])
        rc["scan_kernel_over_ceiling"] = round(rc["avg_launch_us"] / (score_s * 1e6), 4)
        res["read_ceiling"] = rc
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, one core)")
        cb = cpu_baseline(layers[0], cfg)
        cb = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in cb.items()}
        cb["cpu_model"] = cpu_model()
        log("cpu baseline (oracle, all cores)")
        allc = cpu_baseline_all_cores(layers[0], cfg, 1.0 / cb["value"] / cfg["B"]) if not multi else None
        if allc:
            one = cb
            cb = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in allc.items()}
            cb["cpu_model"] = one["cpu_model"]
            cb["one_core"] = {k: one[k] for k in ("value", "cores", "sample", "seconds")}
        res["cpu_baseline"] = cb
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
