"""Python binding of libsparsekv (the gfx950 sparse-KV decode step).

Thin argument marshalling over the C ABI in include/sparsekv.h: every function
here has the name of the C entry point it calls (without the sparsekv_
prefix), takes torch tensors for device buffers, passes their addresses and
the current HIP stream, and raises SkvError on a non-OK status.  All compute
runs in the library's HIP kernels; torch only provides device memory and
streams.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import (KVView, LayerDesc, TierDesc, TierStats, SKV_INDEX_SKETCH_INT4,  # noqa: F401
                   SKV_INDEX_POOLED_BF16, SKV_KV_I8_ROWSCALE, SKV_KV_F16, SKV_KV_BF16, SKV_Q_F16,
                   SKV_Q_BF16, SKV_FLAG_CTX_RANGE, SKV_FLAG_INDEX_RANGE, SKV_FLAG_TOPK_SLOW,
                   SKV_FLAG_TIER_INPUT, SKV_TIER_CLOCK, SKV_TIER_LRU,
                   SKV_TIMER_STREAM, SKV_TIMER_ATTEND, SKV_PATH_MFMA, SKV_PATH_VALU)


class SkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (_lib.STATUS.get(status, status), msg))
        self.status = status


def lib():
    return _lib.load()


def _check(st: int):
    if st != 0:
        raise SkvError(st, (lib().sparsekv_last_error() or b"").decode())


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("device tensor expected")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def token_desc(batch, max_ctx, n_kv_heads, n_q_heads, head_dim, *, rank=64, topk, n_sink, n_tail,
               kv_dtype=SKV_KV_I8_ROWSCALE) -> LayerDesc:
    return LayerDesc(ctypes.sizeof(LayerDesc), batch, max_ctx, n_kv_heads, n_q_heads, head_dim,
                     SKV_INDEX_SKETCH_INT4, rank, 0, 1, topk, n_sink, n_tail, kv_dtype, SKV_Q_F16)


def block_desc(batch, max_ctx, n_kv_heads, n_q_heads, head_dim, *, index_dim=128,
               topk_blocks) -> LayerDesc:
    return LayerDesc(ctypes.sizeof(LayerDesc), batch, max_ctx, n_kv_heads, n_q_heads, head_dim,
                     SKV_INDEX_POOLED_BF16, 0, index_dim, 4, topk_blocks, 0, 0, SKV_KV_BF16,
                     SKV_Q_BF16)


def kv_view(k: torch.Tensor, v: torch.Tensor, k_scale=None, v_scale=None,
            rows: Optional[int] = None) -> KVView:
    """View of K/V rows shaped [B][rows][H_kv][D] (+ fp16 scales [B][rows][H_kv])."""
    _dev(k, v, k_scale, v_scale)
    return KVView(_p(k), _p(v), _p(k_scale), _p(v_scale), int(rows if rows is not None else k.shape[1]))


def abi_version() -> int:
    return lib().sparsekv_abi_version()


def validate(desc: LayerDesc):
    _check(lib().sparsekv_validate(ctypes.byref(desc)))


def select_capacity(desc: LayerDesc) -> int:
    c = _lib.c_i32()
    _check(lib().sparsekv_select_capacity(ctypes.byref(desc), ctypes.byref(c)))
    return c.value


def workspace_size(desc: LayerDesc) -> int:
    n = _lib.c_sz()
    _check(lib().sparsekv_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def workspace(desc: LayerDesc, device="cuda") -> torch.Tensor:
    """A zero-filled workspace of the required size."""
    return torch.zeros(workspace_size(desc), dtype=torch.uint8, device=device)


def qsketch(desc, q, basis, qs, qs_scale, ws, stream=None):
    _dev(q, basis, qs, qs_scale, ws)
    _check(lib().sparsekv_qsketch(ctypes.byref(desc), _p(q), _p(basis), _p(qs), _p(qs_scale),
                                  _p(ws), ws.numel(), _stream(stream)))


def score(desc, ctx_len, index_query, index_keys, index_scale, keys, ws, stream=None):
    _dev(ctx_len, index_query, index_keys, index_scale, keys, ws)
    _check(lib().sparsekv_score(ctypes.byref(desc), _p(ctx_len), _p(index_query), _p(index_keys),
                                _p(index_scale), _p(keys), _p(ws), ws.numel(), _stream(stream)))


def topk(desc, ctx_len, keys, idx, n_sel, ws, stream=None):
    _dev(ctx_len, keys, idx, n_sel, ws)
    _check(lib().sparsekv_topk(ctypes.byref(desc), _p(ctx_len), _p(keys), _p(idx), _p(n_sel),
                               _p(ws), ws.numel(), _stream(stream)))


def score_topk(desc, ctx_len, index_query, index_keys, index_scale, idx, n_sel, ws, stream=None):
    _dev(ctx_len, index_query, index_keys, index_scale, idx, n_sel, ws)
    _check(lib().sparsekv_score_topk(ctypes.byref(desc), _p(ctx_len), _p(index_query),
                                     _p(index_keys), _p(index_scale), _p(idx), _p(n_sel), _p(ws),
                                     ws.numel(), _stream(stream)))


def attend_multi(desc, n_query, q, kv: KVView, idx, n_sel, sm_scale, out, ws, stream=None):
    """sparsekv_attend_multi: q [B][n_query][H_q][D], idx [B][n_query][cap],
    n_sel [B][n_query], out fp32 [B][n_query][H_q][D]; ws from workspace_multi."""
    _dev(q, idx, n_sel, out, ws)
    _check(lib().sparsekv_attend_multi(ctypes.byref(desc), int(n_query), _p(q), ctypes.byref(kv),
                                       _p(idx), _p(n_sel), float(sm_scale), _p(out), _p(ws),
                                       ws.numel(), _stream(stream)))


def attend(desc, q, kv: KVView, idx, n_sel, sm_scale, out, ws, stream=None):
    _dev(q, idx, n_sel, out, ws)
    _check(lib().sparsekv_attend(ctypes.byref(desc), _p(q), ctypes.byref(kv), _p(idx), _p(n_sel),
                                 float(sm_scale), _p(out), _p(ws), ws.numel(), _stream(stream)))


def step(desc, ctx_len, q, basis, qs, qs_scale, index_query, index_keys, index_scale, kv: KVView,
         idx, n_sel, sm_scale, out, ws, stream=None):
    _dev(ctx_len, q, basis, qs, qs_scale, index_query, index_keys, index_scale, idx, n_sel, out, ws)
    _check(lib().sparsekv_step(ctypes.byref(desc), _p(ctx_len), _p(q), _p(basis), _p(qs),
                               _p(qs_scale), _p(index_query), _p(index_keys), _p(index_scale),
                               ctypes.byref(kv), _p(idx), _p(n_sel), float(sm_scale), _p(out),
                               _p(ws), ws.numel(), _stream(stream)))


def step_noalloc(desc, ctx_len, q, basis, qs, qs_scale, index_query, index_keys, index_scale,
                 kv: KVView, idx, n_sel, sm_scale, out, flags=None, stream=None):
    """sparsekv_step without a workspace: the library's own device scratch is
    used.  flags (optional int32/uint32 device tensor of >= 1 element) receives
    the call's device flag word."""
    _dev(ctx_len, q, basis, qs, qs_scale, index_query, index_keys, index_scale, idx, n_sel, out, flags)
    _check(lib().sparsekv_step_noalloc(ctypes.byref(desc), _p(ctx_len), _p(q), _p(basis), _p(qs),
                                       _p(qs_scale), _p(index_query), _p(index_keys), _p(index_scale),
                                       ctypes.byref(kv), _p(idx), _p(n_sel), float(sm_scale), _p(out),
                                       _p(flags), _stream(stream)))


def read_bytes(src_ptr: int, nbytes: int, sink, n_wg: int, stream=None):
    """sparsekv_read_bytes: a plain streaming read of nbytes at device address
    src_ptr (device memory or mapped pinned host memory); sink int32 device
    tensor of >= n_wg elements."""
    _dev(sink)
    _check(lib().sparsekv_read_bytes(ctypes.c_void_p(src_ptr), int(nbytes), _p(sink), int(n_wg),
                                     _stream(stream)))


def workspace_size_multi(desc: LayerDesc, n_query: int) -> int:
    n = _lib.c_sz()
    _check(lib().sparsekv_workspace_size_multi(ctypes.byref(desc), int(n_query), ctypes.byref(n)))
    return n.value


def workspace_multi(desc: LayerDesc, n_query: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for sparsekv_step_multi with n_query queries per sequence."""
    return torch.zeros(workspace_size_multi(desc, n_query), dtype=torch.uint8, device=device)


def step_multi(desc, n_query, ctx_len, q, basis, qs, qs_scale, index_keys, index_scale, kv: KVView,
               idx, n_sel, sm_scale, out, ws, stream=None):
    """n_query query tokens per sequence (the cache's last positions), each with
    its own pick at its causal context (sparsekv_step_multi).  q [B][M][H_q][D];
    qs [B][M][H_kv*R], qs_scale [B][M], idx [B][M][cap], n_sel [B][M],
    out [B][M][H_q][D]."""
    _dev(ctx_len, q, basis, qs, qs_scale, index_keys, index_scale, idx, n_sel, out, ws)
    _check(lib().sparsekv_step_multi(ctypes.byref(desc), int(n_query), _p(ctx_len), _p(q), _p(basis),
                                     _p(qs), _p(qs_scale), _p(index_keys), _p(index_scale),
                                     ctypes.byref(kv), _p(idx), _p(n_sel), float(sm_scale), _p(out),
                                     _p(ws), ws.numel(), _stream(stream)))


def prefill_workspace_size(desc: LayerDesc, n_query: int) -> int:
    n = _lib.c_sz()
    _check(lib().sparsekv_prefill_workspace_size(ctypes.byref(desc), int(n_query), ctypes.byref(n)))
    return n.value


def prefill_attend(desc, q, idx, n_sel, host_k, host_v, chunk_buf, sm_scale, out, ws, stream=None):
    """Attention of P prefill queries over their picked rows of K/V held in host
    memory, streamed once through chunk_buf (sparsekv_prefill_attend).  q
    [P][H_q][D], idx [P][cap], n_sel [P], out [P][H_q][D] on the device;
    host_k / host_v [T][H_kv][D] host tensors (pinned for DMA)."""
    _dev(q, idx, n_sel, chunk_buf, out, ws)
    for t in (host_k, host_v):
        if t.is_cuda or not t.is_contiguous():
            raise ValueError("host_k / host_v must be contiguous host tensors")
    _check(lib().sparsekv_prefill_attend(ctypes.byref(desc), q.shape[0], _p(q), _p(idx), _p(n_sel),
                                         idx.shape[1], ctypes.c_void_p(host_k.data_ptr()),
                                         ctypes.c_void_p(host_v.data_ptr()), host_k.shape[0],
                                         _p(chunk_buf), chunk_buf.numel() * chunk_buf.element_size(),
                                         float(sm_scale), _p(out), _p(ws), ws.numel(),
                                         _stream(stream)))


def append(desc, ctx_len, k_new, v_new, basis, kv: KVView, index_keys, index_scale, ws, stream=None):
    """Writes the new token of every sequence at row ctx_len[b] (K/V rows,
    key sketch) and advances ctx_len (sparsekv_append)."""
    _dev(ctx_len, k_new, v_new, basis, index_keys, index_scale, ws)
    _check(lib().sparsekv_append(ctypes.byref(desc), _p(ctx_len), _p(k_new), _p(v_new), _p(basis),
                                 ctypes.byref(kv), _p(index_keys), _p(index_scale), _p(ws), ws.numel(),
                                 _stream(stream)))


def append_block(desc, ctx_len, k_new, v_new, index_raw, index_stage, kv: KVView, index_keys, ws,
                 stream=None):
    """Block mode: bf16 K/V rows of the new token, its raw indexer key staged,
    the pooled key when its block completes, ctx_len advanced
    (sparsekv_append_block)."""
    _dev(ctx_len, k_new, v_new, index_raw, index_stage, index_keys, ws)
    _check(lib().sparsekv_append_block(ctypes.byref(desc), _p(ctx_len), _p(k_new), _p(v_new),
                                       _p(index_raw), _p(index_stage), ctypes.byref(kv),
                                       _p(index_keys), _p(ws), ws.numel(), _stream(stream)))


def timer_enable(on=True):
    """Diagnostic: bracket each launch of one kind of kernel with events.
    False / 0: off; SKV_TIMER_ATTEND: the attention kernel; True or
    SKV_TIMER_STREAM: the streaming kernel of each call."""
    kind = 0 if not on else (SKV_TIMER_ATTEND if on == SKV_TIMER_ATTEND else SKV_TIMER_STREAM)
    _check(lib().sparsekv_timer_enable(kind))


def set_contraction_path(path: int):
    """sparsekv_set_contraction_path: SKV_PATH_MFMA (default, matrix cores) or
    SKV_PATH_VALU (vector ALUs) for single-query int8 attention and the
    multi-query sketch score; a measurement aid, process-wide."""
    _check(lib().sparsekv_set_contraction_path(int(path)))


def timer_read():
    """(total kernel milliseconds, launches) recorded since timer_enable."""
    ms, n = ctypes.c_double(), _lib.c_i64()
    _check(lib().sparsekv_timer_read(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def check(ws, stream=None, raise_on_error: bool = True) -> int:
    """Synchronizes, returns and clears the device flag bits; raises on error
    flags unless raise_on_error is False."""
    f = _lib.c_u32()
    st = lib().sparsekv_check(_p(ws), ws.numel(), _stream(stream), ctypes.byref(f))
    if st not in (0, 7):
        _check(st)
    if st == 7 and raise_on_error:
        raise SkvError(st, "device flags 0x%x" % f.value)
    return f.value


@dataclass
class _TierHandle:
    ptr: ctypes.c_void_p


class Tier:
    """Host-RAM KV tier with a GPU hot buffer (sparsekv_tier_*); policy
    SKV_TIER_CLOCK (windowed CLOCK) or SKV_TIER_LRU."""

    def __init__(self, layer: LayerDesc, ctx: int, n_slots: int, window: int = 1,
                 host_records: Optional[int] = None, policy: int = SKV_TIER_CLOCK,
                 page_tokens: int = 0, pool_pages: int = 0):
        self.layer = layer
        d = TierDesc(ctypes.sizeof(TierDesc), layer, ctx, n_slots, window,
                     ctypes.c_void_p(host_records) if host_records else None, policy,
                     page_tokens, pool_pages)
        self.page_tokens, self.pool_pages = page_tokens, pool_pages
        h = ctypes.c_void_p()
        _check(lib().sparsekv_tier_create(ctypes.byref(d), ctypes.byref(h)))
        self._h = h
        self.ctx, self.n_slots, self.window = ctx, n_slots, window
        D = layer.head_dim
        self.record_bytes = 2 * (D // 2 + 2 * (D // 64))

    def host_records(self):
        """numpy uint8 view [B][max_ctx][H_kv][record] of the pinned host
        records (the caller fills positions below the creation context)."""
        import numpy as np
        ptr = lib().sparsekv_tier_host_records(self._h)
        cap = self.layer.max_ctx
        n = self.layer.batch * cap * self.layer.n_kv_heads * self.record_bytes
        buf = (ctypes.c_uint8 * n).from_address(ptr)
        return np.frombuffer(buf, dtype=np.uint8).reshape(
            self.layer.batch, cap, self.layer.n_kv_heads, self.record_bytes)

    def append(self, ctx_len, k_new, v_new, basis, index_keys, index_scale, stream=None):
        """sparsekv_tier_append: the new token of every sequence (fp16 k_new,
        v_new [B][H_kv][D]) into the host records, the tail ring and the key
        sketch; ctx_len (device int32 [B]) must equal the tier's context."""
        _dev(ctx_len, k_new, v_new, basis, index_keys, index_scale)
        _check(lib().sparsekv_tier_append(self._h, _p(ctx_len), _p(k_new), _p(v_new), _p(basis),
                                          _p(index_keys), _p(index_scale), _stream(stream)))

    def resident(self) -> KVView:
        v = KVView()
        _check(lib().sparsekv_tier_resident(self._h, ctypes.byref(v)))
        return v

    def load_resident(self, k, v, k_scale, v_scale, stream=None):
        _dev(k, v, k_scale, v_scale)
        _check(lib().sparsekv_tier_load_resident(self._h, _p(k), _p(v), _p(k_scale), _p(v_scale),
                                                 _stream(stream)))

    def resolve(self, idx, n_sel, step: int, rows, stream=None):
        _dev(idx, n_sel, rows)
        _check(lib().sparsekv_tier_resolve(self._h, _p(idx), _p(n_sel), int(step), _p(rows),
                                           _stream(stream)))

    def resolve_multi(self, n_query: int, idx, n_sel, step: int, rows, stream=None):
        """sparsekv_tier_resolve_multi: idx [B][n_query][cap], n_sel
        [B][n_query], rows [B][n_query][cap] (device int32)."""
        _dev(idx, n_sel, rows)
        _check(lib().sparsekv_tier_resolve_multi(self._h, int(n_query), _p(idx), _p(n_sel),
                                                 int(step), _p(rows), _stream(stream)))

    def attend(self, q, rows, n_sel, sm_scale, out, ws, stream=None):
        """sparsekv_tier_attend: attention over the resident rows listed in rows."""
        _dev(q, rows, n_sel, out, ws)
        _check(lib().sparsekv_tier_attend(self._h, _p(q), _p(rows), _p(n_sel), float(sm_scale), _p(out),
                                          _p(ws), ws.numel(), _stream(stream)))

    def map_page(self, seq: int, page: int, block: int, k=None, v=None, k_scale=None, v_scale=None,
                 stream=None):
        """sparsekv_tier_map_page: page `page` of sequence `seq` resident in pool
        block `block`; k, v [P][H_kv][D] int8 and scales [P][H_kv] (device), or
        all None when the block already holds the rows."""
        _dev(k, v, k_scale, v_scale)
        _check(lib().sparsekv_tier_map_page(self._h, int(seq), int(page), int(block), _p(k), _p(v),
                                            _p(k_scale), _p(v_scale), _stream(stream)))

    def unmap_page(self, seq: int, page: int, stream=None):
        _check(lib().sparsekv_tier_unmap_page(self._h, int(seq), int(page), _stream(stream)))

    def stats(self, stream=None) -> TierStats:
        s = TierStats()
        _check(lib().sparsekv_tier_stats(self._h, ctypes.byref(s), _stream(stream)))
        return s

    def slots(self, stream=None):
        import numpy as np
        out = np.empty((self.layer.batch, self.n_slots), dtype=np.int32)
        _check(lib().sparsekv_tier_slots(self._h, out.ctypes.data_as(ctypes.c_void_p),
                                         _stream(stream)))
        return out

    def reset(self, stream=None):
        _check(lib().sparsekv_tier_reset(self._h, _stream(stream)))

    def close(self):
        if self._h:
            lib().sparsekv_tier_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
