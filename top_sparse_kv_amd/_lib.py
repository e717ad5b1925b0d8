"""ctypes declarations of libsparsekv.so (include/sparsekv.h).

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (one runtime per process).  There is no
fallback: if the library is missing, loading raises.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must be loaded first: it provides the HIP runtime)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparsekv.so")

c_i32 = ctypes.c_int32
c_u32 = ctypes.c_uint32
c_i64 = ctypes.c_int64
c_vp = ctypes.c_void_p
c_sz = ctypes.c_size_t

SKV_INDEX_SKETCH_INT4, SKV_INDEX_POOLED_BF16 = 0, 1
SKV_KV_I8_ROWSCALE, SKV_KV_F16, SKV_KV_BF16 = 0, 1, 2
SKV_Q_F16, SKV_Q_BF16 = 0, 1
SKV_FLAG_CTX_RANGE, SKV_FLAG_INDEX_RANGE, SKV_FLAG_TOPK_SLOW, SKV_FLAG_TIER_INPUT = 1, 2, 4, 8
SKV_FLAG_WAIT = 16
SKV_TIER_CLOCK, SKV_TIER_LRU = 0, 1
SKV_TIMER_STREAM, SKV_TIMER_ATTEND = 1, 2
SKV_PATH_MFMA, SKV_PATH_VALU = 0, 1
STATUS = {0: "SKV_OK", 1: "SKV_ERR_INVALID", 2: "SKV_ERR_UNSUPPORTED", 3: "SKV_ERR_WORKSPACE",
          4: "SKV_ERR_OOM", 5: "SKV_ERR_HIP", 6: "SKV_ERR_HOST_MEMORY", 7: "SKV_ERR_STATE"}


class LayerDesc(ctypes.Structure):
    _fields_ = [("struct_size", c_u32), ("batch", c_i32), ("max_ctx", c_i32),
                ("n_kv_heads", c_i32), ("n_q_heads", c_i32), ("head_dim", c_i32),
                ("index_mode", c_i32), ("rank", c_i32), ("index_dim", c_i32), ("block", c_i32),
                ("topk", c_i32), ("n_sink", c_i32), ("n_tail", c_i32), ("kv_dtype", c_i32),
                ("q_dtype", c_i32)]


class KVView(ctypes.Structure):
    _fields_ = [("k", c_vp), ("v", c_vp), ("k_scale", c_vp), ("v_scale", c_vp), ("rows", c_i64)]


class TierDesc(ctypes.Structure):
    _fields_ = [("struct_size", c_u32), ("layer", LayerDesc), ("ctx", c_i32), ("n_slots", c_i32),
                ("window", c_i32), ("host_records", c_vp), ("policy", c_i32),
                ("page_tokens", c_i32), ("pool_pages", c_i32)]


class TierStats(ctypes.Structure):
    _fields_ = [("steps", c_i64), ("picks", c_i64), ("hits", c_i64), ("misses", c_i64),
                ("host_bytes", c_i64), ("in_place", c_i64)]


# (name, restype, argtypes) of every symbol include/sparsekv.h declares
P = ctypes.POINTER
SIGNATURES = [
    ("sparsekv_abi_version", c_i32, []),
    ("sparsekv_status_str", ctypes.c_char_p, [c_i32]),
    ("sparsekv_last_error", ctypes.c_char_p, []),
    ("sparsekv_validate", c_i32, [P(LayerDesc)]),
    ("sparsekv_select_capacity", c_i32, [P(LayerDesc), P(c_i32)]),
    ("sparsekv_workspace_size", c_i32, [P(LayerDesc), P(c_sz)]),
    ("sparsekv_qsketch", c_i32, [P(LayerDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    ("sparsekv_score", c_i32, [P(LayerDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    ("sparsekv_topk", c_i32, [P(LayerDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    ("sparsekv_score_topk", c_i32, [P(LayerDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz,
                                    c_vp]),
    ("sparsekv_attend", c_i32, [P(LayerDesc), c_vp, P(KVView), c_vp, c_vp, ctypes.c_float, c_vp,
                                c_vp, c_sz, c_vp]),
    ("sparsekv_step", c_i32, [P(LayerDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                              P(KVView), c_vp, c_vp, ctypes.c_float, c_vp, c_vp, c_sz, c_vp]),
    ("sparsekv_step_noalloc", c_i32, [P(LayerDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                      c_vp, P(KVView), c_vp, c_vp, ctypes.c_float, c_vp, c_vp,
                                      c_vp]),
    ("sparsekv_read_bytes", c_i32, [c_vp, c_sz, c_vp, c_i32, c_vp]),
    ("sparsekv_workspace_size_multi", c_i32, [P(LayerDesc), c_i32, P(c_sz)]),
    ("sparsekv_step_multi", c_i32, [P(LayerDesc), c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                    P(KVView), c_vp, c_vp, ctypes.c_float, c_vp, c_vp, c_sz, c_vp]),
    ("sparsekv_attend_multi", c_i32, [P(LayerDesc), c_i32, c_vp, P(KVView), c_vp, c_vp,
                                      ctypes.c_float, c_vp, c_vp, c_sz, c_vp]),
    ("sparsekv_prefill_workspace_size", c_i32, [P(LayerDesc), c_i32, P(c_sz)]),
    ("sparsekv_prefill_attend", c_i32, [P(LayerDesc), c_i32, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp,
                                        c_i64, c_vp, c_sz, ctypes.c_float, c_vp, c_vp, c_sz, c_vp]),
    ("sparsekv_append", c_i32, [P(LayerDesc), c_vp, c_vp, c_vp, c_vp, P(KVView), c_vp, c_vp, c_vp,
                                c_sz, c_vp]),
    ("sparsekv_append_block", c_i32, [P(LayerDesc), c_vp, c_vp, c_vp, c_vp, c_vp, P(KVView), c_vp,
                                      c_vp, c_sz, c_vp]),
    ("sparsekv_check", c_i32, [c_vp, c_sz, c_vp, P(c_u32)]),
    ("sparsekv_timer_enable", c_i32, [c_i32]),
    ("sparsekv_timer_read", c_i32, [P(ctypes.c_double), P(c_i64)]),
    ("sparsekv_set_contraction_path", c_i32, [c_i32]),
    ("sparsekv_tier_create", c_i32, [P(TierDesc), P(c_vp)]),
    ("sparsekv_tier_host_records", c_vp, [c_vp]),
    ("sparsekv_tier_host_ptr", c_vp, [c_vp]),
    ("sparsekv_tier_resident", c_i32, [c_vp, P(KVView)]),
    ("sparsekv_tier_load_resident", c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    ("sparsekv_tier_resolve", c_i32, [c_vp, c_vp, c_vp, c_i32, c_vp, c_vp]),
    ("sparsekv_tier_resolve_multi", c_i32, [c_vp, c_i32, c_vp, c_vp, c_i32, c_vp, c_vp]),
    ("sparsekv_tier_attend", c_i32, [c_vp, c_vp, c_vp, c_vp, ctypes.c_float, c_vp, c_vp, c_sz, c_vp]),
    ("sparsekv_tier_map_page", c_i32, [c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]),
    ("sparsekv_tier_unmap_page", c_i32, [c_vp, c_i32, c_i32, c_vp]),
    ("sparsekv_tier_append", c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    ("sparsekv_tier_stats", c_i32, [c_vp, P(TierStats), c_vp]),
    ("sparsekv_tier_slots", c_i32, [c_vp, c_vp, c_vp]),
    ("sparsekv_tier_reset", c_i32, [c_vp, c_vp]),
    ("sparsekv_tier_destroy", None, [c_vp]),
]

_LIB = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libsparsekv.so once.  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError("libsparsekv.so is not built (%s); run python -m top_sparse_kv_amd.build"
                           % path)
    lib = ctypes.CDLL(path)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib
