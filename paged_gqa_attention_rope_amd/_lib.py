"""ctypes view of libastr.so: the prototypes of include/astr.h and
include/astr_ceiling.h, nothing else."""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libastr.so")

ASTR_OK = 0
ASTR_E_INVAL = -1
ASTR_E_UNSUPPORTED = -2
ASTR_E_NOMEM = -3
ASTR_E_LAUNCH = -4
ASTR_F32 = 0
ASTR_BF16 = 1

# every symbol include/*.h declares
EXPORTS = (
    "astr_last_error", "astr_rope_table", "astr_rope_kv_write", "astr_rope_backward",
    "astr_decode_num_splits", "astr_decode_workspace_bytes", "astr_decode_split_items", "astr_decode_attn_write",
    "astr_decode_attn", "astr_decode_attn_noalloc", "astr_prefill_attn", "astr_prefill_workspace_bytes", "astr_prefill_plan",
    "astr_pagepool_create", "astr_pagepool_destroy",
    "astr_pagepool_admit", "astr_pagepool_extend", "astr_pagepool_bind", "astr_pagepool_insert",
    "astr_pagepool_release", "astr_pagepool_table", "astr_pagepool_free_pages",
    "astr_pagepool_page_ref", "astr_pagepool_complete", "astr_pagepool_evict",
    "astr_pagepool_cached_pages", "astr_pagepool_evicted_pages",
    # include/astr_ceiling.h
    "astr_ceiling_stream_read", "astr_ceiling_mfma_loop",
)

c_int, c_i32p, c_vp = ctypes.c_int, ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p


class KvMeta(ctypes.Structure):
    """astr_kv_meta."""
    _fields_ = [
        ("k_buffer", c_vp), ("v_buffer", c_vp), ("pool_slots", ctypes.c_int64),
        ("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("req_to_token", c_vp), ("num_reqs", ctypes.c_int32), ("max_ctx_len", ctypes.c_int32),
        ("req_pool_indices", c_vp), ("kv_indptr", c_vp), ("qo_indptr", c_vp),
        ("q_tile_to_batch", c_vp), ("q_tile_to_index", c_vp),
        ("batch", ctypes.c_int32), ("max_len", ctypes.c_int32),
        ("num_q_tiles", ctypes.c_int32), ("q_tile", ctypes.c_int32),
        ("split_item_batch", c_vp), ("split_item_index", c_vp),
        ("num_split_items", ctypes.c_int32), ("split_item_chunk", ctypes.c_int32),
        ("prefill_units", c_vp), ("num_prefill_units", ctypes.c_int32),
        ("num_prefill_pairs", ctypes.c_int32), ("prefill_workspace", c_vp),
        ("prefill_workspace_bytes", ctypes.c_size_t),
    ]


_lib = None


def lib():
    """Load libastr.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: run `python -m paged_gqa_attention_rope_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.astr_last_error.restype = ctypes.c_char_p
    L.astr_last_error.argtypes = []
    L.astr_rope_table.argtypes = [c_vp, c_int, c_int, ctypes.c_double, c_vp]
    L.astr_rope_kv_write.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_vp, c_int,
                                     ctypes.POINTER(KvMeta), c_int, c_int, c_vp]
    L.astr_rope_backward.argtypes = [c_vp, c_vp, c_int, c_int, c_int, c_vp, c_int, c_int, c_vp]
    L.astr_decode_num_splits.argtypes = [c_int, c_int]
    L.astr_decode_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int]
    L.astr_decode_workspace_bytes.restype = ctypes.c_size_t
    L.astr_decode_split_items.argtypes = [c_i32p, c_int, c_int, c_i32p, c_i32p, c_int, ctypes.POINTER(c_int)]
    L.astr_decode_attn.argtypes = [c_vp, c_int, ctypes.POINTER(KvMeta), c_int, c_int, ctypes.c_float,
                                   c_vp, c_vp, c_vp, c_int, c_vp]
    L.astr_decode_attn_noalloc.argtypes = [c_vp, c_int, ctypes.POINTER(KvMeta), c_int, c_int, ctypes.c_float,
                                           c_vp, c_int, c_vp]
    L.astr_decode_attn_write.argtypes = [c_vp, c_vp, c_vp, c_int, ctypes.POINTER(KvMeta), c_int, c_vp, c_int,
                                         c_int, ctypes.c_float, c_vp, c_vp, c_vp, c_int, c_vp]
    L.astr_prefill_attn.argtypes = [c_vp, c_int, c_int, ctypes.POINTER(KvMeta), c_int, ctypes.c_float,
                                    c_vp, c_int, c_vp]
    L.astr_prefill_workspace_bytes.argtypes = [c_int, c_int, c_int]
    L.astr_prefill_workspace_bytes.restype = ctypes.c_size_t
    L.astr_prefill_plan.argtypes = [c_i32p, c_i32p, c_i32p, c_int, c_i32p, c_i32p, c_int, c_int, c_int, c_int,
                                    c_i32p, c_int, ctypes.POINTER(c_int), ctypes.POINTER(c_int)]
    L.astr_pagepool_create.argtypes = [ctypes.POINTER(c_vp), c_int, ctypes.c_int64, c_int, c_int,
                                       c_int, c_i32p]
    L.astr_pagepool_destroy.argtypes = [c_vp]
    L.astr_pagepool_destroy.restype = None
    L.astr_pagepool_admit.argtypes = [c_vp, c_i32p, c_int, ctypes.POINTER(c_int), ctypes.POINTER(c_int)]
    L.astr_pagepool_extend.argtypes = [c_vp, c_int, c_int]
    L.astr_pagepool_bind.argtypes = [c_vp, c_i32p, c_i32p, c_int, c_int, c_i32p, c_i32p, c_i32p,
                                     c_i32p, c_i32p, c_i32p, c_int, ctypes.POINTER(c_int),
                                     ctypes.POINTER(c_int)]
    L.astr_pagepool_insert.argtypes = [c_vp, c_int, c_i32p, c_int]
    L.astr_pagepool_release.argtypes = [c_vp, c_int]
    L.astr_pagepool_table.argtypes = [c_vp]
    L.astr_pagepool_table.restype = c_i32p
    L.astr_pagepool_free_pages.argtypes = [c_vp]
    L.astr_pagepool_free_pages.restype = ctypes.c_int64
    L.astr_pagepool_page_ref.argtypes = [c_vp, ctypes.c_int64]
    L.astr_pagepool_complete.argtypes = [c_vp, c_int, c_i32p, c_int]
    L.astr_pagepool_evict.argtypes = [c_vp, ctypes.c_int64]
    L.astr_pagepool_evict.restype = ctypes.c_int64
    L.astr_pagepool_cached_pages.argtypes = [c_vp]
    L.astr_pagepool_cached_pages.restype = ctypes.c_int64
    L.astr_pagepool_evicted_pages.argtypes = [c_vp]
    L.astr_pagepool_evicted_pages.restype = ctypes.c_int64
    L.astr_ceiling_stream_read.argtypes = [c_vp, ctypes.c_size_t, c_int, c_int, c_vp, c_vp]
    L.astr_ceiling_mfma_loop.argtypes = [c_int, c_int, c_vp, c_vp]
    _lib = L
    return L


class AstrError(RuntimeError):
    """A non-OK status from libastr (pool exhausted, launch rejected)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"astr status {status}: {message}")
        self.status = status


class AstrArgError(ValueError):
    """ASTR_E_INVAL or ASTR_E_UNSUPPORTED: the call was rejected before any launch."""

    def __init__(self, status: int, message: str):
        super().__init__(f"astr status {status}: {message}")
        self.status = status


def check(status: int):
    if status != ASTR_OK:
        msg = lib().astr_last_error().decode(errors="replace")
        if status in (ASTR_E_INVAL, ASTR_E_UNSUPPORTED):
            raise AstrArgError(status, msg)
        raise AstrError(status, msg)
