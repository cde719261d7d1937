"""Paged grouped-query attention with rotary embeddings for AMD MI355X (gfx950).

The compute lives in libastr.so (hand-written HIP kernels behind the C ABI in
include/astr.h); this package is its Python binding.  Importing it does not
touch the GPU; the library is loaded on first use and a missing library is an
error, never a fallback.
"""

from .api import (  # noqa: F401
    KVCache, PagePool, cache_from_bind, ceiling_mfma_loop, ceiling_stream_read, decode_attn, decode_attn_noalloc, decode_attn_write, decode_num_splits, decode_split_items,
    decode_workspace, decode_workspace_bytes,
    prefill_attn, prefill_plan, prefill_workspace_bytes, rope_backward, rope_kv_write, rope_table,
)
from ._lib import AstrArgError, AstrError, LIB_PATH  # noqa: F401
