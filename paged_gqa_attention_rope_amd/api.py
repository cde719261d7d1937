"""Python binding of libastr: argument marshalling around the C ABI.

Every step of the attention path runs in the library's HIP kernels; torch
only supplies device memory and the current stream.  The library receives
raw pointers, so this layer checks what a pointer cannot carry -- device,
dtype, contiguity and buffer sizes -- before passing tensors down, so that a
wrong shape is a Python error rather than an out-of-bounds access.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from ._lib import ASTR_BF16, ASTR_E_INVAL, ASTR_F32, KvMeta, check, lib

_DTYPES = {torch.float32: ASTR_F32, torch.bfloat16: ASTR_BF16}


def _vp(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _dev_tensor(t: torch.Tensor, name: str, dtype=None, device=None, numel_at_least: int = 0):
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.is_cuda, f"{name} must be a device tensor")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    if device is not None:
        _need(t.device == device, f"{name} is on {t.device}, expected {device}")
    _need(t.numel() >= numel_at_least, f"{name} holds {t.numel()} elements, needs {numel_at_least}")


# ---------------------------------------------------------------------------
# the KVCache record
# ---------------------------------------------------------------------------

@dataclass
class KVCache:
    """Per-step view of the KV cache (the KVCache record: data, no behaviour).

    k_buffer / v_buffer: [n_layers, pool_slots, n_kv_heads, head_dim].
    req_to_token: [num_reqs, max_ctx_len] int32.  Index tensors are int32 on
    the pool's device; batch, max_len and num_q_tiles are host ints.
    """

    k_buffer: torch.Tensor
    v_buffer: torch.Tensor
    req_to_token: torch.Tensor
    req_pool_indices: torch.Tensor
    seq_lens: torch.Tensor
    out_cache_loc: torch.Tensor
    kv_indptr: torch.Tensor
    max_len: int
    qo_indptr: Optional[torch.Tensor] = None
    q_tile_to_batch: Optional[torch.Tensor] = None
    q_tile_to_index: Optional[torch.Tensor] = None
    num_q_tiles: int = 0
    q_tile: int = 64
    # decode work items (batch entry, split) for split_item_chunk; optional
    split_item_batch: Optional[torch.Tensor] = None
    split_item_index: Optional[torch.Tensor] = None
    num_split_items: int = 0
    split_item_chunk: int = 0
    # prefill work plan ([n, 8] int32 units) and its workspace; optional
    prefill_units: Optional[torch.Tensor] = None
    num_prefill_pairs: int = 0
    prefill_workspace: Optional[torch.Tensor] = None

    @property
    def batch(self) -> int:
        return int(self.req_pool_indices.numel())


def decode_split_items(seq_lens, split_chunk: int):
    """Host (batch entry, split) work items of a decode step
    (astr_decode_split_items); returns two int32 arrays."""
    seq = np.ascontiguousarray(seq_lens, dtype=np.int32)
    _need(split_chunk >= 1, "split_chunk must be positive")
    cap = int(sum(max(1, -(-int(x) // split_chunk)) for x in seq))
    ib = np.zeros(max(cap, 1), np.int32)
    ix = np.zeros(max(cap, 1), np.int32)
    n = ctypes.c_int()
    check(lib().astr_decode_split_items(_i32p(seq), int(seq.size), int(split_chunk), _i32p(ib), _i32p(ix),
                                        max(cap, 1), ctypes.byref(n)))
    return ib[:n.value], ix[:n.value]


def prefill_plan(meta: dict, n_heads: int, num_cus: int = 256):
    """Host prefill work plan of a bound step (astr_prefill_plan) for a model
    with n_heads query heads; returns ([n, 8] int32 units, number of pairs)."""
    _need(n_heads >= 4, "the prefill plan is for 4 or more query heads")
    nt = int(meta["num_q_tiles"])
    qo, kv = _i32(meta["qo_indptr"]), _i32(meta["kv_indptr"])
    rpi = _i32(meta["req_pool_indices"])
    _need(rpi.size == qo.size - 1, "req_pool_indices must have one entry per batch entry")
    t2b, t2i = _i32(meta["q_tile_to_batch"])[:nt], _i32(meta["q_tile_to_index"])[:nt]
    cap = max(16 * nt, 8)
    units = np.zeros((cap, 8), np.int32)
    n, pairs = ctypes.c_int(), ctypes.c_int()
    check(lib().astr_prefill_plan(_i32p(qo), _i32p(kv), _i32p(rpi), int(qo.size) - 1, _i32p(t2b), _i32p(t2i), nt,
                                  int(meta["q_tile"]), int(n_heads) // 4, int(num_cus), _i32p(units), cap,
                                  ctypes.byref(n), ctypes.byref(pairs)))
    return units[:n.value].copy(), pairs.value


def prefill_workspace_bytes(pairs: int, n_heads: int, head_dim: int) -> int:
    return int(lib().astr_prefill_workspace_bytes(int(pairs), int(n_heads), int(head_dim)))


def cache_from_bind(k_buffer: torch.Tensor, v_buffer: torch.Tensor, table: np.ndarray,
                    meta: dict, split_chunk: Optional[int] = None, prefill_heads: Optional[int] = None,
                    prefill_workspace: Optional[torch.Tensor] = None, num_cus: int = 256) -> KVCache:
    """Upload one step's host metadata (PagePool.bind) next to the pool; with
    split_chunk, also the decode work items for that chunk; with prefill_heads
    (the query heads of the prefill call), also the prefill work plan and a
    workspace for it (prefill_workspace is used when large enough, else a
    zeroed one is allocated).  Only the bf16 head_dim-128 prefill with a
    multiple of 4 query heads per KV head follows plans; for other pools no
    plan is built."""
    dev = k_buffer.device
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    c = KVCache(k_buffer=k_buffer, v_buffer=v_buffer, req_to_token=up(table),
                req_pool_indices=up(meta["req_pool_indices"]), seq_lens=up(meta["seq_lens"]),
                out_cache_loc=up(meta["out_cache_loc"]), kv_indptr=up(meta["kv_indptr"]),
                max_len=int(meta["max_len"]), qo_indptr=up(meta["qo_indptr"]),
                q_tile_to_batch=up(meta["q_tile_to_batch"]),
                q_tile_to_index=up(meta["q_tile_to_index"]),
                num_q_tiles=int(meta["num_q_tiles"]), q_tile=int(meta["q_tile"]))
    if split_chunk is not None:
        ib, ix = decode_split_items(meta["seq_lens"], split_chunk)
        c.split_item_batch, c.split_item_index = up(ib), up(ix)
        c.num_split_items, c.split_item_chunk = int(ib.size), int(split_chunk)
    n_kv, hd = int(k_buffer.shape[2]), int(k_buffer.shape[3])
    if (prefill_heads is not None and int(meta["num_q_tiles"]) > 0 and k_buffer.dtype == torch.bfloat16
            and hd == 128 and prefill_heads % n_kv == 0 and (prefill_heads // n_kv) % 4 == 0):
        units, pairs = prefill_plan(meta, prefill_heads, num_cus)
        c.prefill_units = up(units)
        c.num_prefill_pairs = pairs
        need = prefill_workspace_bytes(pairs, prefill_heads, hd)
        if need > 0:
            if prefill_workspace is not None and prefill_workspace.numel() * prefill_workspace.element_size() >= need:
                c.prefill_workspace = prefill_workspace
            else:
                c.prefill_workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
    return c


def _meta(c: KVCache, need_prefill: bool = False) -> KvMeta:
    kb, vb = c.k_buffer, c.v_buffer
    _need(kb.dim() == 4 and kb.shape == vb.shape, "k_buffer/v_buffer must be equal 4-d tensors")
    _need(kb.dtype in _DTYPES and vb.dtype == kb.dtype, "pool dtype must be float32 or bfloat16")
    _dev_tensor(kb, "k_buffer")
    _dev_tensor(vb, "v_buffer", device=kb.device)
    b = c.batch
    _dev_tensor(c.req_to_token, "req_to_token", torch.int32, kb.device)
    _need(c.req_to_token.dim() == 2, "req_to_token must be [num_reqs, max_ctx_len]")
    _dev_tensor(c.req_pool_indices, "req_pool_indices", torch.int32, kb.device)
    _dev_tensor(c.kv_indptr, "kv_indptr", torch.int32, kb.device, b + 1)
    m = KvMeta()
    m.k_buffer, m.v_buffer = kb.data_ptr(), vb.data_ptr()
    m.n_layers, m.pool_slots, m.n_kv_heads, m.head_dim = (int(x) for x in kb.shape)
    m.kv_dtype = _DTYPES[kb.dtype]
    m.req_to_token = c.req_to_token.data_ptr()
    m.num_reqs, m.max_ctx_len = (int(x) for x in c.req_to_token.shape)
    m.req_pool_indices = c.req_pool_indices.data_ptr()
    m.kv_indptr = c.kv_indptr.data_ptr()
    m.batch, m.max_len = b, int(c.max_len)
    if c.num_split_items > 0:
        _dev_tensor(c.split_item_batch, "split_item_batch", torch.int32, kb.device, c.num_split_items)
        _dev_tensor(c.split_item_index, "split_item_index", torch.int32, kb.device, c.num_split_items)
        m.split_item_batch = c.split_item_batch.data_ptr()
        m.split_item_index = c.split_item_index.data_ptr()
        m.num_split_items, m.split_item_chunk = int(c.num_split_items), int(c.split_item_chunk)
    if need_prefill and c.prefill_units is not None:
        _dev_tensor(c.prefill_units, "prefill_units", torch.int32, kb.device)
        _need(c.prefill_units.dim() == 2 and c.prefill_units.shape[1] == 8, "prefill_units must be [n, 8]")
        m.prefill_units = c.prefill_units.data_ptr()
        m.num_prefill_units, m.num_prefill_pairs = int(c.prefill_units.shape[0]), int(c.num_prefill_pairs)
        if c.prefill_workspace is not None:
            _dev_tensor(c.prefill_workspace, "prefill_workspace", device=kb.device)
            m.prefill_workspace = c.prefill_workspace.data_ptr()
            m.prefill_workspace_bytes = c.prefill_workspace.numel() * c.prefill_workspace.element_size()
    if need_prefill:
        _dev_tensor(c.qo_indptr, "qo_indptr", torch.int32, kb.device, b + 1)
        _dev_tensor(c.q_tile_to_batch, "q_tile_to_batch", torch.int32, kb.device, c.num_q_tiles)
        _dev_tensor(c.q_tile_to_index, "q_tile_to_index", torch.int32, kb.device, c.num_q_tiles)
        m.qo_indptr = c.qo_indptr.data_ptr()
        m.q_tile_to_batch = c.q_tile_to_batch.data_ptr()
        m.q_tile_to_index = c.q_tile_to_index.data_ptr()
        m.num_q_tiles, m.q_tile = int(c.num_q_tiles), int(c.q_tile)
    return m


# ---------------------------------------------------------------------------
# device calls
# ---------------------------------------------------------------------------

def rope_table(max_pos: int, head_dim: int, theta: float = 10000.0, device="cuda") -> torch.Tensor:
    """freqs_cis [max_pos, head_dim/2, 2] float32 of [cos, sin] (astr_rope_table)."""
    t = torch.empty((max_pos, head_dim // 2, 2), dtype=torch.float32, device=device)
    check(lib().astr_rope_table(_vp(t), int(max_pos), int(head_dim), float(theta), _stream(t)))
    return t


def rope_kv_write(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, positions: torch.Tensor,
                  out_cache_loc: torch.Tensor, freqs_cis: torch.Tensor, cache: KVCache,
                  layer_id: int) -> torch.Tensor:
    """Rotate q (in place) and k, write rotated k and v into the pool (astr_rope_kv_write)."""
    kb = cache.k_buffer
    n_layers, pool_slots, n_kv, d = kb.shape
    _need(q.dim() == 3 and q.shape[2] == d, "q must be [tokens, n_heads, head_dim]")
    t = int(q.shape[0])
    _dev_tensor(q, "q", kb.dtype, kb.device)
    _dev_tensor(k, "k", kb.dtype, kb.device)
    _dev_tensor(v, "v", kb.dtype, kb.device)
    _need(tuple(k.shape) == (t, n_kv, d) and tuple(v.shape) == (t, n_kv, d),
          "k and v must be [tokens, n_kv_heads, head_dim]")
    _dev_tensor(positions, "positions", torch.int32, kb.device, t)
    _dev_tensor(out_cache_loc, "out_cache_loc", torch.int32, kb.device, t)
    _dev_tensor(freqs_cis, "freqs_cis", torch.float32, kb.device)
    _need(freqs_cis.dim() == 3 and tuple(freqs_cis.shape[1:]) == (d // 2, 2),
          "freqs_cis must be [max_pos, head_dim/2, 2]")
    m = KvMeta()
    m.k_buffer, m.v_buffer = kb.data_ptr(), cache.v_buffer.data_ptr()
    m.n_layers, m.pool_slots, m.n_kv_heads, m.head_dim = n_layers, pool_slots, n_kv, d
    m.kv_dtype = _DTYPES[kb.dtype]
    check(lib().astr_rope_kv_write(_vp(q), _vp(k), _vp(v), _vp(positions), _vp(out_cache_loc), t,
                                   int(q.shape[1]), _vp(freqs_cis), int(freqs_cis.shape[0]),
                                   ctypes.byref(m), int(layer_id), _DTYPES[q.dtype], _stream(q)))
    return q


def rope_backward(grad: torch.Tensor, positions: torch.Tensor, freqs_cis: torch.Tensor) -> torch.Tensor:
    """Gradient of the rotation, in place (astr_rope_backward): grad [tokens, heads, head_dim]
    of the rotated tensor becomes the gradient of the unrotated one."""
    _need(grad.dim() == 3, "grad must be [tokens, n_heads, head_dim]")
    _need(grad.dtype in _DTYPES, "grad must be float32 or bfloat16")
    t, h, d = (int(x) for x in grad.shape)
    _dev_tensor(grad, "grad", grad.dtype, grad.device)
    _dev_tensor(positions, "positions", torch.int32, grad.device, t)
    _dev_tensor(freqs_cis, "freqs_cis", torch.float32, grad.device)
    _need(freqs_cis.dim() == 3 and tuple(freqs_cis.shape[1:]) == (d // 2, 2),
          "freqs_cis must be [max_pos, head_dim/2, 2]")
    check(lib().astr_rope_backward(_vp(grad), _vp(positions), t, h, d, _vp(freqs_cis),
                                   int(freqs_cis.shape[0]), _DTYPES[grad.dtype], _stream(grad)))
    return grad


def decode_num_splits(max_len: int, split_chunk: int) -> int:
    return int(lib().astr_decode_num_splits(int(max_len), int(split_chunk)))


def decode_workspace_bytes(batch: int, n_heads: int, head_dim: int, max_len: int, split_chunk: int) -> int:
    """Bytes of the split-K scratch (o_part then lse_part) of one decode call
    (astr_decode_workspace_bytes); 0 when one split covers max_len."""
    return int(lib().astr_decode_workspace_bytes(int(batch), int(n_heads), int(head_dim), int(max_len),
                                                 int(split_chunk)))


def decode_workspace(cache: KVCache, n_heads: int, split_chunk: int):
    """(o_part [B, H, S, D], lse_part [B, H, S]) float32 for astr_decode_attn,
    carved from one allocation of astr_decode_workspace_bytes (None, None
    when one split covers max_len and no scratch is used)."""
    d = int(cache.k_buffer.shape[3])
    b = cache.batch
    nbytes = decode_workspace_bytes(b, n_heads, d, cache.max_len, split_chunk)
    if nbytes == 0:
        return None, None
    s = decode_num_splits(cache.max_len, split_chunk)
    rows = b * n_heads * s
    _need(nbytes == 4 * rows * (d + 1), "decode workspace size disagrees with its layout")
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device=cache.k_buffer.device)
    return ws[:rows * d].view(b, n_heads, s, d), ws[rows * d:].view(b, n_heads, s)


def decode_attn(q: torch.Tensor, cache: KVCache, layer_id: int, split_chunk: int,
                sm_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                o_part: Optional[torch.Tensor] = None,
                lse_part: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Split-K paged decode attention (astr_decode_attn); q [B, H, D] rotated."""
    m = _meta(cache)
    kb = cache.k_buffer
    b, d = cache.batch, int(kb.shape[3])
    _need(q.dim() == 3 and q.shape[0] == b and q.shape[2] == d, "q must be [batch, n_heads, head_dim]")
    h = int(q.shape[1])
    _dev_tensor(q, "q", kb.dtype, kb.device)
    if out is None:
        out = torch.empty_like(q)
    _dev_tensor(out, "out", kb.dtype, kb.device, q.numel())
    s = decode_num_splits(cache.max_len, split_chunk)
    if s > 1:
        if o_part is None or lse_part is None:
            o_part, lse_part = decode_workspace(cache, h, split_chunk)
        _dev_tensor(o_part, "o_part", torch.float32, kb.device, b * h * s * d)
        _dev_tensor(lse_part, "lse_part", torch.float32, kb.device, b * h * s)
    check(lib().astr_decode_attn(_vp(q), h, ctypes.byref(m), int(layer_id), int(split_chunk), float(sm_scale),
                                 _vp(o_part) if s > 1 else None, _vp(lse_part) if s > 1 else None,
                                 _vp(out), _DTYPES[q.dtype], _stream(q)))
    return out


def decode_attn_noalloc(q: torch.Tensor, cache: KVCache, layer_id: int, split_chunk: int,
                        sm_scale: float = 0.0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """decode_attn with the split-K scratch in the library's static device array
    (astr_decode_attn_noalloc): the call allocates nothing when out is given."""
    m = _meta(cache)
    kb = cache.k_buffer
    b, d = cache.batch, int(kb.shape[3])
    _need(q.dim() == 3 and q.shape[0] == b and q.shape[2] == d, "q must be [batch, n_heads, head_dim]")
    _dev_tensor(q, "q", kb.dtype, kb.device)
    if out is None:
        out = torch.empty_like(q)
    _dev_tensor(out, "out", kb.dtype, kb.device, q.numel())
    check(lib().astr_decode_attn_noalloc(_vp(q), int(q.shape[1]), ctypes.byref(m), int(layer_id), int(split_chunk),
                                         float(sm_scale), _vp(out), _DTYPES[q.dtype], _stream(q)))
    return out


def decode_attn_write(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, cache: KVCache,
                      layer_id: int, freqs_cis: torch.Tensor, split_chunk: int, sm_scale: float = 0.0,
                      out: Optional[torch.Tensor] = None, o_part: Optional[torch.Tensor] = None,
                      lse_part: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode with the rotary write of the new token fused in (astr_decode_attn_write):
    q [B, H, D] and k_new/v_new [B, Hkv, D] unrotated; the new token sits at position L_b - 1."""
    m = _meta(cache)
    kb = cache.k_buffer
    b, n_kv, d = cache.batch, int(kb.shape[2]), int(kb.shape[3])
    _need(q.dim() == 3 and q.shape[0] == b and q.shape[2] == d, "q must be [batch, n_heads, head_dim]")
    h = int(q.shape[1])
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new)):
        _dev_tensor(t, name, kb.dtype, kb.device)
    _need(tuple(k_new.shape) == (b, n_kv, d) and tuple(v_new.shape) == (b, n_kv, d),
          "k_new and v_new must be [batch, n_kv_heads, head_dim]")
    _dev_tensor(freqs_cis, "freqs_cis", torch.float32, kb.device)
    _need(freqs_cis.dim() == 3 and tuple(freqs_cis.shape[1:]) == (d // 2, 2),
          "freqs_cis must be [max_pos, head_dim/2, 2]")
    if out is None:
        out = torch.empty_like(q)
    _dev_tensor(out, "out", kb.dtype, kb.device, q.numel())
    s = decode_num_splits(cache.max_len, split_chunk)
    if s > 1:
        if o_part is None or lse_part is None:
            o_part, lse_part = decode_workspace(cache, h, split_chunk)
        _dev_tensor(o_part, "o_part", torch.float32, kb.device, b * h * s * d)
        _dev_tensor(lse_part, "lse_part", torch.float32, kb.device, b * h * s)
    check(lib().astr_decode_attn_write(_vp(q), _vp(k_new), _vp(v_new), h, ctypes.byref(m),
                                       int(layer_id), _vp(freqs_cis), int(freqs_cis.shape[0]),
                                       int(split_chunk), float(sm_scale),
                                       _vp(o_part) if s > 1 else None, _vp(lse_part) if s > 1 else None,
                                       _vp(out), _DTYPES[q.dtype], _stream(q)))
    return out


def prefill_attn(q: torch.Tensor, cache: KVCache, layer_id: int, sm_scale: float = 0.0,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Ragged causal prefill (astr_prefill_attn); q [sum e_b, H, D] rotated, qo order."""
    m = _meta(cache, need_prefill=True)
    kb = cache.k_buffer
    d = int(kb.shape[3])
    _need(q.dim() == 3 and q.shape[2] == d, "q must be [tokens, n_heads, head_dim]")
    _dev_tensor(q, "q", kb.dtype, kb.device)
    if out is None:
        out = torch.empty_like(q)
    _dev_tensor(out, "out", kb.dtype, kb.device, q.numel())
    check(lib().astr_prefill_attn(_vp(q), int(q.shape[0]), int(q.shape[1]), ctypes.byref(m), int(layer_id),
                                  float(sm_scale), _vp(out), _DTYPES[q.dtype], _stream(q)))
    return out


# ---------------------------------------------------------------------------
# attainable-rate probes (include/astr_ceiling.h)
# ---------------------------------------------------------------------------

def ceiling_stream_read(buf: torch.Tensor, workgroups: int = 2048, nontemporal: bool = True,
                        sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Read every byte of buf once (astr_ceiling_stream_read); returns the sink."""
    _dev_tensor(buf, "buf")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(workgroups, dtype=torch.int32, device=buf.device)
    _dev_tensor(sink, "sink", torch.int32, buf.device, workgroups)
    check(lib().astr_ceiling_stream_read(_vp(buf), nbytes, int(workgroups), int(bool(nontemporal)), _vp(sink),
                                         _stream(buf)))
    return sink


def ceiling_mfma_loop(workgroups: int, iters: int, sink: torch.Tensor) -> int:
    """Run the matrix-core loop (astr_ceiling_mfma_loop); returns its flop count."""
    _dev_tensor(sink, "sink", torch.float32, None, 256 * workgroups)
    check(lib().astr_ceiling_mfma_loop(int(workgroups), int(iters), _vp(sink), _stream(sink)))
    return 2 * 16 * 16 * 32 * 8 * int(iters) * 4 * int(workgroups)


# ---------------------------------------------------------------------------
# the host page-table builder
# ---------------------------------------------------------------------------

def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class PagePool:
    """Host page-table builder (astr_pagepool_*): contiguous or paged slots,
    bitmask allocation with reference counts, exact page-aligned radix reuse."""

    def __init__(self, mode: int, pool_slots: int, page_size: int, max_reqs: int,
                 max_ctx_len: int, page_perm=None):
        self._h = ctypes.c_void_p()
        perm = None if page_perm is None else _i32(page_perm)
        if perm is not None and mode == 1:
            _need(perm.size == pool_slots // page_size, "page_perm needs one entry per page")
        check(lib().astr_pagepool_create(ctypes.byref(self._h), int(mode), int(pool_slots),
                                         int(page_size), int(max_reqs), int(max_ctx_len),
                                         None if perm is None else _i32p(perm)))
        self.mode, self.pool_slots, self.page_size = mode, pool_slots, page_size
        self.max_reqs, self.max_ctx_len = max_reqs, max_ctx_len

    def close(self):
        if self._h:
            lib().astr_pagepool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def admit(self, tokens=None, n_tokens: Optional[int] = None):
        tok = None if tokens is None else _i32(tokens)
        n = int(n_tokens if n_tokens is not None else (0 if tok is None else tok.size))
        if tok is not None:
            _need(tok.size >= n, "tokens shorter than n_tokens")
        r, c = ctypes.c_int(), ctypes.c_int()
        check(lib().astr_pagepool_admit(self._h, None if tok is None else _i32p(tok), n,
                                        ctypes.byref(r), ctypes.byref(c)))
        return r.value, c.value

    def extend(self, req: int, n_new: int):
        check(lib().astr_pagepool_extend(self._h, int(req), int(n_new)))

    def bind(self, reqs, q_lens, q_tile: int = 64) -> dict:
        reqs, q_lens = _i32(reqs), _i32(q_lens)
        _need(reqs.size == q_lens.size, "reqs and q_lens differ in length")
        b = int(reqs.size)
        total = int(q_lens.sum())
        cap = int(sum(-(-int(x) // q_tile) for x in q_lens)) if q_tile > 0 else 0
        seq = np.zeros(b, np.int32)
        loc = np.zeros(max(total, 1), np.int32)
        kv = np.zeros(b + 1, np.int32)
        qo = np.zeros(b + 1, np.int32)
        t2b = np.zeros(max(cap, 1), np.int32)
        t2i = np.zeros(max(cap, 1), np.int32)
        nt, ml = ctypes.c_int(), ctypes.c_int()
        check(lib().astr_pagepool_bind(self._h, _i32p(reqs), _i32p(q_lens), b, int(q_tile),
                                       _i32p(seq), _i32p(loc), _i32p(kv), _i32p(qo), _i32p(t2b),
                                       _i32p(t2i), max(cap, 1), ctypes.byref(nt), ctypes.byref(ml)))
        return dict(req_pool_indices=reqs, seq_lens=seq, out_cache_loc=loc[:total], kv_indptr=kv,
                    qo_indptr=qo, q_tile_to_batch=t2b[:nt.value], q_tile_to_index=t2i[:nt.value],
                    num_q_tiles=nt.value, max_len=ml.value, q_tile=int(q_tile))

    def insert(self, req: int, tokens, n_materialized: int):
        tok = _i32(tokens)
        _need(tok.size >= n_materialized, "tokens shorter than n_materialized")
        check(lib().astr_pagepool_insert(self._h, int(req), _i32p(tok), int(n_materialized)))

    def release(self, req: int):
        check(lib().astr_pagepool_release(self._h, int(req)))

    def complete(self, req: int, tokens, n_tokens: Optional[int] = None):
        """Finish a request: cache the complete pages of tokens[:n_tokens - 1]
        (the final sampled token has no KV) and release it."""
        tok = _i32(tokens)
        n = int(tok.size if n_tokens is None else n_tokens)
        _need(0 <= n <= tok.size, "n_tokens outside the tokens given")
        check(lib().astr_pagepool_complete(self._h, int(req), _i32p(tok) if tok.size else None, n))

    def evict(self, n_pages: int) -> int:
        """Free up to n_pages cached pages, least recently used first."""
        n = int(lib().astr_pagepool_evict(self._h, int(n_pages)))
        if n < 0:
            check(ASTR_E_INVAL)
        return n

    def cached_pages(self) -> int:
        return int(lib().astr_pagepool_cached_pages(self._h))

    def evicted_pages(self) -> int:
        return int(lib().astr_pagepool_evicted_pages(self._h))

    def table(self) -> np.ndarray:
        """A copy of the host table [max_reqs, max_ctx_len] int32."""
        p = lib().astr_pagepool_table(self._h)
        n = self.max_reqs * self.max_ctx_len
        return np.ctypeslib.as_array(p, shape=(n,)).reshape(self.max_reqs, self.max_ctx_len).copy()

    def free_pages(self) -> int:
        return int(lib().astr_pagepool_free_pages(self._h))

    def page_ref(self, logical_page: int) -> int:
        return int(lib().astr_pagepool_page_ref(self._h, int(logical_page)))
