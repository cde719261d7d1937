"""Seeded input generators for the five paged-attention workloads.

Every value comes from ``numpy.random.default_rng`` (PCG64).  Draw order inside
one case: lengths (and prefix groups) -> token ids -> page permutation ->
q -> k -> v of the new tokens -> layer id.  History KV (cache contents that
precede this step) comes from separate per-request (decode) or per-group
(prefix prefill) streams seeded with ``[seed, 7, index]`` so that one
request's history can be regenerated alone.

Values are N(0, 1) float32; for bf16 workloads they are rounded to the nearest
bf16 (ties to even) and returned as float32 arrays whose values are exactly
representable in bf16, so both consumers read identical stored inputs.
History KV stands for already-rotated cache contents: it is placed in the pool
as drawn.

Nothing here computes a rotation, an attention output or a page table.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np

CASE_IDS = (1, 2, 3, 4, 5)
ROPE_THETA = 10000.0


def bf16_storage(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    out = ((bits + bias) >> np.uint32(16)) << np.uint32(16)
    return out.astype(np.uint32).view(np.float32)


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    return bf16_storage(x) if dtype == "bf16" else x


@dataclass
class Case:
    """One batch of synthetic input for one step of the attention path."""

    case_id: int
    seed: int
    name: str
    kind: str                 # "decode" or "prefill"
    dtype: str                # "f32" or "bf16" (activations and KV pool)
    mode: int                 # 0 contiguous, 1 paged
    page_size: int
    pool_slots: int
    n_layers: int
    layer_id: int
    max_reqs: int
    max_ctx_len: int
    batch: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    theta: float
    split_chunk: int          # decode: KV positions per split (0 for prefill)
    q_tile: int               # prefill: query rows per tile
    seq_lens: np.ndarray      # [B] KV length of each request after this step
    new_lens: np.ndarray      # [B] tokens rotated and written this step
    prefix_lens: np.ndarray   # [B] expected cached (radix) prefix length
    q: np.ndarray             # [sum(new_lens), n_heads, D] float32, pre-rotation
    k: np.ndarray             # [sum(new_lens), n_kv_heads, D] float32, pre-rotation
    v: np.ndarray             # [sum(new_lens), n_kv_heads, D] float32
    page_perm: Optional[np.ndarray] = None      # logical page -> physical page
    tokens: Optional[list] = None               # per-request prompt token ids
    group_of: Optional[np.ndarray] = None       # [B] prefix group of each request
    group_tokens: Optional[list] = None         # per-group prefix token ids
    _hist: Optional[Callable] = field(default=None, repr=False)
    _group_hist: Optional[Callable] = field(default=None, repr=False)

    # -- derived sizes (no method arithmetic: bookkeeping of the draw) ------
    @property
    def hist_lens(self) -> np.ndarray:
        return self.seq_lens - self.new_lens

    @property
    def n_new(self) -> int:
        return int(self.new_lens.sum())

    def history(self, b: int):
        """(K, V) float32 [hist_len_b, n_kv_heads, D] for request ``b``."""
        return self._hist(b)

    def group_history(self, g: int):
        """(K, V) float32 [len(group_tokens[g]), n_kv_heads, D] for prefix group ``g``."""
        return self._group_hist(g)


def _hist_stream(seed: int, idx: int, n: int, hkv: int, d: int, dtype: str):
    rng = np.random.default_rng([seed, 7, idx])
    kh = _normal(rng, (n, hkv, d), dtype)
    vh = _normal(rng, (n, hkv, d), dtype)
    return kh, vh


def decode_case(seed: int, *, case_id: int = 0, name: str = "decode",
                batch: int, n_heads: int, n_kv_heads: int, head_dim: int,
                dtype: str, mode: int, page_size: int, split_chunk: int,
                n_layers: int = 1, random_layer: bool = False,
                lens: Optional[list] = None, len_lo: int = 1, len_hi: int = 1,
                log_uniform: bool = False, max_ctx_len: int = 0,
                pool_slots: int = 0, shuffle_pages: bool = False,
                all_new: bool = False) -> Case:
    """A decode step: each request appends one token (or, with ``all_new``,
    writes every position through the rotary write) and attends over its
    whole KV range with one query."""
    rng = np.random.default_rng(seed)
    if lens is not None:
        seq = np.asarray(lens, dtype=np.int64)
    elif log_uniform:
        u = rng.uniform(np.log(len_lo), np.log(len_hi), size=batch)
        seq = np.floor(np.exp(u)).astype(np.int64)
    else:
        seq = rng.integers(len_lo, len_hi, size=batch, endpoint=True).astype(np.int64)
    batch = len(seq)
    if max_ctx_len <= 0:
        max_ctx_len = int(seq.max())
    if mode == 0:
        pool_slots = batch * max_ctx_len
        n_pages = pool_slots
    else:
        if pool_slots <= 0:
            pages_needed = int(sum((int(s) + page_size - 1) // page_size for s in seq))
            pool_slots = pages_needed * page_size
        n_pages = pool_slots // page_size
    perm = rng.permutation(n_pages).astype(np.int32) if (mode == 1 and shuffle_pages) else None
    new = seq.copy() if all_new else np.ones(batch, dtype=np.int64)
    t = int(new.sum())
    q = _normal(rng, (t, n_heads, head_dim), dtype)
    k = _normal(rng, (t, n_kv_heads, head_dim), dtype)
    v = _normal(rng, (t, n_kv_heads, head_dim), dtype)
    layer_id = int(rng.integers(0, n_layers)) if random_layer else 0
    hist = seq - new

    def _h(b: int):
        return _hist_stream(seed, b, int(hist[b]), n_kv_heads, head_dim, dtype)

    return Case(case_id=case_id, seed=seed, name=name, kind="decode", dtype=dtype,
                mode=mode, page_size=page_size, pool_slots=int(pool_slots),
                n_layers=n_layers, layer_id=layer_id, max_reqs=batch,
                max_ctx_len=int(max_ctx_len), batch=batch, n_heads=n_heads,
                n_kv_heads=n_kv_heads, head_dim=head_dim, theta=ROPE_THETA,
                split_chunk=split_chunk, q_tile=0, seq_lens=seq, new_lens=new,
                prefix_lens=np.zeros(batch, dtype=np.int64), q=q, k=k, v=v,
                page_perm=perm, _hist=_h)


def prefill_case(seed: int, *, case_id: int = 0, name: str = "prefill",
                 batch: int, n_heads: int, n_kv_heads: int, head_dim: int,
                 dtype: str, mode: int, page_size: int, q_tile: int,
                 ext_lo: int, ext_hi: int, max_ctx_len: int = 0,
                 pool_slots: int = 0, n_groups: int = 0,
                 prefix_pages_hi: int = 0, shuffle_pages: bool = False,
                 n_layers: int = 1) -> Case:
    """A prefill step over ragged extend lengths, optionally behind a cached
    page-aligned prefix shared by requests of the same prefix group."""
    rng = np.random.default_rng(seed)
    ext = rng.integers(ext_lo, ext_hi, size=batch, endpoint=True).astype(np.int64)
    if n_groups > 0:
        group_of = rng.integers(0, n_groups, size=batch).astype(np.int64)
        pre = page_size * rng.integers(0, prefix_pages_hi, size=batch, endpoint=True).astype(np.int64)
    else:
        group_of = None
        pre = np.zeros(batch, dtype=np.int64)
    seq = pre + ext
    if max_ctx_len <= 0:
        max_ctx_len = int(seq.max())
    # token ids: prefix groups draw from [0, 50000), extends from [50000, 100000),
    # so a prefix lookup can never run into the extend part.
    tokens = group_tokens = None
    if n_groups > 0:
        glen = [int(pre[group_of == g].max()) if np.any(group_of == g) else 0
                for g in range(n_groups)]
        group_tokens = [rng.integers(0, 50000, size=gl).astype(np.int32) for gl in glen]
        tokens = []
        for b in range(batch):
            ext_tok = rng.integers(50000, 100000, size=int(ext[b])).astype(np.int32)
            tokens.append(np.concatenate([group_tokens[group_of[b]][: pre[b]], ext_tok]))
    if mode == 0:
        pool_slots = batch * max_ctx_len
        n_pages = pool_slots
    else:
        n_pages = pool_slots // page_size
    perm = rng.permutation(n_pages).astype(np.int32) if (mode == 1 and shuffle_pages) else None
    t = int(ext.sum())
    q = _normal(rng, (t, n_heads, head_dim), dtype)
    k = _normal(rng, (t, n_kv_heads, head_dim), dtype)
    v = _normal(rng, (t, n_kv_heads, head_dim), dtype)

    def _gh(g: int):
        return _hist_stream(seed, g, len(group_tokens[g]), n_kv_heads, head_dim, dtype)

    return Case(case_id=case_id, seed=seed, name=name, kind="prefill", dtype=dtype,
                mode=mode, page_size=page_size, pool_slots=int(pool_slots),
                n_layers=n_layers, layer_id=0, max_reqs=batch,
                max_ctx_len=int(max_ctx_len), batch=batch, n_heads=n_heads,
                n_kv_heads=n_kv_heads, head_dim=head_dim, theta=ROPE_THETA,
                split_chunk=0, q_tile=q_tile, seq_lens=seq, new_lens=ext,
                prefix_lens=pre, q=q, k=k, v=v, page_perm=perm, tokens=tokens,
                group_of=group_of, group_tokens=group_tokens,
                _group_hist=_gh if n_groups > 0 else None)


def make_case(case_id: int, seed: Optional[int] = None) -> Case:
    """The five workloads at their full sizes (seed defaults to the case id)."""
    s = case_id if seed is None else seed
    if case_id == 1:
        # contiguous, fp32, every position goes through the rotary write
        return decode_case(s, case_id=1, name="decode-contig-fp32-b2-h4kv2-d64",
                           batch=2, n_heads=4, n_kv_heads=2, head_dim=64, dtype="f32",
                           mode=0, page_size=1, split_chunk=16, lens=[17, 33],
                           max_ctx_len=64, all_new=True)
    if case_id == 2:
        return decode_case(s, case_id=2, name="decode-page1-bf16-b8-h16kv4-d128",
                           batch=8, n_heads=16, n_kv_heads=4, head_dim=128, dtype="bf16",
                           mode=1, page_size=1, split_chunk=256, len_lo=128, len_hi=2048,
                           max_ctx_len=2048, pool_slots=65536, shuffle_pages=True)
    if case_id == 3:
        return prefill_case(s, case_id=3, name="prefill-contig-bf16-b4-h16kv4-d128",
                            batch=4, n_heads=16, n_kv_heads=4, head_dim=128, dtype="bf16",
                            mode=0, page_size=1, q_tile=64, ext_lo=64, ext_hi=1024,
                            max_ctx_len=1024)
    if case_id == 4:
        return prefill_case(s, case_id=4, name="prefill-radix-page16-bf16-b16-h16kv4-d128",
                            batch=16, n_heads=16, n_kv_heads=4, head_dim=128, dtype="bf16",
                            mode=1, page_size=16, q_tile=64, ext_lo=32, ext_hi=512,
                            max_ctx_len=2048 + 512, pool_slots=65536, n_groups=4,
                            prefix_pages_hi=128)
    if case_id == 5:
        return decode_case(s, case_id=5, name="decode-page16-bf16-b256-h16kv4-d128-l24",
                           batch=256, n_heads=16, n_kv_heads=4, head_dim=128, dtype="bf16",
                           mode=1, page_size=16, split_chunk=512, len_lo=1024,
                           len_hi=32768, log_uniform=True, max_ctx_len=32768,
                           shuffle_pages=True, n_layers=24, random_layer=True)
    raise ValueError(f"unknown case {case_id}")
