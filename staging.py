"""Stage a synthetic workload on the GPU through the library.

Used by the GPU tests and by bench.py.  It builds the page tables with the
library's PagePool, allocates the pool with torch, places the history KV
drawn by ``workloads`` at the slots the tables give (history stands for cache
contents written by earlier steps), uploads the new tokens' q/k/v, and runs
the path's calls: rope_kv_write, decode_attn, prefill_attn.  A prefill step
carries the library's work plan unless plan=False.  Nothing here computes
attention or rotation itself.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

import paged_gqa_attention_rope_amd as astr
from workloads import Case

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class Staged:
    cs: Case
    pool: astr.PagePool
    reqs: list
    cached: list
    k_buffer: torch.Tensor
    v_buffer: torch.Tensor
    freqs: torch.Tensor
    write_meta: dict                    # host metadata of the rotary write step
    write_cache: astr.KVCache
    q: torch.Tensor                     # [n_new, Hq, D] new tokens (rotated in place by the write)
    k: torch.Tensor
    v: torch.Tensor
    positions: torch.Tensor             # [n_new] int32
    attn_cache: Optional[astr.KVCache] = None   # decode: one query per request
    attn_meta: Optional[dict] = None
    q_index: Optional[torch.Tensor] = None      # decode: row of q used by each request
    extra: dict = field(default_factory=dict)


def _to_dev(a: np.ndarray, dtype, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)


def build_tables(cs: Case):
    """Run the case's admissions on the library's PagePool (radix warm-up first)."""
    extra = 4 if cs.group_tokens is not None else 0
    pp = astr.PagePool(cs.mode, cs.pool_slots, cs.page_size, cs.max_reqs + extra, cs.max_ctx_len,
                       cs.page_perm)
    warm = []
    if cs.group_tokens is not None:
        for g, toks in enumerate(cs.group_tokens):
            if len(toks) == 0:
                continue
            r, c = pp.admit(toks, len(toks))
            pp.extend(r, len(toks) - c)
            warm.append((g, r))
    reqs, cached = [], []
    return pp, warm, reqs, cached


def stage(cs: Case, device="cuda", canary: bool = True, threads: int = 16, plan: bool = True) -> Staged:
    dev = torch.device(device)
    dt = TORCH_DTYPE[cs.dtype]
    pp, warm, reqs, cached = build_tables(cs)
    shape = (cs.n_layers, cs.pool_slots, cs.n_kv_heads, cs.head_dim)
    fill = float("nan") if canary else 0.0
    k_buffer = torch.full(shape, fill, dtype=dt, device=dev)
    v_buffer = torch.full(shape, fill, dtype=dt, device=dev)
    L = cs.layer_id

    def place(slots: np.ndarray, kh: np.ndarray, vh: np.ndarray):
        if len(slots) == 0:
            return
        idx = _to_dev(slots.astype(np.int64), torch.int64, dev)
        k_buffer[L].index_copy_(0, idx, _to_dev(kh, dt, dev))
        v_buffer[L].index_copy_(0, idx, _to_dev(vh, dt, dev))

    # prefix groups: materialise each group's prefix, publish its pages, release
    if warm:
        tab = pp.table()
        for g, r in warm:
            kh, vh = cs.group_history(g)
            place(tab[r, :len(kh)], kh, vh)
            pp.insert(r, cs.group_tokens[g], len(cs.group_tokens[g]))
            pp.release(r)
    for b in range(cs.batch):
        if cs.tokens is not None:
            r, c = pp.admit(cs.tokens[b], len(cs.tokens[b]))
        else:
            r, c = pp.admit(None, 0)
        pp.extend(r, int(cs.seq_lens[b]) - c)
        reqs.append(r)
        cached.append(c)
    table = pp.table()
    if cs._hist is not None:
        # decode history, generated per request in parallel, placed per request
        def gen(b):
            return b, cs.history(b)
        with ThreadPoolExecutor(max_workers=threads) as ex:
            for lo in range(0, cs.batch, 2 * threads):          # bounded host memory
                for b, (kh, vh) in ex.map(gen, range(lo, min(cs.batch, lo + 2 * threads))):
                    place(table[reqs[b], :len(kh)], kh, vh)
                    del kh, vh
    wmeta = pp.bind(reqs, cs.new_lens, cs.q_tile or 64)
    wcache = astr.cache_from_bind(k_buffer, v_buffer, table, wmeta,
                                  prefill_heads=cs.n_heads if cs.kind == "prefill" and plan else None)
    pos = np.concatenate([np.arange(int(s) - int(n), int(s)) for s, n in zip(cs.seq_lens, cs.new_lens)])
    st = Staged(cs=cs, pool=pp, reqs=reqs, cached=cached, k_buffer=k_buffer, v_buffer=v_buffer,
                freqs=astr.rope_table(cs.max_ctx_len, cs.head_dim, cs.theta, dev),
                write_meta=wmeta, write_cache=wcache, q=_to_dev(cs.q, dt, dev),
                k=_to_dev(cs.k, dt, dev), v=_to_dev(cs.v, dt, dev),
                positions=_to_dev(pos.astype(np.int32), torch.int32, dev))
    if cs.kind == "decode":
        ameta = pp.bind(reqs, np.ones(cs.batch, dtype=np.int32), 64)
        st.attn_meta = ameta
        st.attn_cache = astr.cache_from_bind(k_buffer, v_buffer, table, ameta, split_chunk=cs.split_chunk)
        last = wmeta["qo_indptr"][1:] - 1
        st.q_index = _to_dev(last.astype(np.int64), torch.int64, dev)
    else:
        st.attn_meta = wmeta
        st.attn_cache = wcache
    return st


def run_write(st: Staged):
    astr.rope_kv_write(st.q, st.k, st.v, st.positions, st.write_cache.out_cache_loc, st.freqs,
                       st.write_cache, st.cs.layer_id)


def decode_query(st: Staged) -> torch.Tensor:
    """The rotated query of each request's newest token, [B, Hq, D]."""
    if st.q.shape[0] == st.cs.batch:          # one new token per request: q is already [B, Hq, D]
        return st.q
    return st.q.index_select(0, st.q_index).contiguous()


def run_decode(st: Staged, q_dec: Optional[torch.Tensor] = None, out=None, o_part=None,
               lse_part=None) -> torch.Tensor:
    if q_dec is None:
        q_dec = decode_query(st)
    return astr.decode_attn(q_dec, st.attn_cache, st.cs.layer_id, st.cs.split_chunk, out=out,
                            o_part=o_part, lse_part=lse_part)


def run_prefill(st: Staged, out=None) -> torch.Tensor:
    return astr.prefill_attn(st.q, st.attn_cache, st.cs.layer_id, out=out)
