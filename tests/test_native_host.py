"""Host-side checks of libastr.so (CPU only, no device calls).

* the library loads and exports every symbol include/astr.h declares;
* the C++ page-table builder is bit-exact against the oracle's Python builder
  (AstrAI docs/guides/inference.md, "KVCache System") on the five workloads
  and several seeds, including the radix warm-up of the prefix workload;
* argument validation rejects bad calls before any launch (the kernel
  wrappers raise rather than fall back: inference.md, "Attention Backend").
"""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle.pagepool import PagePool as OraclePool, PoolError
from workloads import make_case

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from paged_gqa_attention_rope_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libastr.so not built")
    return _lib


def test_library_exports_every_declared_symbol():
    L = _lib()
    inc = os.path.join(ROOT, "include")
    declared = set()
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            declared |= set(re.findall(r"\b(astr_[a-z_0-9]+)\s*\(", open(os.path.join(inc, h)).read()))
    assert declared == set(L.EXPORTS)
    so = ctypes.CDLL(L.LIB_PATH)
    for name in declared:
        assert hasattr(so, name), name


class _Native:
    """Adapter so both builders run the same flows."""

    def __init__(self, *a):
        from paged_gqa_attention_rope_amd import PagePool
        self.p = PagePool(*a)

    def admit(self, tokens, n):
        return self.p.admit(tokens, n)

    def extend(self, r, n):
        self.p.extend(r, n)

    def insert(self, r, tokens, n):
        self.p.insert(r, tokens, n)

    def release(self, r):
        self.p.release(r)

    def bind(self, reqs, q_lens, q_tile):
        return self.p.bind(reqs, q_lens, q_tile)

    def table(self):
        return self.p.table()


class _Oracle(_Native):
    def __init__(self, *a):
        self.p = OraclePool(*a)

    def table(self):
        return self.p.table.copy()


def _flow(pool_cls, cs):
    """Admit, warm and extend the case's requests; return (pool, reqs, cached, meta)."""
    extra = 4 if cs.group_tokens is not None else 0
    pp = pool_cls(cs.mode, cs.pool_slots, cs.page_size, cs.max_reqs + extra, cs.max_ctx_len,
                  cs.page_perm)
    if cs.group_tokens is not None:
        for toks in cs.group_tokens:
            if len(toks) == 0:
                continue
            r, c = pp.admit(toks, len(toks))
            pp.extend(r, len(toks) - c)
            pp.insert(r, toks, len(toks))
            pp.release(r)
    reqs, cached = [], []
    for b in range(cs.batch):
        if cs.tokens is not None:
            r, c = pp.admit(cs.tokens[b], len(cs.tokens[b]))
        else:
            r, c = pp.admit(None, 0)
        pp.extend(r, int(cs.seq_lens[b]) - c)
        reqs.append(r)
        cached.append(c)
    q_lens = cs.new_lens if cs.kind == "prefill" else np.ones(cs.batch, dtype=np.int64)
    meta = pp.bind(reqs, q_lens, cs.q_tile or 64)
    return pp, reqs, cached, meta


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("seed_off", [0, 101])
def test_builder_bit_exact_against_oracle(cid, seed_off):
    _lib()
    cs = make_case(cid, None if seed_off == 0 else seed_off + cid)
    pn, rn, cn, mn = _flow(_Native, cs)
    po, ro, co, mo = _flow(_Oracle, cs)
    assert rn == ro and cn == co
    assert np.array_equal(cn, cs.prefix_lens)
    assert np.array_equal(pn.table(), po.table())
    for key in ("req_pool_indices", "seq_lens", "out_cache_loc", "kv_indptr", "qo_indptr"):
        assert np.array_equal(np.asarray(mn[key]), np.asarray(mo[key])), key
    assert mn["num_q_tiles"] == mo["num_q_tiles"] and mn["max_len"] == mo["max_len"]
    # the tile -> request maps are fixed, their order is not: the same set of
    # (batch entry, tile index) pairs, each once; the builder's own order is
    # checked against its stated rule in test_builder_lists_tiles_heaviest_first
    tn = list(zip(np.asarray(mn["q_tile_to_batch"]).tolist(), np.asarray(mn["q_tile_to_index"]).tolist()))
    to = list(zip(np.asarray(mo["q_tile_to_batch"]).tolist(), np.asarray(mo["q_tile_to_index"]).tolist()))
    assert len(set(tn)) == len(tn) and sorted(tn) == sorted(to)
    if cs.mode == 1:
        assert pn.p.free_pages() == sum(po.p.free)
        for page in range(0, cs.pool_slots // cs.page_size, max(1, cs.pool_slots // cs.page_size // 97)):
            assert pn.p.page_ref(page) == po.p.ref[page]


@pytest.mark.parametrize("cid", [3, 4])
@pytest.mark.parametrize("seed_off", [0, 101, 202])
def test_builder_lists_tiles_heaviest_first(cid, seed_off):
    """The library's own tile order (a scheduling choice, not part of the
    definition): by decreasing KV extent seen by the tile's last row, ties by
    batch entry, then tile index.  Stated here as a sort over the request-
    major tiles, independently of both builders."""
    _lib()
    cs = make_case(cid, None if seed_off == 0 else seed_off + cid)
    _, _, _, mn = _flow(_Native, cs)
    e = cs.new_lens.astype(int)
    p = (cs.seq_lens - cs.new_lens).astype(int)
    q_tile = cs.q_tile
    tiles = [(b, t) for b in range(cs.batch) for t in range(-(-int(e[b]) // q_tile))]
    extent = {(b, t): int(p[b] + min(q_tile * (t + 1), e[b])) for b, t in tiles}
    want = sorted(tiles, key=lambda bt: (-extent[bt], bt[0], bt[1]))
    got = list(zip(mn["q_tile_to_batch"].tolist(), mn["q_tile_to_index"].tolist()))
    assert got == want


def test_builder_lifecycle_matches_oracle():
    _lib()
    rng = np.random.default_rng(7)
    ps = 4
    pn, po = _Native(1, ps * 40, ps, 6, 64, None), _Oracle(1, ps * 40, ps, 6, 64, None)
    base = rng.integers(0, 50, size=64).astype(np.int32)
    live = []
    for step in range(60):
        op = rng.integers(0, 4)
        if op == 0 or not live:
            n = int(rng.integers(1, 40))
            toks = base.copy()
            toks[rng.integers(0, 64, size=2)] = rng.integers(0, 50, size=2)
            outs = []
            for p in (pn, po):
                try:
                    r, c = p.admit(toks, n)
                    p.extend(r, n - c)
                    outs.append((r, c))
                except Exception as e:
                    outs.append(type(getattr(e, "status", None) or getattr(e, "kind", None)).__name__)
                    if isinstance(e, PoolError) or hasattr(e, "status"):
                        outs[-1] = "err"
            assert outs[0] == outs[1], (step, outs)
            if outs[0] != "err":
                live.append((outs[0][0], toks, n))
        elif op == 1:
            r, toks, n = live.pop(int(rng.integers(0, len(live))))
            for p in (pn, po):
                p.insert(r, toks, n)
                p.release(r)
        elif op == 2:
            r, toks, n = live[int(rng.integers(0, len(live)))]
            for p in (pn, po):
                p.insert(r, toks, n - 1)
        else:
            reqs = [x[0] for x in live]
            q = [int(rng.integers(0, x[2] + 1)) for x in live]
            mn, mo = pn.bind(reqs, q, 8), po.bind(reqs, q, 8)
            for key in ("out_cache_loc", "kv_indptr", "qo_indptr"):
                assert np.array_equal(mn[key], mo[key])
            assert sorted(zip(mn["q_tile_to_batch"].tolist(), mn["q_tile_to_index"].tolist())) == \
                sorted(zip(mo["q_tile_to_batch"].tolist(), mo["q_tile_to_index"].tolist()))
        assert np.array_equal(pn.table(), po.table()), step
        assert pn.p.free_pages() == sum(po.p.free)


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_builder_eviction_lifecycle_matches_oracle(seed):
    """Random admit / extend / complete / insert / evict sequences on a pool
    small enough that extends evict; both builders must agree on every
    return, table, reference count and counter."""
    _lib()
    from paged_gqa_attention_rope_amd import AstrError, PagePool
    rng = np.random.default_rng(seed)
    ps, n_pages, max_reqs = 4, 32, 6
    perm = rng.permutation(n_pages).astype(np.int32)
    pn = PagePool(1, ps * n_pages, ps, max_reqs, 96, perm)
    po = OraclePool(1, ps * n_pages, ps, max_reqs, 96, perm)
    prompts = [rng.integers(0, 3, size=96).astype(np.int32) for _ in range(3)]
    live = {}

    def both(fn_n, fn_o):
        try:
            a = fn_n()
        except AstrError:
            a = "err"
        try:
            b = fn_o()
        except PoolError:
            b = "err"
        return a, b

    evictions = 0
    for step in range(500):
        op = rng.integers(0, 5)
        if op <= 1 or not live:
            toks = prompts[rng.integers(0, 3)].copy()
            cut = int(rng.integers(0, 96))
            toks[cut:] = rng.integers(0, 3, size=96 - cut)
            n = int(rng.integers(1, 60))
            a, b = both(lambda: pn.admit(toks, n), lambda: po.admit(toks, n))
            assert a == b, (step, a, b)
            if a == "err":
                continue
            r, c = a
            ev = po.evicted
            a, b = both(lambda: pn.extend(r, n - c), lambda: po.extend(r, n - c))
            assert a == b, (step, a, b)
            evictions += po.evicted > ev
            if a == "err":
                pn.release(r)
                po.release(r)
                continue
            live[r] = (toks, n)
        elif op == 2:
            r = sorted(live)[rng.integers(0, len(live))]
            toks, n = live.pop(r)
            k = int(rng.integers(0, n + 1))        # tokens seen, the last one sampled
            pn.complete(r, toks, k)
            po.complete(r, toks, k)
        elif op == 3:
            r = sorted(live)[rng.integers(0, len(live))]
            toks, n = live[r]
            k = int(rng.integers(0, n + 1))
            pn.insert(r, toks, k)
            po.insert(r, toks, k)
        else:
            k = int(rng.integers(0, 5))
            assert pn.evict(k) == po.evict(k)
        assert np.array_equal(pn.table(), po.table), step
        assert pn.free_pages() == po.n_free
        assert pn.cached_pages() == po.cached_pages()
        assert pn.evicted_pages() == po.evicted
        assert [pn.page_ref(p) for p in range(n_pages)] == po.ref
    assert evictions > 10


def test_builder_errors():
    L = _lib()
    from paged_gqa_attention_rope_amd import AstrArgError, AstrError, PagePool
    with pytest.raises(AstrArgError):
        PagePool(1, 100, 16, 2, 10)                       # pool not a multiple of pages
    with pytest.raises(AstrArgError):
        PagePool(1, 64, 16, 2, 10, np.array([0, 1, 1, 2]))  # not a permutation
    pp = PagePool(1, 16 * 4, 16, 2, 200)
    r, _ = pp.admit()
    pp.extend(r, 40)
    before = (pp.table(), pp.free_pages())
    with pytest.raises(AstrError) as ei:
        pp.extend(r, 40)
    assert ei.value.status == L.ASTR_E_NOMEM
    assert np.array_equal(pp.table(), before[0]) and pp.free_pages() == before[1]
    with pytest.raises(AstrArgError):
        pp.extend(r, 500)                                 # past max_ctx_len
    with pytest.raises(AstrArgError):
        pp.bind([r], [41])                                # q_len > seq_len
    with pytest.raises(AstrArgError):
        pp.release(1)                                     # not live
    pp.admit()
    with pytest.raises(AstrError):
        pp.admit()                                        # no request slot


def test_attention_calls_validate_before_launch():
    """Bad dtype/head_dim/group/layer are rejected with no device involved."""
    L = _lib()
    so = L.lib()
    m = L.KvMeta()
    m.k_buffer = m.v_buffer = 0x1000                      # never dereferenced: rejected first
    m.pool_slots, m.n_layers, m.n_kv_heads, m.head_dim, m.kv_dtype = 64, 2, 2, 128, L.ASTR_BF16
    m.batch, m.max_len = 1, 8
    cases = [
        (dict(head_dim=96), L.ASTR_E_UNSUPPORTED),
        (dict(kv_dtype=7), L.ASTR_E_UNSUPPORTED),
        (dict(n_kv_heads=3), L.ASTR_E_INVAL),             # 8 heads not a multiple of 3
        (dict(n_kv_heads=1, n_layers=2), L.ASTR_E_INVAL),  # table missing
    ]
    for change, want in cases:
        mm = L.KvMeta.from_buffer_copy(m)
        for k, v in change.items():
            setattr(mm, k, v)
        st = so.astr_decode_attn(ctypes.c_void_p(0x2000), 8, ctypes.byref(mm), 0, 64, 0.0, None, None,
                                 ctypes.c_void_p(0x3000), L.ASTR_BF16, None)
        assert st == want, (change, st)
    st = so.astr_decode_attn(None, 8, ctypes.byref(m), 5, 64, 0.0, None, None, None, L.ASTR_BF16, None)
    assert st == L.ASTR_E_INVAL                          # layer out of range
    # the fused decode write: table first, then its own checks
    mt = L.KvMeta.from_buffer_copy(m)
    mt.req_to_token = mt.req_pool_indices = mt.kv_indptr = 0x4000
    mt.num_reqs, mt.max_ctx_len = 1, 8
    q = ctypes.c_void_p(0x2000)
    assert so.astr_decode_attn_write(q, q, q, 8, ctypes.byref(mt), 0, q, 4, 64, 0.0, None, None, q,
                                     L.ASTR_BF16, None) == L.ASTR_E_INVAL   # max_pos 4 < max_len 8
    assert so.astr_decode_attn_write(q, None, q, 8, ctypes.byref(mt), 0, q, 8, 64, 0.0, None, None, q,
                                     L.ASTR_BF16, None) == L.ASTR_E_INVAL   # k_new missing
    mt.kv_dtype = L.ASTR_F32
    assert so.astr_decode_attn_write(q, q, q, 8, ctypes.byref(mt), 0, q, 8, 64, 0.0, None, None, q,
                                     L.ASTR_F32, None) == L.ASTR_E_UNSUPPORTED   # bf16 only
    st = so.astr_rope_kv_write(None, None, None, None, None, 0, 8, None, 1, ctypes.byref(m), 0, L.ASTR_BF16, None)
    assert st == L.ASTR_OK                               # zero tokens: a no-op
    st = so.astr_rope_table(None, 10, 64, 10000.0, None)
    assert st == L.ASTR_E_INVAL
    # rotary gradient: zero tokens is a no-op; shape and type errors come first
    assert so.astr_rope_backward(None, None, 0, 4, 128, None, 1, L.ASTR_BF16, None) == L.ASTR_OK
    assert so.astr_rope_backward(None, None, 5, 4, 96, None, 1, L.ASTR_BF16, None) == L.ASTR_E_UNSUPPORTED
    assert so.astr_rope_backward(None, None, 5, 4, 128, None, 1, 9, None) == L.ASTR_E_UNSUPPORTED
    assert so.astr_rope_backward(None, None, 5, 4, 128, None, 1, L.ASTR_F32, None) == L.ASTR_E_INVAL
    assert so.astr_rope_backward(None, None, -1, 4, 128, None, 1, L.ASTR_F32, None) == L.ASTR_E_INVAL
    assert so.astr_decode_num_splits(1000, 256) == 4
    assert so.astr_decode_num_splits(0, 256) == 1
    assert so.astr_decode_num_splits(10, 0) == 0
    assert b"rope_backward: n_tokens -1" in so.astr_last_error()


def test_activation_dtype_must_match_the_pool():
    """act_dtype is checked before anything is launched: a value outside the
    enum, or activations in another dtype than the pool, are rejected."""
    L = _lib()
    so = L.lib()
    m = L.KvMeta()
    m.k_buffer = m.v_buffer = 0x1000
    m.pool_slots, m.n_layers, m.n_kv_heads, m.head_dim, m.kv_dtype = 64, 1, 2, 128, L.ASTR_BF16
    m.req_to_token = m.req_pool_indices = m.kv_indptr = m.qo_indptr = 0x4000
    m.q_tile_to_batch = m.q_tile_to_index = 0x4000
    m.num_reqs, m.max_ctx_len, m.batch, m.max_len, m.num_q_tiles, m.q_tile = 1, 8, 1, 8, 1, 64
    q = ctypes.c_void_p(0x2000)
    for act, want in ((L.ASTR_F32, L.ASTR_E_UNSUPPORTED), (5, L.ASTR_E_UNSUPPORTED)):
        assert so.astr_rope_kv_write(q, q, q, q, q, 1, 8, q, 8, ctypes.byref(m), 0, act, None) == want
        assert b"act_dtype" in so.astr_last_error()
        assert so.astr_decode_attn(q, 8, ctypes.byref(m), 0, 64, 0.0, None, None, q, act, None) == want
        assert so.astr_decode_attn_write(q, q, q, 8, ctypes.byref(m), 0, q, 8, 64, 0.0, None, None, q, act,
                                         None) == want
        assert so.astr_prefill_attn(q, 8, 8, ctypes.byref(m), 0, 0.0, q, act, None) == want
        assert b"act_dtype" in so.astr_last_error()


def test_noalloc_decode_rejects_scratch_beyond_its_array():
    """The allocation-free decode checks its scratch size on the host before
    touching the device: 256 requests x 16 heads x 128 splits of a 128-wide
    head need 270 MB, more than the 160 MiB static array."""
    L = _lib()
    so = L.lib()
    m = L.KvMeta()
    m.k_buffer = m.v_buffer = 0x1000
    m.pool_slots, m.n_layers, m.n_kv_heads, m.head_dim, m.kv_dtype = 1 << 20, 1, 4, 128, L.ASTR_BF16
    m.req_to_token = m.req_pool_indices = m.kv_indptr = 0x4000
    m.num_reqs, m.max_ctx_len, m.batch, m.max_len = 256, 32768, 256, 32768
    q = ctypes.c_void_p(0x2000)
    need = so.astr_decode_workspace_bytes(256, 16, 128, 32768, 256)
    assert need > 160 << 20
    st = so.astr_decode_attn_noalloc(q, 16, ctypes.byref(m), 0, 256, 0.0, q, L.ASTR_BF16, None)
    assert st == L.ASTR_E_INVAL and b"static scratch holds" in so.astr_last_error()
    assert so.astr_decode_attn_noalloc(q, 16, None, 0, 256, 0.0, q, L.ASTR_BF16, None) == L.ASTR_E_INVAL


def test_decode_workspace_bytes():
    """The split-K scratch: float32 o_part [B, H, S, D] then lse_part [B, H, S],
    S = ceil(max_len / chunk); nothing when one split covers max_len."""
    L = _lib()
    so = L.lib()
    import paged_gqa_attention_rope_amd as astr
    for b, h, d, ml, c in ((256, 16, 128, 32768, 512), (8, 16, 128, 2048, 256), (2, 4, 64, 33, 16),
                           (3, 24, 64, 1000, 7), (0, 8, 128, 4000, 256)):
        s = -(-ml // c)
        assert so.astr_decode_workspace_bytes(b, h, d, ml, c) == 4 * b * h * s * (d + 1)
        assert astr.decode_workspace_bytes(b, h, d, ml, c) == 4 * b * h * s * (d + 1)
    assert so.astr_decode_workspace_bytes(4, 8, 128, 256, 256) == 0       # one split
    assert so.astr_decode_workspace_bytes(4, 8, 128, 0, 256) == 0
    for bad in ((-1, 8, 128, 100, 16), (4, 0, 128, 100, 16), (4, 8, 0, 100, 16), (4, 8, 128, -1, 16),
                (4, 8, 128, 100, 0)):
        assert so.astr_decode_workspace_bytes(*bad) == 0


def _items_rule(lens, chunk):
    """The decode work items stated as a rule: every split of every entry
    (split 0 for an empty one); full splits in batch order, then the last
    splits, longest first, ties by batch entry."""
    ns = [max(1, -(-int(x) // chunk)) for x in lens]
    full = [(b, s) for b in range(len(lens)) for s in range(ns[b] - 1)]
    last = sorted(range(len(lens)), key=lambda b: (-(int(lens[b]) - (ns[b] - 1) * chunk), b))
    return full + [(b, ns[b] - 1) for b in last]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_split_items_follow_the_rule(seed):
    import paged_gqa_attention_rope_amd as astr
    _lib()
    rng = np.random.default_rng(seed)
    lens = np.concatenate([rng.integers(0, 3000, size=40), [0, 1, 512, 513, 1024]]).astype(np.int32)
    for chunk in (1, 7, 256, 512, 4096):
        ib, ix = astr.decode_split_items(lens, chunk)
        got = list(zip(ib.tolist(), ix.tolist()))
        assert got == _items_rule(lens, chunk), chunk
        # each (entry, split) once, and exactly the splits that hold keys (split 0 always)
        assert len(set(got)) == len(got)
        assert sorted(got) == sorted((b, s) for b in range(lens.size)
                                     for s in range(max(1, -(-int(lens[b]) // chunk))))


def test_decode_split_items_errors_and_abi_checks():
    import paged_gqa_attention_rope_amd as astr
    L = _lib()
    so = L.lib()
    with pytest.raises(Exception):
        astr.decode_split_items(np.array([5, -1], np.int32), 4)
    seq = np.array([10, 20], np.int32)
    ib = np.zeros(2, np.int32)
    n = ctypes.c_int()
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert so.astr_decode_split_items(p(seq), 2, 8, p(ib), p(ib), 2, ctypes.byref(n)) == L.ASTR_E_INVAL  # needs 5
    assert so.astr_decode_split_items(p(seq), 2, 0, p(ib), p(ib), 8, ctypes.byref(n)) == L.ASTR_E_INVAL
    assert so.astr_decode_split_items(p(seq), 0, 8, None, None, 0, ctypes.byref(n)) == L.ASTR_OK
    assert n.value == 0
    # the decode calls check the work items before anything is launched
    m = L.KvMeta()
    m.k_buffer = m.v_buffer = 0x1000
    m.pool_slots, m.n_layers, m.n_kv_heads, m.head_dim, m.kv_dtype = 64, 2, 2, 128, L.ASTR_BF16
    m.req_to_token = m.req_pool_indices = m.kv_indptr = 0x4000
    m.num_reqs, m.max_ctx_len, m.batch, m.max_len = 1, 8, 1, 8
    q = ctypes.c_void_p(0x2000)
    m.split_item_batch = 0x5000                          # index list missing
    m.num_split_items, m.split_item_chunk = 1, 64
    assert so.astr_decode_attn(q, 8, ctypes.byref(m), 0, 64, 0.0, None, None, q, L.ASTR_BF16, None) == L.ASTR_E_INVAL
    m.split_item_index = 0x6000
    m.split_item_chunk = 32                              # built for another chunk
    assert so.astr_decode_attn(q, 8, ctypes.byref(m), 0, 64, 0.0, None, None, q, L.ASTR_BF16, None) == L.ASTR_E_INVAL
    assert b"split_chunk 32" in so.astr_last_error()
    m.split_item_chunk, m.num_split_items = 64, 0        # no count
    assert so.astr_decode_attn(q, 8, ctypes.byref(m), 0, 64, 0.0, None, None, q, L.ASTR_BF16, None) == L.ASTR_E_INVAL


# ---------------------------------------------------------------------------
# prefill work plan
# ---------------------------------------------------------------------------

def _plan_meta(seq, ext, q_tile=64):
    """Host step metadata of a ragged prefill (tiles heaviest first, as the
    builder lists them)."""
    seq, ext = np.asarray(seq), np.asarray(ext)
    kv = np.concatenate([[0], np.cumsum(seq)]).astype(np.int32)
    qo = np.concatenate([[0], np.cumsum(ext)]).astype(np.int32)
    tiles = sorted((-(int(seq[b] - ext[b]) + min(q_tile * (i + 1), int(ext[b]))), b, i)
                   for b in range(len(seq)) for i in range(-(-int(ext[b]) // q_tile)))
    return dict(qo_indptr=qo, kv_indptr=kv, q_tile_to_batch=np.array([t[1] for t in tiles], np.int32),
                q_tile_to_index=np.array([t[2] for t in tiles], np.int32), num_q_tiles=len(tiles),
                q_tile=q_tile, req_pool_indices=(np.arange(len(seq)) * 7 + 3).astype(np.int32))


def _plan_rule(meta, wg, num_cus):
    """The prefill work plan stated as its documented rule, in Python."""
    qo, kv, rpi = meta["qo_indptr"], meta["kv_indptr"], meta["req_pool_indices"]
    qt = meta["q_tile"]
    steps, rows_of, group = [], [], []
    for b, i in zip(meta["q_tile_to_batch"], meta["q_tile_to_index"]):
        e = int(qo[b + 1] - qo[b])
        p = int(kv[b + 1] - kv[b]) - e
        row0 = int(i) * qt
        ok = e > 0 and p >= 0 and row0 < e
        steps.append(-(-(p + row0 + min(qt, e - row0)) // 32) if ok else 0)
        group.append(int(b) if ok else -1)
        rows_of.append([int(rpi[b]), int(qo[b]) + row0, min(qt, e - row0), p + row0] if ok else [0, 0, 0, 0])
    big = 2 ** 31 - 1

    def units(split, num, den):
        out = []
        for t, n in enumerate(steps):
            if t in split and n >= 2:
                h = max(1, n * num // den)
                out += [(8.5 + h, t, 0, 0, h), (9.5 + n - h, t, 1, h, big)]
            else:
                out.append((7.0 + n if n > 0 else 0.1, t, -1, 0, big))
        return sorted(out, key=lambda u: (-u[0], u[1], u[2]))

    def deal(lst):
        # earliest end; on ties an XCD holding 1 to 3 units of the same
        # request first, then fewer units queued, then the lower XCD
        free = [[0.0] * (num_cus // 8) for _ in range(8)]
        queue = [[] for _ in range(8)]
        holds = [dict() for _ in range(8)]
        end = 0.0
        w = min(wg, num_cus // 8)
        for u in lst:
            ends = [sorted(free[x])[w - 1] + u[0] for x in range(8)]
            grp = group[u[1]]
            joins = [grp >= 0 and 0 < holds[x].get(grp, 0) < 4 for x in range(8)]
            x = min(range(8), key=lambda x: (ends[x], 0 if joins[x] else 1, len(queue[x]), x))
            if grp >= 0:
                holds[x][grp] = holds[x].get(grp, 0) + 1
            for _ in range(wg):
                f = sorted(free[x])
                f[0] += u[0]
                end = max(end, f[0])
                free[x] = f
            queue[x].append(u)
        return end, queue

    base, queue = deal(units(set(), 1, 2))
    mx = max(steps) if steps else 0
    by_len = sorted(range(len(steps)), key=lambda t: -steps[t])      # stable: ties by tile order
    cands = [({t for t, n in enumerate(steps) if n > mx * k // 10}, 1, 2) for k in range(9, 2, -1)]
    cands += [(set(by_len[:top]), 3, 10) for top in (1, 2, 3, 4, 5, 6, 8, 10, 12, 16) if top < len(steps)]
    best_end, best_q = base, None
    for split, num, den in cands:
        e, q = deal(units(split, num, den))
        if e < best_end:
            best_end, best_q = e, q
    if best_q is not None and best_end <= 0.90 * base:
        queue = best_q
    pair_of, rows = {}, []
    for k in range(max(len(q) for q in queue)):
        for x in range(8):
            if k >= len(queue[x]):
                rows.append([-1, 0, 0, -1, 0, 0, 0, 0])
                continue
            u = queue[x][k]
            pw = -1
            if u[2] >= 0:
                pair_of.setdefault(u[1], len(pair_of))
                pw = 2 * pair_of[u[1]] + u[2]
            rows.append([u[1], u[3], u[4], pw] + rows_of[u[1]])
    return np.array(rows, np.int32).reshape(-1, 8), len(pair_of)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_prefill_plan_follows_the_rule(seed):
    import paged_gqa_attention_rope_amd as astr
    _lib()
    rng = np.random.default_rng(seed)
    shapes = [
        (rng.integers(0, 129, 16) * 16, rng.integers(32, 513, 16)),     # radix prefixes, mixed extends
        (np.full(64, 2048), np.full(64, 64)),                           # balanced
        (np.zeros(4, int), rng.integers(64, 1025, 4)),                  # few long prompts
        (rng.integers(0, 40, 7), rng.integers(1, 4, 7)),                # tiny
    ]
    for pre, ext in shapes:
        meta = _plan_meta(np.asarray(pre) + np.asarray(ext), ext)
        for wg, cus in ((4, 256), (2, 256), (4, 64)):
            units, pairs = astr.prefill_plan(meta, 4 * wg, cus)
            want, want_pairs = _plan_rule(meta, wg, cus)
            assert np.array_equal(units, want) and pairs == want_pairs
            # every tile once whole, or twice as halves [0, h) and [h, end)
            assert len(units) % 8 == 0
            seen = {}
            for t, lo, hi, pw, *rest in units.tolist():
                if t == -1:
                    assert (lo, hi, pw, *rest) == (0, 0, -1, 0, 0, 0, 0)      # padding
                    continue
                seen.setdefault(t, []).append((lo, hi, pw))
                # the tile's rows and keys, as its maps give them
                b, i = meta["q_tile_to_batch"][t], meta["q_tile_to_index"][t]
                e = meta["qo_indptr"][b + 1] - meta["qo_indptr"][b]
                pre = meta["kv_indptr"][b + 1] - meta["kv_indptr"][b] - e
                assert rest == [meta["req_pool_indices"][b], meta["qo_indptr"][b] + 64 * i,
                                min(64, e - 64 * i), pre + 64 * i]
            assert sorted(seen) == list(range(meta["num_q_tiles"]))
            for t, us in seen.items():
                if len(us) == 1:
                    assert us[0] == (0, 2 ** 31 - 1, -1)
                else:
                    (lo0, hi0, p0), (lo1, hi1, p1) = sorted(us)
                    assert lo0 == 0 and hi0 == lo1 > 0 and hi1 == 2 ** 31 - 1
                    assert p0 // 2 == p1 // 2 and p0 % 2 == 0 and p1 % 2 == 1
            assert sorted({u[3] // 2 for u in units.tolist() if u[3] >= 0}) == list(range(pairs))


def test_prefill_plan_splits_only_what_dominates():
    import paged_gqa_attention_rope_amd as astr
    _lib()
    # balanced: no split
    units, pairs = astr.prefill_plan(_plan_meta(np.full(64, 2112), np.full(64, 64)), 16)
    assert pairs == 0 and len(units) == 64 and (units[:, 0] >= 0).all()
    # one long tile among many short ones: split
    seq = np.concatenate([[2560], np.full(300, 200)])
    ext = np.concatenate([[64], np.full(300, 64)])
    units, pairs = astr.prefill_plan(_plan_meta(seq, ext), 16)
    # both halves lead XCD 0's queue (positions 0 and 8: its first two units),
    # which has room for both at once; they stay together on one L2
    assert pairs == 1 and units[0][0] == 0 and units[8][0] == 0 and (units[1:8, 0] != 0).all()
    assert astr.prefill_workspace_bytes(0, 16, 128) == 0
    per = 2 * (8 * 2 * 8 * 64 * 4 + 8 * 2 * 64 * 2) * 4
    assert astr.prefill_workspace_bytes(3, 16, 128) == 256 + 12 * per
    assert astr.prefill_workspace_bytes(-1, 16, 128) == 0


def test_prefill_plan_errors_and_abi_checks():
    import paged_gqa_attention_rope_amd as astr
    L = _lib()
    so = L.lib()
    meta = _plan_meta([100, 300], [50, 200])
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    n, pr = ctypes.c_int(), ctypes.c_int()
    cap = 16 * meta["num_q_tiles"]                     # documented to always suffice
    u = np.zeros((cap, 8), np.int32)
    args = [p(meta["qo_indptr"]), p(meta["kv_indptr"]), p(meta["req_pool_indices"]), 2,
            p(meta["q_tile_to_batch"]), p(meta["q_tile_to_index"]), meta["num_q_tiles"], 64]
    assert so.astr_prefill_plan(*args, 4, 256, p(u), cap, ctypes.byref(n), ctypes.byref(pr)) == L.ASTR_OK
    need = n.value
    assert need % 8 == 0 and 8 <= need <= cap
    assert so.astr_prefill_plan(*args, 4, 256, p(u), need, ctypes.byref(n), ctypes.byref(pr)) == L.ASTR_OK
    assert so.astr_prefill_plan(*args, 4, 4, p(u), cap, ctypes.byref(n), ctypes.byref(pr)) == L.ASTR_E_INVAL
    assert so.astr_prefill_plan(*args, 0, 256, p(u), cap, ctypes.byref(n), ctypes.byref(pr)) == L.ASTR_E_INVAL
    assert so.astr_prefill_plan(*args, 4, 256, p(u), need - 1, ctypes.byref(n), ctypes.byref(pr)) == L.ASTR_E_INVAL
    # the prefill call checks the plan before anything is launched
    m = L.KvMeta()
    m.k_buffer = m.v_buffer = 0x1000
    m.pool_slots, m.n_layers, m.n_kv_heads, m.head_dim, m.kv_dtype = 1024, 1, 4, 128, L.ASTR_BF16
    m.req_to_token = m.req_pool_indices = m.kv_indptr = m.qo_indptr = 0x4000
    m.q_tile_to_batch = m.q_tile_to_index = 0x4000
    m.num_reqs, m.max_ctx_len, m.batch, m.max_len, m.num_q_tiles, m.q_tile = 2, 512, 2, 300, 5, 64
    q = ctypes.c_void_p(0x2000)

    def call():
        return so.astr_prefill_attn(q, 250, 16, ctypes.byref(m), 0, 0.0, q, L.ASTR_BF16, None)

    m.prefill_units = 0x8000                             # no count
    assert call() == L.ASTR_E_INVAL and b"incomplete" in so.astr_last_error()
    m.num_prefill_units, m.prefill_units = 6, 0x8004     # misaligned
    assert call() == L.ASTR_E_INVAL and b"aligned" in so.astr_last_error()
    m.prefill_units, m.num_prefill_pairs = 0x8000, 4     # more pairs than units can hold
    assert call() == L.ASTR_E_INVAL and b"split tiles" in so.astr_last_error()
    m.prefill_units, m.num_prefill_pairs = 0x8000, 1     # pairs without workspace
    assert call() == L.ASTR_E_INVAL and b"workspace" in so.astr_last_error()
    m.prefill_workspace = 0x9000
    m.prefill_workspace_bytes = astr.prefill_workspace_bytes(1, 16, 128) - 1
    assert call() == L.ASTR_E_INVAL and b"needs" in so.astr_last_error()
    m.prefill_workspace_bytes += 1
    m.num_prefill_units = 81                             # more than 16 * num_q_tiles
    assert call() == L.ASTR_E_INVAL and b"too large" in so.astr_last_error()
