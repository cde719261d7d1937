"""Pins for the oracle's page-table builder (CPU only).

Facts used (AstrAI docs/guides/inference.md, "KVCache System"): the contiguous
closed form slot = req_idx * max_seq_len + pos; kv_indptr / qo_indptr are
prefix sums of the KV and query lengths; the radix matches exact token pages
under the same parent only, shares only complete materialised pages, and a
request resumes right after the longest hit.  The allocation order is this
build's stated reading (lowest free first), checked here through its closed
forms.
"""

import numpy as np
import pytest

from oracle.pagepool import PagePool, PoolError
from workloads import make_case


def test_contiguous_closed_form():
    pp = PagePool(0, 4 * 64, 1, 4, 64)
    lens = [17, 64, 1, 40]
    for L in lens:
        r, c = pp.admit(None, L)
        assert c == 0
        pp.extend(r, L)
    for r, L in enumerate(lens):
        assert np.array_equal(pp.table[r, :L], r * 64 + np.arange(L))
        assert np.all(pp.table[r, L:] == -1)
    m = pp.bind([0, 1, 2, 3], [1, 1, 1, 1])
    assert np.array_equal(m["out_cache_loc"], [r * 64 + L - 1 for r, L in enumerate(lens)])
    assert np.array_equal(m["kv_indptr"], np.concatenate([[0], np.cumsum(lens)]))
    assert m["max_len"] == 64


def test_page1_permutation_gives_consecutive_chunks():
    rng = np.random.default_rng(0)
    perm = rng.permutation(1000)
    pp = PagePool(1, 1000, 1, 5, 300, perm)
    lens = [13, 300, 2, 77, 150]
    for L in lens:
        r, _ = pp.admit(None, L)
        pp.extend(r, L)
    off = np.concatenate([[0], np.cumsum(lens)])
    for r, L in enumerate(lens):
        assert np.array_equal(pp.table[r, :L], perm[off[r]:off[r] + L])


def test_paged_slots_and_growth():
    pp = PagePool(1, 16 * 20, 16, 3, 200)
    r0, _ = pp.admit(None, 0)
    pp.extend(r0, 20)            # logical pages 0, 1
    r1, _ = pp.admit(None, 0)
    pp.extend(r1, 16)            # page 2
    pp.extend(r0, 13)            # 33 tokens: page 3 joins request 0
    assert np.array_equal(pp.table[r0, :33],
                          np.concatenate([np.arange(32), 48 + np.arange(1)]))
    assert np.array_equal(pp.table[r1, :16], 32 + np.arange(16))
    m = pp.bind([r0, r1], [13, 16], q_tile=8)
    assert np.array_equal(m["out_cache_loc"], np.concatenate([pp.table[r0, 20:33], pp.table[r1, :16]]))
    assert np.array_equal(m["qo_indptr"], [0, 13, 29])
    # request-major tiles: request 0 rows [0, 8), [8, 13); request 1 rows [0, 8), [8, 16)
    assert np.array_equal(m["q_tile_to_batch"], [0, 0, 1, 1])
    assert np.array_equal(m["q_tile_to_index"], [0, 1, 0, 1])


def test_tile_maps_cover_every_row_request_major():
    rng = np.random.default_rng(1)
    q = rng.integers(1, 300, size=9)
    pre = 16 * rng.integers(0, 20, size=9)
    pp = PagePool(0, 9 * 700, 1, 9, 700)
    for p, L in zip(pre, q):
        r, _ = pp.admit(None, 0)
        pp.extend(r, int(p + L))
    m = pp.bind(list(range(9)), list(q), q_tile=64)
    n = -(-q // 64)
    assert m["num_q_tiles"] == n.sum()
    pairs = list(zip(m["q_tile_to_batch"].tolist(), m["q_tile_to_index"].tolist()))
    assert pairs == [(b, t) for b in range(9) for t in range(n[b])]
    # every query row lies in exactly one tile, the last tile of a request may be partial
    rows = [(b, i) for b, t in pairs for i in range(64 * t, min(64 * (t + 1), int(q[b])))]
    assert sorted(rows) == [(b, i) for b in range(9) for i in range(int(q[b]))]


def test_nomem_leaves_state_unchanged():
    pp = PagePool(1, 16 * 4, 16, 2, 200)
    r, _ = pp.admit(None, 0)
    pp.extend(r, 40)             # 3 pages
    before = (pp.table.copy(), list(pp.free), list(pp.ref), list(pp.length))
    with pytest.raises(PoolError) as ei:
        pp.extend(r, 40)         # would need 3 more pages, 1 left
    assert ei.value.kind == "nomem"
    assert np.array_equal(pp.table, before[0]) and pp.free == before[1]
    assert pp.ref == before[2] and pp.length == before[3]
    r2, _ = pp.admit(None, 0)
    with pytest.raises(PoolError) as ei:
        pp.admit(None, 0)
    assert ei.value.kind == "nomem"
    with pytest.raises(PoolError):
        pp.bind([r2], [1])       # q_len exceeds its (zero) length


def test_radix_exact_pages_same_parent_only():
    ps = 4
    pp = PagePool(1, ps * 64, ps, 8, 64)
    a = np.arange(100, 120)                         # 5 pages
    r, c = pp.admit(a, 20)
    assert c == 0
    pp.extend(r, 20)
    pp.insert(r, a, 20)
    pages_a = list(pp.pages[r])
    pp.release(r)
    # full prompt match is capped so that one token remains to compute
    r1, c1 = pp.admit(a, 20)
    assert c1 == 16
    assert np.array_equal(pp.table[r1, :16], np.arange(16))      # pages 0..3 reused
    # a prompt that shares 2 pages then diverges
    b = np.concatenate([a[:8], [1, 2, 3, 4], a[12:20]])
    r2, c2 = pp.admit(b, 20)
    assert c2 == 8
    # an identical page under a different parent is not a match
    d = np.concatenate([[7, 7, 7, 7], a[4:20]])
    r3, c3 = pp.admit(d, 20)
    assert c3 == 0
    # partial pages never enter the radix
    pp.extend(r2, 12)
    pp.insert(r2, b, 19)                                            # 4 complete pages
    e = np.concatenate([b[:19], [9, 9, 9, 9, 9]])
    r4, c4 = pp.admit(e, 24)
    assert c4 == 16 and np.array_equal(pp.table[r4, :16], pp.table[r2, :16])
    # reference counts: radix holds one, every live holder one more
    assert pp.ref[pages_a[0]] == 1 + 3                              # radix + r1, r2, r4
    for rr in (r1, r2, r3, r4):
        pp.release(rr)
    assert pp.ref[pages_a[0]] == 1
    assert all(pp.ref[p] == 1 for p in pages_a[:5])


def test_prefix_workload_hits_exactly_the_drawn_prefix():
    cs = make_case(4)
    pp = PagePool(cs.mode, cs.pool_slots, cs.page_size, cs.max_reqs + 4, cs.max_ctx_len)
    for g, toks in enumerate(cs.group_tokens):
        if len(toks) == 0:
            continue
        r, c = pp.admit(toks, len(toks))
        pp.extend(r, len(toks) - c)
        pp.insert(r, toks, len(toks))
        pp.release(r)
    reqs = []
    for b in range(cs.batch):
        r, c = pp.admit(cs.tokens[b], len(cs.tokens[b]))
        assert c == cs.prefix_lens[b]
        pp.extend(r, len(cs.tokens[b]) - c)
        reqs.append(r)
    # requests of one group with equal-length prefixes share every prefix slot
    for b1 in range(cs.batch):
        for b2 in range(cs.batch):
            if cs.group_of[b1] == cs.group_of[b2]:
                n = min(cs.prefix_lens[b1], cs.prefix_lens[b2])
                assert np.array_equal(pp.table[reqs[b1], :n], pp.table[reqs[b2], :n])
    # extend slots are private
    ext = np.concatenate([pp.table[reqs[b], cs.prefix_lens[b]:cs.seq_lens[b]] for b in range(cs.batch)])
    assert len(np.unique(ext)) == len(ext)


# -- lifecycle: completion and LRU eviction ----------------------------------------
# The scenarios below are worked by hand from the rules in the oracle's header
# (leaf-first LRU over pages only the radix holds; one tick per admit or
# insert; an extend evicts just what it lacks, or nothing and fails).

def _two_cached_chains():
    """Page size 2, 8 pages.  Chain A = pages 0 -> 1 -> 2 (tokens 1..6),
    cached before chain B = pages 3 -> 4 (tokens 11..14); pages 5..7 free."""
    pp = PagePool(1, 16, 2, 4, 32)
    a = np.arange(1, 7)
    b = np.arange(11, 15)
    r, c = pp.admit(a, 6)
    assert (r, c) == (0, 0)
    pp.extend(r, 6)
    pp.complete(r, np.concatenate([a, [99]]), 7)       # 6 tokens have KV: 3 pages
    r, c = pp.admit(b, 4)
    assert (r, c) == (0, 0)
    pp.extend(r, 4)
    pp.complete(r, np.concatenate([b, [98]]), 5)       # 4 tokens have KV: 2 pages
    assert pp.cached_pages() == 5 and pp.n_free == 3
    assert [pp.ref[p] for p in range(8)] == [1, 1, 1, 1, 1, 0, 0, 0]
    return pp, a, b


def test_eviction_takes_least_recent_leaves_first():
    pp, a, b = _two_cached_chains()
    r, c = pp.admit(np.arange(21, 31), 10)
    assert c == 0
    pp.extend(r, 10)                 # 5 pages, 3 free: evict A's leaf 2, then 1
    assert pp.evicted == 2 and pp.cached_pages() == 3
    assert np.array_equal(pp.table[r, :10], [2, 3, 4, 5, 10, 11, 12, 13, 14, 15])
    # A's root page and chain B survive: a prompt of A matches one page only
    pp.release(r)
    r2, c2 = pp.admit(a, 6)
    assert c2 == 2 and pp.table[r2, 0] == 0
    r3, c3 = pp.admit(b, 5)
    assert c3 == 4


def test_a_lookup_makes_pages_recent():
    pp, a, b = _two_cached_chains()
    r, c = pp.admit(a, 6)            # touches pages 0 and 1, not the leaf 2
    assert c == 4
    pp.release(r)
    r, c = pp.admit(np.arange(21, 31), 10)
    pp.extend(r, 10)                 # evicts leaf 2 (oldest), then B's leaf 4
    assert np.array_equal(pp.table[r, :10], [4, 5, 8, 9, 10, 11, 12, 13, 14, 15])
    assert sorted(pp.node_of_page) == [0, 1, 3]


def test_held_pages_are_never_evicted_and_nomem_evicts_nothing():
    pp, a, b = _two_cached_chains()
    holder, c = pp.admit(a, 6)       # holds pages 0, 1: only 2, 3, 4 can go
    assert c == 4 and pp.evictable_pages() == 3
    snap = (pp.table.copy(), list(pp.free), list(pp.ref), pp.cached_pages())
    r, _ = pp.admit(None, 0)
    with pytest.raises(PoolError) as ei:
        pp.extend(r, 14)             # 7 pages > 3 free + 3 evictable
    assert ei.value.kind == "nomem"
    assert np.array_equal(pp.table, snap[0]) and pp.free == snap[1]
    assert pp.ref == snap[2] and pp.cached_pages() == snap[3] and pp.evicted == 0
    pp.extend(r, 12)                 # 6 pages: evicts 2, then 4, then 3
    assert np.array_equal(pp.table[r, :12], [4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15])
    assert sorted(pp.node_of_page) == [0, 1]
    assert pp.ref[0] == 2 and pp.ref[1] == 2


def test_completion_caches_only_pages_with_kv():
    ps = 4
    toks = np.arange(50, 59)                           # 7 prompt + 2 generated tokens
    for n_tokens, n_cached in ((9, 2), (8, 1), (5, 1), (4, 0), (1, 0)):
        pp = PagePool(1, ps * 16, ps, 4, 64)
        r, _ = pp.admit(toks[:7], 7)
        pp.extend(r, n_tokens)                         # the sampled token's slot too
        pages = list(pp.pages[r])
        pp.complete(r, toks, n_tokens)
        assert pp.cached_pages() == n_cached
        # the cached pages are the request's first ones; the rest (partial
        # page included) went back to the free set
        assert sorted(pp.node_of_page) == pages[:n_cached]
        assert pp.n_free == 16 - n_cached
        r2, c2 = pp.admit(np.concatenate([toks, [1, 2, 3, 4]]), 13)
        assert c2 == ps * n_cached


def _peel_count(pp):
    """Evictable pages by brute force: on a copy of the radix, repeatedly
    remove every childless node whose page only the radix holds."""
    nodes = {p: n for p, n in pp.node_of_page.items()}
    parent = {p: (None if n.parent is pp.root else n.parent.page) for p, n in nodes.items()}
    alive = set(nodes)
    removed = 0
    while True:
        has_child = {parent[p] for p in alive if parent[p] is not None}
        leaves = [p for p in alive if p not in has_child and pp.ref[p] == 1]
        if not leaves:
            return removed
        alive -= set(leaves)
        removed += len(leaves)


def test_lifecycle_invariants_under_pressure():
    rng = np.random.default_rng(5)
    ps, n_pages = 4, 24
    pp = PagePool(1, ps * n_pages, ps, 6, 64)
    prompts = [rng.integers(0, 4, size=64) for _ in range(3)]
    live = {}
    n_evict_events = 0
    for step in range(400):
        op = rng.integers(0, 4)
        if op == 0 or not live:
            toks = prompts[rng.integers(0, 3)].copy()
            cut = int(rng.integers(0, 64))
            toks[cut:] = rng.integers(0, 4, size=64 - cut)
            n = int(rng.integers(1, 40))
            try:
                r, c = pp.admit(toks, n)
            except PoolError:
                continue
            free_before, ev_before = pp.n_free, pp.evicted
            need = -(-n // ps) - len(pp.pages[r])
            can = _peel_count(pp)
            try:
                pp.extend(r, n - c)
            except PoolError as e:
                assert e.kind == "nomem" and need > free_before + can
                assert pp.evicted == ev_before
                pp.release(r)
                continue
            assert need <= free_before + can
            assert pp.evicted - ev_before == max(0, need - free_before)
            n_evict_events += pp.evicted > ev_before
            live[r] = (toks, n)
        elif op == 1:
            r = list(live)[rng.integers(0, len(live))]
            toks, n = live.pop(r)
            pp.complete(r, toks, n)
        elif op == 2:
            r = list(live)[rng.integers(0, len(live))]
            toks, n = live[r]
            pp.insert(r, toks, int(rng.integers(0, n + 1)))
        else:
            k = int(rng.integers(0, 4))
            can, before = _peel_count(pp), pp.cached_pages()
            assert pp.evict(k) == min(k, can)
            assert pp.cached_pages() == before - min(k, can)
        # reference counts: one per live holder, one for the radix
        held = [0] * n_pages
        for r in live:
            for p in pp.pages[r]:
                held[p] += 1
        for p in pp.node_of_page:
            held[p] += 1
        assert held == pp.ref, step
        assert [pp.ref[p] == 0 for p in range(n_pages)] == pp.free
        assert pp.n_free == sum(pp.free)
        # the radix stays a tree: every cached node's parent is cached
        for p, n in pp.node_of_page.items():
            assert n.parent is pp.root or pp.node_of_page.get(n.parent.page) is n.parent
            kids = sum(1 for m in pp.node_of_page.values() if m.parent is n)
            assert kids == n.n_children
        for r in live:
            L = pp.length[r]
            assert np.array_equal(pp.table[r, :L], [pp.pages[r][i // ps] * ps + i % ps for i in range(L)])
    assert n_evict_events > 5
