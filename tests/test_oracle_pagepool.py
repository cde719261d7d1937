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
    # KV extents seen by each tile's last row: (0,0) 28, (0,1) 33, (1,0) 8, (1,1) 16
    assert np.array_equal(m["q_tile_to_batch"], [0, 0, 1, 1])
    assert np.array_equal(m["q_tile_to_index"], [1, 0, 1, 0])


def test_tile_maps_cover_every_row_heaviest_first():
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
    assert sorted(pairs) == [(b, t) for b in range(9) for t in range(n[b])]
    ext = [int(pre[b] + min(64 * (t + 1), q[b])) for b, t in pairs]
    assert all(ext[i] >= ext[i + 1] for i in range(len(ext) - 1))
    for i in range(len(ext) - 1):
        if ext[i] == ext[i + 1]:
            assert pairs[i] < pairs[i + 1]


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
