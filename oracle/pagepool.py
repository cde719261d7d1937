"""Page-table builder, restated in plain Python.

AstrAI docs/guides/inference.md, "KVCache System" (and internals.md, "Cache
Architecture"):

* contiguous mode: ``req_to_token`` is the linear map
  slot = req_idx * max_seq_len + pos, nothing is allocated dynamically;
* paged mode (page_size 1, or larger): a shared pool, slots allocated on demand
  by a bitmask page allocator with reference counts;
* with page_size > 1 a radix cache indexes complete token pages as
  parent-linked edges; a lookup walks from the root comparing each page's
  exact token tuple, so a page is reused only under the same parent prefix;
  hashes are kept for introspection and never decide a match; only complete,
  materialised pages enter it; a new request resumes prefill right after the
  longest complete-page hit;
* ``bind_tasks()`` emits ``req_pool_indices``, ``seq_lens``, ``out_cache_loc``
  (the slots written this step), ``max_len`` (host int), ``kv_indptr`` and
  ``qo_indptr`` (prefix sums of KV and query lengths) and the query-tile maps
  ``q_tile_to_batch`` / ``q_tile_to_index``.

Readings where the pages are silent (the allocation order is needed for
bit-exact tables): request slots and pages are taken lowest-free-first;
requests are served in the order given and positions in increasing order;
a logical page maps to physical page ``page_perm[logical]`` when a permutation
is given; slot = physical_page * page_size + pos % page_size; unused table
entries are -1; a lookup leaves at least one prompt token to compute, so it
matches at most floor((n_tokens - 1) / page_size) pages; query tiles cover
q_tile rows each, the last one of a request possibly partial, and are listed
request-major (requests in batch order, a request's tiles in row order -- the
pages fix only the tile -> request maps, not their order, so the library may
list them in another order of its own);
``out_cache_loc`` is flat in ``qo_indptr`` order.

Lifecycle (same pages: the allocator's reference counts and LRU eviction;
the completion rule that records the prompt plus the generated tokens already
decoded into KV, never the final sampled token, and releases the partial
page).  Readings where the pages are silent: a cached page is evictable when
only the radix still holds it and it has no cached children (evicting a
parent first would orphan its children); the least recently used one goes
first, where a lookup that matches a page and an insert that passes over it
both use it, each call counting as one tick; an ``extend`` short of free pages
first evicts just enough of them, and when even evicting every evictable page
would not be enough it evicts nothing and fails; a page is cached at most once
(an insert that would cache an already cached page under another prefix
stops there).
"""

import numpy as np


class PoolError(Exception):
    """Raised with ``kind`` 'nomem' (pool or request slots exhausted; the state
    is left unchanged) or 'inval' (bad argument)."""

    def __init__(self, kind: str, msg: str):
        super().__init__(msg)
        self.kind = kind


class _Node:
    __slots__ = ("page", "parent", "digest", "key", "n_children", "stamp", "serial")

    def __init__(self, page, parent, digest, key=None, serial=0):
        self.page = page
        self.parent = parent
        self.digest = digest      # for introspection only
        self.key = key            # its entry in PagePool.children
        self.n_children = 0
        self.stamp = 0            # tick of its last use
        self.serial = serial      # creation order


class PagePool:
    def __init__(self, mode: int, pool_slots: int, page_size: int, max_reqs: int,
                 max_ctx_len: int, page_perm=None):
        if mode not in (0, 1):
            raise PoolError("inval", "mode")
        self.mode = mode
        self.page_size = 1 if mode == 0 else int(page_size)
        self.max_reqs = int(max_reqs)
        self.max_ctx_len = int(max_ctx_len)
        self.pool_slots = int(pool_slots)
        if mode == 0 and pool_slots < max_reqs * max_ctx_len:
            raise PoolError("inval", "contiguous pool too small")
        if mode == 1 and (page_size < 1 or pool_slots % page_size):
            raise PoolError("inval", "pool_slots must be a multiple of page_size")
        self.n_pages = pool_slots // self.page_size if mode == 1 else 0
        self.perm = None if page_perm is None else [int(x) for x in page_perm]
        if self.perm is not None and sorted(self.perm) != list(range(self.n_pages)):
            raise PoolError("inval", "page_perm is not a permutation")
        self.table = np.full((self.max_reqs, self.max_ctx_len), -1, dtype=np.int32)
        self.live = [False] * self.max_reqs
        self.length = [0] * self.max_reqs
        self.pages = [[] for _ in range(self.max_reqs)]   # logical pages, position order
        self.free = [True] * self.n_pages
        self.n_free = self.n_pages
        self.first_free = 0                               # no free page below this index
        self.ref = [0] * self.n_pages
        self.children = {}                                # (parent id, token tuple) -> node
        self.root = _Node(None, None, None)
        self.node_of_page = {}                            # cached page -> its node
        self.clock = 0
        self.n_created = 0
        self.evicted = 0                                  # pages evicted so far

    # -- helpers --------------------------------------------------------------
    def _slot(self, req: int, pos: int) -> int:
        if self.mode == 0:
            return req * self.max_ctx_len + pos
        lp = self.pages[req][pos // self.page_size]
        pp = lp if self.perm is None else self.perm[lp]
        return pp * self.page_size + pos % self.page_size

    def _radix_on(self) -> bool:
        return self.mode == 1 and self.page_size > 1

    def _page_tokens(self, tokens, k):
        ps = self.page_size
        return tuple(int(t) for t in tokens[k * ps:(k + 1) * ps])

    def _check_live(self, req):
        if not (0 <= req < self.max_reqs) or not self.live[req]:
            raise PoolError("inval", f"request {req} is not live")

    # -- the calls -------------------------------------------------------------
    def admit(self, tokens=None, n_tokens: int = 0):
        """Take the lowest free request slot; match cached pages.  -> (req, cached_len)."""
        if n_tokens < 0 or n_tokens > self.max_ctx_len:
            raise PoolError("inval", "n_tokens out of range")
        try:
            req = self.live.index(False)
        except ValueError:
            raise PoolError("nomem", "no free request slot")
        matched = []
        if self._radix_on() and tokens is not None and n_tokens > 0:
            self.clock += 1
            node = self.root
            for k in range((n_tokens - 1) // self.page_size):
                child = self.children.get((id(node), self._page_tokens(tokens, k)))
                if child is None:
                    break
                child.stamp = self.clock
                matched.append(child.page)
                node = child
        self.live[req] = True
        self.pages[req] = list(matched)
        for p in matched:
            self.ref[p] += 1
        n = len(matched) * self.page_size
        self.length[req] = n
        for pos in range(n):
            self.table[req, pos] = self._slot(req, pos)
        return req, n

    def extend(self, req: int, n_new: int):
        """Give request ``req`` slots for positions [len, len + n_new)."""
        self._check_live(req)
        old = self.length[req]
        new = old + int(n_new)
        if n_new < 0 or new > self.max_ctx_len:
            raise PoolError("inval", "length exceeds max_ctx_len")
        if self.mode == 1:
            need = -(-new // self.page_size) - len(self.pages[req])
            if need > self.n_free:
                if need > self.n_free + self.evictable_pages():
                    raise PoolError("nomem", "pool exhausted")
                self.evict(need - self.n_free)
            for _ in range(max(need, 0)):
                lp = self.free.index(True, self.first_free)
                self.first_free = lp + 1
                self.n_free -= 1
                self.free[lp] = False
                self.ref[lp] = 1
                self.pages[req].append(lp)
        self.length[req] = new
        for pos in range(old, new):
            self.table[req, pos] = self._slot(req, pos)

    def bind(self, reqs, q_lens, q_tile: int = 64):
        """Per-step metadata for a batch of live requests."""
        reqs = [int(r) for r in reqs]
        q_lens = [int(x) for x in q_lens]
        if len(reqs) != len(q_lens) or q_tile < 1:
            raise PoolError("inval", "batch arguments")
        for r, ql in zip(reqs, q_lens):
            self._check_live(r)
            if ql < 0 or ql > self.length[r]:
                raise PoolError("inval", "q_len exceeds seq_len")
        seq = [self.length[r] for r in reqs]
        kv_indptr = [0]
        qo_indptr = [0]
        loc = []
        t2b, t2i = [], []
        for b, (r, L, ql) in enumerate(zip(reqs, seq, q_lens)):
            kv_indptr.append(kv_indptr[-1] + L)
            qo_indptr.append(qo_indptr[-1] + ql)
            loc.extend(int(self.table[r, p]) for p in range(L - ql, L))
            # the request's query tiles, request-major: tile t holds rows
            # [t * q_tile, min((t + 1) * q_tile, q_len)); the pages fix which
            # rows a tile holds, not the order in which tiles are listed
            for t in range(-(-ql // q_tile)):
                t2b.append(b)
                t2i.append(t)
        i32 = lambda a: np.asarray(a, dtype=np.int32)
        return dict(req_pool_indices=i32(reqs), seq_lens=i32(seq),
                    out_cache_loc=i32(loc), kv_indptr=i32(kv_indptr),
                    qo_indptr=i32(qo_indptr), q_tile_to_batch=i32(t2b),
                    q_tile_to_index=i32(t2i), num_q_tiles=len(t2b),
                    max_len=max(seq) if seq else 0)

    def insert(self, req: int, tokens, n_materialized: int):
        """Record the request's complete, materialised pages in the radix."""
        self._check_live(req)
        if not self._radix_on():
            return
        n_full = min(int(n_materialized), self.length[req]) // self.page_size
        self.clock += 1
        node = self.root
        for k in range(n_full):
            key = (id(node), self._page_tokens(tokens, k))
            child = self.children.get(key)
            if child is None:
                page = self.pages[req][k]
                if page in self.node_of_page:
                    break                 # already cached under another prefix
                child = _Node(page, node, hash(key[1]), key, self.n_created)
                self.n_created += 1
                self.children[key] = child
                self.node_of_page[page] = child
                node.n_children += 1
                self.ref[page] += 1
            child.stamp = self.clock
            node = child

    def release(self, req: int):
        """Drop the request's page references and free its request slot."""
        self._check_live(req)
        if self.mode == 1:
            for p in self.pages[req]:
                self.ref[p] -= 1
                if self.ref[p] == 0:
                    self.free[p] = True
                    self.n_free += 1
                    self.first_free = min(self.first_free, p)
        self.pages[req] = []
        self.length[req] = 0
        self.live[req] = False
        self.table[req, :] = -1

    def complete(self, req: int, tokens, n_tokens: int):
        """A finished request: ``tokens[:n_tokens]`` is its prompt plus every
        generated token, the last one sampled but never run through the model,
        so only the first n_tokens - 1 have KV; cache their complete pages, then
        release the request (its partial page with it)."""
        self._check_live(req)
        if n_tokens > 1:
            self.insert(req, tokens, n_tokens - 1)
        self.release(req)

    # -- eviction ----------------------------------------------------------------
    def _evictable_leaves(self):
        return [n for n in self.node_of_page.values()
                if n.n_children == 0 and self.ref[n.page] == 1]

    def evictable_pages(self) -> int:
        """Cached pages that repeated leaf eviction could free: those with no
        page in their cached subtree (themselves included) held by a request."""
        pinned = set()
        for n in self.node_of_page.values():
            if self.ref[n.page] > 1:
                while n is not self.root and id(n) not in pinned:
                    pinned.add(id(n))
                    n = n.parent
        return len(self.node_of_page) - len(pinned)

    def evict(self, n_pages: int) -> int:
        """Free up to n_pages cached pages, least recently used leaf first
        (ties: the earlier created); returns how many were freed."""
        done = 0
        while done < n_pages:
            leaves = self._evictable_leaves()
            if not leaves:
                break
            n = min(leaves, key=lambda x: (x.stamp, x.serial))
            del self.children[n.key]
            del self.node_of_page[n.page]
            n.parent.n_children -= 1
            self.ref[n.page] -= 1
            self.free[n.page] = True
            self.n_free += 1
            self.first_free = min(self.first_free, n.page)
            done += 1
        self.evicted += done
        return done

    def cached_pages(self) -> int:
        return len(self.node_of_page)
