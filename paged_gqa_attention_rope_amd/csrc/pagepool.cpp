// Host page-table builder: KVStorage slot allocation, the request-to-token
// table, reference-counted pages and the exact page-aligned radix cache
// (AstrAI docs/guides/inference.md, "KVCache System"; docs/developer/
// internals.md, "Cache Architecture").  Host memory only; no device calls.
//
// Allocation is deterministic: lowest free request slot, lowest free logical
// page (a bitmask scanned word by word), logical -> physical through an
// optional permutation.  The radix keys a child by (parent node, 64-bit FNV-1a
// digest of the page's tokens) only to find candidates; a match always
// compares the stored token tuple exactly, so the digest never decides it.
//
// Lifecycle: a finished request caches the complete pages of its prompt and
// of the generated tokens already decoded into KV (the final sampled token
// has none), then releases everything else.  Under pool pressure the
// allocator evicts cached pages that only the radix holds, least recently
// used leaf first: a leaf, because evicting a parent would orphan its cached
// children; recency is a tick per lookup or insert call, given to every node
// the call passes over.  An extend evicts only when it must, and nothing at
// all when evicting every evictable page would still leave it short.
#include <cstdint>
#include <algorithm>
#include <array>
#include <cstring>
#include <new>
#include <set>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "astr.h"
#include "status.hpp"

namespace {

struct Node {
    int32_t page = -1;            // logical page id (-1: the slot is unused)
    int32_t parent = -1;          // node index, -1 for children of the root
    int32_t n_children = 0;
    uint64_t digest = 0;          // FNV-1a of the page's tokens (introspection, bucketing)
    uint64_t stamp = 0;           // tick of its last use
    uint64_t serial = 0;          // creation order
    bool in_lru = false;          // listed in astr_pagepool::lru
    std::vector<int32_t> tokens;  // the exact page contents
};

using LruKey = std::tuple<uint64_t, uint64_t, int32_t>;   // (stamp, serial, node)

struct KeyHash {
    size_t operator()(const std::pair<int32_t, uint64_t> &k) const {
        return static_cast<size_t>(k.second ^ (static_cast<uint64_t>(k.first) * 0x9E3779B97F4A7C15ull));
    }
};

uint64_t fnv1a(const int32_t *t, int n) {
    uint64_t h = 0xcbf29ce484222325ull;
    for (int i = 0; i < n; ++i) {
        uint32_t x = static_cast<uint32_t>(t[i]);
        for (int b = 0; b < 4; ++b) {
            h ^= (x >> (8 * b)) & 0xffu;
            h *= 0x100000001b3ull;
        }
    }
    return h;
}

}  // namespace

struct astr_pagepool {
    int mode = 0;
    int page_size = 1;
    int max_reqs = 0;
    int max_ctx_len = 0;
    int64_t pool_slots = 0;
    int64_t n_pages = 0;
    std::vector<int32_t> perm;            // logical -> physical (empty = identity)
    std::vector<int32_t> table;           // [max_reqs, max_ctx_len]
    std::vector<uint8_t> live;
    std::vector<int32_t> length;
    std::vector<std::vector<int32_t>> pages;   // logical pages of each request, in position order
    std::vector<uint64_t> free_bits;      // bit set = page free
    int64_t free_count = 0;
    int64_t free_hint = 0;                // no free page below word free_hint
    std::vector<int32_t> ref;
    std::vector<Node> nodes;
    std::vector<int32_t> free_nodes;      // unused slots of nodes
    std::unordered_map<std::pair<int32_t, uint64_t>, std::vector<int32_t>, KeyHash> children;
    std::vector<int32_t> node_of_page;    // cached page -> node (-1: not cached)
    std::set<LruKey> lru;                 // evictable leaves, least recently used first
    int64_t cached = 0;                   // pages held by the radix
    int64_t evicted = 0;                  // pages evicted so far
    uint64_t clock = 0;
    uint64_t n_created = 0;

    bool radix_on() const { return mode == 1 && page_size > 1; }

    // keep node n listed in lru exactly when it is an evictable leaf
    void refresh(int32_t n) {
        Node &nd = nodes[n];
        if (nd.in_lru) {
            lru.erase(LruKey{nd.stamp, nd.serial, n});
            nd.in_lru = false;
        }
        if (nd.page >= 0 && nd.n_children == 0 && ref[nd.page] == 1) {
            lru.insert(LruKey{nd.stamp, nd.serial, n});
            nd.in_lru = true;
        }
    }

    void touch(int32_t n) {
        if (nodes[n].stamp == clock) return;
        if (nodes[n].in_lru) lru.erase(LruKey{nodes[n].stamp, nodes[n].serial, n});
        nodes[n].stamp = clock;
        if (nodes[n].in_lru) lru.insert(LruKey{nodes[n].stamp, nodes[n].serial, n});
    }

    // a page's reference count changed: its node may enter or leave lru
    void ref_changed(int32_t page) {
        if (node_of_page.empty()) return;
        int32_t n = node_of_page[page];
        if (n >= 0) refresh(n);
    }

    // cached pages that repeated leaf eviction could free: those whose cached
    // subtree (themselves included) holds no page a request still holds
    int64_t evictable_pages() const {
        std::vector<uint8_t> pinned(nodes.size(), 0);
        int64_t n_pinned = 0;
        for (size_t i = 0; i < nodes.size(); ++i) {
            if (nodes[i].page < 0 || ref[nodes[i].page] <= 1) continue;
            for (int32_t n = static_cast<int32_t>(i); n >= 0 && !pinned[n]; n = nodes[n].parent) {
                pinned[n] = 1;
                ++n_pinned;
            }
        }
        return cached - n_pinned;
    }

    int64_t evict(int64_t want) {
        int64_t done = 0;
        while (done < want && !lru.empty()) {
            const int32_t n = std::get<2>(*lru.begin());
            lru.erase(lru.begin());
            Node &nd = nodes[n];
            nd.in_lru = false;
            auto it = children.find({nd.parent, nd.digest});
            auto &bucket = it->second;
            bucket.erase(std::find(bucket.begin(), bucket.end(), n));
            if (bucket.empty()) children.erase(it);
            const int32_t page = nd.page, parent = nd.parent;
            node_of_page[page] = -1;
            nd.page = -1;
            nd.tokens.clear();
            free_nodes.push_back(n);
            --cached;
            if (--ref[page] == 0) give_back_page(page);
            if (parent >= 0) {
                --nodes[parent].n_children;
                refresh(parent);
            }
            ++done;
        }
        evicted += done;
        return done;
    }

    int64_t slot_of(int req, int pos) const {
        if (mode == 0) return static_cast<int64_t>(req) * max_ctx_len + pos;
        int32_t lp = pages[req][pos / page_size];
        int64_t pp = perm.empty() ? lp : perm[lp];
        return pp * page_size + pos % page_size;
    }

    int64_t take_lowest_page() {
        for (int64_t w = free_hint; w < static_cast<int64_t>(free_bits.size()); ++w) {
            if (free_bits[w]) {
                int bit = __builtin_ctzll(free_bits[w]);
                free_bits[w] &= ~(1ull << bit);
                free_hint = w;
                --free_count;
                return w * 64 + bit;
            }
        }
        return -1;
    }

    void give_back_page(int64_t p) {
        free_bits[p / 64] |= 1ull << (p % 64);
        if (p / 64 < free_hint) free_hint = p / 64;
        ++free_count;
    }

    int find_child(int32_t parent, const int32_t *tok) const {
        auto it = children.find({parent, fnv1a(tok, page_size)});
        if (it == children.end()) return -1;
        for (int32_t n : it->second) {
            if (nodes[n].parent == parent &&
                std::memcmp(nodes[n].tokens.data(), tok, sizeof(int32_t) * page_size) == 0)
                return n;
        }
        return -1;
    }
};

static int check_live(const astr_pagepool *pp, int req) {
    if (!pp) return astr::fail(ASTR_E_INVAL, "pagepool: null handle");
    if (req < 0 || req >= pp->max_reqs || !pp->live[req])
        return astr::fail(ASTR_E_INVAL, "pagepool: request %d is not live", req);
    return ASTR_OK;
}

extern "C" int astr_pagepool_create(astr_pagepool **out, int mode, int64_t pool_slots, int page_size,
                                    int max_reqs, int max_ctx_len, const int32_t *page_perm) {
    if (!out) return astr::fail(ASTR_E_INVAL, "pagepool_create: null out");
    *out = nullptr;
    if (mode != 0 && mode != 1) return astr::fail(ASTR_E_INVAL, "pagepool_create: mode %d", mode);
    if (max_reqs < 1 || max_ctx_len < 1 || pool_slots < 1)
        return astr::fail(ASTR_E_INVAL, "pagepool_create: sizes must be positive");
    if (mode == 0 && pool_slots < static_cast<int64_t>(max_reqs) * max_ctx_len)
        return astr::fail(ASTR_E_INVAL, "pagepool_create: contiguous pool needs max_reqs*max_ctx_len slots");
    if (mode == 1 && (page_size < 1 || pool_slots % page_size != 0))
        return astr::fail(ASTR_E_INVAL, "pagepool_create: pool_slots must be a multiple of page_size");
    if (mode == 1 && pool_slots / page_size > INT32_MAX)
        return astr::fail(ASTR_E_INVAL, "pagepool_create: too many pages");
    astr_pagepool *pp = new (std::nothrow) astr_pagepool();
    if (!pp) return astr::fail(ASTR_E_NOMEM, "pagepool_create: host allocation");
    try {
        pp->mode = mode;
        pp->page_size = mode == 0 ? 1 : page_size;
        pp->max_reqs = max_reqs;
        pp->max_ctx_len = max_ctx_len;
        pp->pool_slots = pool_slots;
        pp->n_pages = mode == 1 ? pool_slots / page_size : 0;
        pp->table.assign(static_cast<size_t>(max_reqs) * max_ctx_len, -1);
        pp->live.assign(max_reqs, 0);
        pp->length.assign(max_reqs, 0);
        pp->pages.assign(max_reqs, {});
        if (mode == 1) {
            pp->free_bits.assign((pp->n_pages + 63) / 64, 0);
            for (int64_t p = 0; p < pp->n_pages; ++p) pp->free_bits[p / 64] |= 1ull << (p % 64);
            pp->free_count = pp->n_pages;
            pp->ref.assign(pp->n_pages, 0);
            if (pp->radix_on()) pp->node_of_page.assign(pp->n_pages, -1);
            if (page_perm) {
                pp->perm.assign(page_perm, page_perm + pp->n_pages);
                std::vector<uint8_t> seen(pp->n_pages, 0);
                for (int64_t i = 0; i < pp->n_pages; ++i) {
                    int32_t x = pp->perm[i];
                    if (x < 0 || x >= pp->n_pages || seen[x]) {
                        delete pp;
                        return astr::fail(ASTR_E_INVAL, "pagepool_create: page_perm is not a permutation");
                    }
                    seen[x] = 1;
                }
            }
        }
    } catch (const std::bad_alloc &) {
        delete pp;
        return astr::fail(ASTR_E_NOMEM, "pagepool_create: host allocation");
    }
    *out = pp;
    return ASTR_OK;
}

extern "C" void astr_pagepool_destroy(astr_pagepool *pp) { delete pp; }

extern "C" int astr_pagepool_admit(astr_pagepool *pp, const int32_t *tokens, int n_tokens,
                                   int *req_idx, int *cached_len) {
    if (!pp || !req_idx || !cached_len) return astr::fail(ASTR_E_INVAL, "pagepool_admit: null argument");
    if (n_tokens < 0 || n_tokens > pp->max_ctx_len)
        return astr::fail(ASTR_E_INVAL, "pagepool_admit: n_tokens %d outside [0, %d]", n_tokens, pp->max_ctx_len);
    int req = -1;
    for (int r = 0; r < pp->max_reqs; ++r) {
        if (!pp->live[r]) { req = r; break; }
    }
    if (req < 0) return astr::fail(ASTR_E_NOMEM, "pagepool_admit: no free request slot");
    std::vector<int32_t> matched;
    if (pp->radix_on() && tokens && n_tokens > 0) {
        ++pp->clock;
        int32_t parent = -1;
        int max_pages = (n_tokens - 1) / pp->page_size;
        for (int k = 0; k < max_pages; ++k) {
            int n = pp->find_child(parent, tokens + static_cast<size_t>(k) * pp->page_size);
            if (n < 0) break;
            pp->touch(n);
            matched.push_back(pp->nodes[n].page);
            parent = n;
        }
    }
    pp->live[req] = 1;
    pp->pages[req] = matched;
    for (int32_t p : matched) {
        ++pp->ref[p];
        pp->ref_changed(p);
    }
    int len = static_cast<int>(matched.size()) * pp->page_size;
    pp->length[req] = len;
    int32_t *row = pp->table.data() + static_cast<size_t>(req) * pp->max_ctx_len;
    for (int pos = 0; pos < len; ++pos) row[pos] = static_cast<int32_t>(pp->slot_of(req, pos));
    *req_idx = req;
    *cached_len = len;
    return ASTR_OK;
}

extern "C" int astr_pagepool_extend(astr_pagepool *pp, int req_idx, int n_new) {
    int st = check_live(pp, req_idx);
    if (st) return st;
    int old = pp->length[req_idx];
    if (n_new < 0 || static_cast<int64_t>(old) + n_new > pp->max_ctx_len)
        return astr::fail(ASTR_E_INVAL, "pagepool_extend: length %lld exceeds max_ctx_len %d",
                          static_cast<long long>(old) + n_new, pp->max_ctx_len);
    int nw = old + n_new;
    if (pp->mode == 1) {
        int64_t need = (static_cast<int64_t>(nw) + pp->page_size - 1) / pp->page_size -
                       static_cast<int64_t>(pp->pages[req_idx].size());
        if (need > pp->free_count) {
            const int64_t can = pp->radix_on() ? pp->evictable_pages() : 0;
            if (need > pp->free_count + can)
                return astr::fail(ASTR_E_NOMEM, "pagepool_extend: need %lld pages, %lld free, %lld evictable",
                                  static_cast<long long>(need), static_cast<long long>(pp->free_count),
                                  static_cast<long long>(can));
            pp->evict(need - pp->free_count);
        }
        for (int64_t i = 0; i < need; ++i) {
            int64_t lp = pp->take_lowest_page();
            pp->ref[lp] = 1;
            pp->pages[req_idx].push_back(static_cast<int32_t>(lp));
        }
    }
    pp->length[req_idx] = nw;
    int32_t *row = pp->table.data() + static_cast<size_t>(req_idx) * pp->max_ctx_len;
    for (int pos = old; pos < nw; ++pos) row[pos] = static_cast<int32_t>(pp->slot_of(req_idx, pos));
    return ASTR_OK;
}

extern "C" int astr_pagepool_bind(astr_pagepool *pp, const int32_t *req_idx, const int32_t *q_lens,
                                  int batch, int q_tile, int32_t *seq_lens, int32_t *out_cache_loc,
                                  int32_t *kv_indptr, int32_t *qo_indptr, int32_t *q_tile_to_batch,
                                  int32_t *q_tile_to_index, int tile_capacity, int *num_q_tiles,
                                  int *max_len) {
    if (!pp || batch < 0 || (batch > 0 && (!req_idx || !q_lens)) || !seq_lens || !kv_indptr ||
        !qo_indptr || !num_q_tiles || !max_len || q_tile < 1 || tile_capacity < 0)
        return astr::fail(ASTR_E_INVAL, "pagepool_bind: bad argument");
    if (tile_capacity > 0 && (!q_tile_to_batch || !q_tile_to_index))
        return astr::fail(ASTR_E_INVAL, "pagepool_bind: null tile arrays");
    int64_t n_tiles = 0, total_q = 0;
    for (int b = 0; b < batch; ++b) {
        int st = check_live(pp, req_idx[b]);
        if (st) return st;
        if (q_lens[b] < 0 || q_lens[b] > pp->length[req_idx[b]])
            return astr::fail(ASTR_E_INVAL, "pagepool_bind: q_len %d of entry %d exceeds its length %d",
                              q_lens[b], b, pp->length[req_idx[b]]);
        n_tiles += (q_lens[b] + q_tile - 1) / q_tile;
        total_q += q_lens[b];
    }
    if (total_q > 0 && !out_cache_loc) return astr::fail(ASTR_E_INVAL, "pagepool_bind: null out_cache_loc");
    if (tile_capacity > 0 && n_tiles > tile_capacity)
        return astr::fail(ASTR_E_INVAL, "pagepool_bind: %lld tiles exceed capacity %d",
                          static_cast<long long>(n_tiles), tile_capacity);
    kv_indptr[0] = 0;
    qo_indptr[0] = 0;
    int mx = 0;
    int64_t w = 0;
    // query tiles, each with the KV extent its last row sees
    struct Tile {
        int32_t extent, b, idx;
    };
    std::vector<Tile> tiles;
    try {
        tiles.reserve(static_cast<size_t>(n_tiles));
    } catch (const std::bad_alloc &) {
        return astr::fail(ASTR_E_NOMEM, "pagepool_bind: host allocation");
    }
    for (int b = 0; b < batch; ++b) {
        int r = req_idx[b];
        int L = pp->length[r];
        int ql = q_lens[b];
        seq_lens[b] = L;
        kv_indptr[b + 1] = kv_indptr[b] + L;
        qo_indptr[b + 1] = qo_indptr[b] + ql;
        if (L > mx) mx = L;
        const int32_t *row = pp->table.data() + static_cast<size_t>(r) * pp->max_ctx_len;
        for (int pos = L - ql; pos < L; ++pos) out_cache_loc[w++] = row[pos];
        for (int i = 0; i * q_tile < ql; ++i) {
            const int last = (i + 1) * q_tile < ql ? (i + 1) * q_tile : ql;
            tiles.push_back({L - ql + last, b, i});
        }
    }
    // longest first (ties: request, then tile index), so that an attention
    // launch can hand out the heaviest tiles first
    std::stable_sort(tiles.begin(), tiles.end(),
                     [](const Tile &x, const Tile &y) { return x.extent > y.extent; });
    if (tile_capacity > 0) {
        for (size_t t = 0; t < tiles.size(); ++t) {
            q_tile_to_batch[t] = tiles[t].b;
            q_tile_to_index[t] = tiles[t].idx;
        }
    }
    *num_q_tiles = static_cast<int>(n_tiles);
    *max_len = mx;
    return ASTR_OK;
}

extern "C" int astr_pagepool_insert(astr_pagepool *pp, int req_idx, const int32_t *tokens,
                                    int n_materialized) {
    int st = check_live(pp, req_idx);
    if (st) return st;
    if (!pp->radix_on()) return ASTR_OK;
    if (n_materialized < 0 || (n_materialized > 0 && !tokens))
        return astr::fail(ASTR_E_INVAL, "pagepool_insert: bad tokens");
    int n = n_materialized < pp->length[req_idx] ? n_materialized : pp->length[req_idx];
    int full = n / pp->page_size;
    ++pp->clock;
    int32_t parent = -1;
    try {
        for (int k = 0; k < full; ++k) {
            const int32_t *tok = tokens + static_cast<size_t>(k) * pp->page_size;
            int c = pp->find_child(parent, tok);
            if (c < 0) {
                const int32_t page = pp->pages[req_idx][k];
                if (pp->node_of_page[page] >= 0) break;   // already cached under another prefix
                if (pp->free_nodes.empty()) {
                    pp->nodes.emplace_back();
                    pp->free_nodes.push_back(static_cast<int32_t>(pp->nodes.size() - 1));
                }
                const uint64_t digest = fnv1a(tok, pp->page_size);
                auto &bucket = pp->children[{parent, digest}];
                bucket.reserve(bucket.size() + 1);
                c = pp->free_nodes.back();
                Node &nd = pp->nodes[c];
                nd.tokens.assign(tok, tok + pp->page_size);
                pp->free_nodes.pop_back();          // nothing below throws
                bucket.push_back(c);
                nd.page = page;
                nd.parent = parent;
                nd.n_children = 0;
                nd.digest = digest;
                nd.stamp = pp->clock;
                nd.serial = pp->n_created++;
                nd.in_lru = false;
                pp->node_of_page[page] = c;
                ++pp->cached;
                ++pp->ref[page];
                if (parent >= 0) {
                    ++pp->nodes[parent].n_children;
                    pp->refresh(parent);
                }
                pp->refresh(c);
            } else {
                pp->touch(c);
            }
            parent = c;
        }
    } catch (const std::bad_alloc &) {
        return astr::fail(ASTR_E_NOMEM, "pagepool_insert: host allocation");
    }
    return ASTR_OK;
}

extern "C" int astr_pagepool_release(astr_pagepool *pp, int req_idx) {
    int st = check_live(pp, req_idx);
    if (st) return st;
    if (pp->mode == 1) {
        for (int32_t p : pp->pages[req_idx]) {
            if (--pp->ref[p] == 0) pp->give_back_page(p);
            pp->ref_changed(p);
        }
    }
    pp->pages[req_idx].clear();
    pp->length[req_idx] = 0;
    pp->live[req_idx] = 0;
    int32_t *row = pp->table.data() + static_cast<size_t>(req_idx) * pp->max_ctx_len;
    for (int i = 0; i < pp->max_ctx_len; ++i) row[i] = -1;
    return ASTR_OK;
}

extern "C" int astr_pagepool_complete(astr_pagepool *pp, int req_idx, const int32_t *tokens, int n_tokens) {
    int st = check_live(pp, req_idx);
    if (st) return st;
    if (n_tokens < 0 || (n_tokens > 0 && !tokens))
        return astr::fail(ASTR_E_INVAL, "pagepool_complete: bad tokens");
    if (n_tokens > 1) {
        st = astr_pagepool_insert(pp, req_idx, tokens, n_tokens - 1);
        if (st) return st;
    }
    return astr_pagepool_release(pp, req_idx);
}

extern "C" int64_t astr_pagepool_evict(astr_pagepool *pp, int64_t n_pages) {
    if (!pp || n_pages < 0) {
        astr::fail(ASTR_E_INVAL, "pagepool_evict: bad argument");
        return -1;
    }
    return pp->radix_on() ? pp->evict(n_pages) : 0;
}

extern "C" int64_t astr_pagepool_cached_pages(const astr_pagepool *pp) { return pp ? pp->cached : -1; }

extern "C" int64_t astr_pagepool_evicted_pages(const astr_pagepool *pp) { return pp ? pp->evicted : -1; }

extern "C" const int32_t *astr_pagepool_table(const astr_pagepool *pp) {
    return pp ? pp->table.data() : nullptr;
}

extern "C" int64_t astr_pagepool_free_pages(const astr_pagepool *pp) {
    return pp ? pp->free_count : -1;
}

extern "C" int astr_pagepool_page_ref(const astr_pagepool *pp, int64_t logical_page) {
    if (!pp || logical_page < 0 || logical_page >= pp->n_pages) return -1;
    return pp->ref[logical_page];
}

extern "C" int astr_decode_split_items(const int32_t *seq_lens, int batch, int split_chunk, int32_t *item_batch,
                                       int32_t *item_index, int capacity, int *num_items) {
    if (!seq_lens || !num_items || batch < 0 || split_chunk < 1 || capacity < 0 ||
        (capacity > 0 && (!item_batch || !item_index)))
        return astr::fail(ASTR_E_INVAL, "decode_split_items: bad argument");
    int64_t total = 0;
    for (int b = 0; b < batch; ++b) {
        if (seq_lens[b] < 0) return astr::fail(ASTR_E_INVAL, "decode_split_items: seq_lens[%d] < 0", b);
        total += std::max<int64_t>(1, (static_cast<int64_t>(seq_lens[b]) + split_chunk - 1) / split_chunk);
    }
    if (total > capacity)
        return astr::fail(ASTR_E_INVAL, "decode_split_items: %lld items, capacity %d",
                          static_cast<long long>(total), capacity);
    // full splits (every split but the last) in batch order
    int n = 0;
    for (int b = 0; b < batch; ++b) {
        const int ns = std::max(1, (seq_lens[b] + split_chunk - 1) / split_chunk);
        for (int s = 0; s + 1 < ns; ++s) {
            item_batch[n] = b;
            item_index[n] = s;
            ++n;
        }
    }
    // each entry's last split, longest first, ties by batch entry
    std::vector<std::pair<int, int>> last;      // (-length of the last split, b)
    last.reserve(batch);
    for (int b = 0; b < batch; ++b) {
        const int ns = std::max(1, (seq_lens[b] + split_chunk - 1) / split_chunk);
        last.emplace_back(-(seq_lens[b] - (ns - 1) * split_chunk), b);
    }
    std::sort(last.begin(), last.end());
    for (const auto &e : last) {
        const int b = e.second;
        item_batch[n] = b;
        item_index[n] = std::max(1, (seq_lens[b] + split_chunk - 1) / split_chunk) - 1;
        ++n;
    }
    *num_items = n;
    return ASTR_OK;
}

// ---------------------------------------------------------------------------
// Prefill work plan: which query tiles to split by keys, and on which XCD and
// in which order the units run.  The cost model and the rule are the ones
// documented with astr_prefill_plan.
// ---------------------------------------------------------------------------
namespace {

constexpr int kPlanXcds = 8;               // the prefill kernel deals units to 8 XCDs
constexpr int kPlanStep = 32;              // keys per step of the kernel
constexpr double kWhole = 7.0;             // per whole tile: prologue and output, in steps
constexpr double kLower = 8.5;             // lower half: prologue and publishing its state
constexpr double kUpper = 9.5;             // upper half: prologue, merge and output
constexpr double kEmpty = 0.1;             // a tile the kernel skips
constexpr int kJoinCap = 4;                // most units of one request an XCD takes by preference

struct PlanUnit {
    double cost;
    int tile, piece;                       // piece -1: whole tile (or padding when tile is -1)
    int lo, hi;                            // key steps [lo, hi)
    int group;                             // the tile's batch entry (its request)
};

// Units of the tiles, those marked in `split` cut in two halves at h =
// max(1, floor(n * num / den)) steps, by decreasing cost (ties: tile order,
// then lower half first).
std::vector<PlanUnit> plan_units(const std::vector<int> &steps, const std::vector<int> &group,
                                 const std::vector<char> &split, int num, int den) {
    std::vector<PlanUnit> list;
    list.reserve(2 * steps.size());
    for (int t = 0; t < static_cast<int>(steps.size()); ++t) {
        const int n = steps[t];
        if (split[t] && n >= 2) {
            const int h = std::max(1, static_cast<int>(static_cast<int64_t>(n) * num / den));
            list.push_back({kLower + h, t, 0, 0, h, group[t]});
            list.push_back({kUpper + (n - h), t, 1, h, INT32_MAX, group[t]});
        } else {
            list.push_back({n > 0 ? kWhole + n : kEmpty, t, -1, 0, INT32_MAX, group[t]});
        }
    }
    std::stable_sort(list.begin(), list.end(), [](const PlanUnit &a, const PlanUnit &b) {
        if (a.cost != b.cost) return a.cost > b.cost;
        if (a.tile != b.tile) return a.tile < b.tile;
        return a.piece < b.piece;
    });
    return list;
}

// Deal a cost-ordered list to the XCDs: each unit goes to an XCD where it
// would end first; among those, one that already holds at least one and
// fewer than kJoinCap units of the same request comes first (it can serve
// the request's keys and values from its own L2), then the one with fewer
// units queued, then the lower XCD.  An XCD runs its queue in order on
// cus_per_xcd compute units, one workgroup per compute unit, the unit's
// wg_per_unit workgroups on the ones free first.  Returns the simulated end;
// queue[x] receives the units of XCD x.
double deal(const std::vector<PlanUnit> &list, int wg_per_unit, int cus_per_xcd, int groups,
            std::vector<std::vector<int>> &queue) {
    // free times of each XCD's compute units, ascending
    std::vector<std::vector<double>> free_at(kPlanXcds, std::vector<double>(cus_per_xcd, 0.0));
    std::vector<double> merged(cus_per_xcd);
    // units of each request dealt to each XCD so far
    std::vector<std::vector<int>> holds(kPlanXcds, std::vector<int>(std::max(groups, 1), 0));
    queue.assign(kPlanXcds, {});
    const int wg = std::min(wg_per_unit, cus_per_xcd);
    double end = 0.0;
    for (int i = 0; i < static_cast<int>(list.size()); ++i) {
        const double c = list[i].cost;
        const int grp = list[i].group;
        int best = -1;
        double best_end = 0.0;
        bool best_joins = false;
        for (int x = 0; x < kPlanXcds; ++x) {
            // the unit's last workgroup starts when its wg-th compute unit frees
            const double e = free_at[x][wg - 1] + c;
            const bool joins = grp >= 0 && holds[x][grp] > 0 && holds[x][grp] < kJoinCap;
            bool take = best < 0 || e < best_end;
            if (!take && e == best_end)
                take = (joins && !best_joins) ||
                       (joins == best_joins && queue[x].size() < queue[best].size());
            if (take) {
                best = x;
                best_end = e;
                best_joins = joins;
            }
        }
        if (grp >= 0) ++holds[best][grp];
        // the k compute units free first take a workgroup each: their times
        // grow by c and merge back into the sorted rest
        std::vector<double> &f = free_at[best];
        for (int left = wg_per_unit; left > 0;) {
            const int k = std::min(left, cus_per_xcd);
            end = std::max(end, f[k - 1] + c);
            for (int w = 0; w < k; ++w) f[w] += c;
            std::merge(f.begin(), f.begin() + k, f.begin() + k, f.end(), merged.begin());
            f.swap(merged);
            left -= k;
        }
        queue[best].push_back(i);
    }
    return end;
}

}  // namespace

extern "C" int astr_prefill_plan(const int32_t *qo_indptr, const int32_t *kv_indptr,
                                 const int32_t *req_pool_indices, int batch, const int32_t *q_tile_to_batch,
                                 const int32_t *q_tile_to_index, int num_q_tiles, int q_tile,
                                 int workgroups_per_tile, int num_cus, int32_t *units, int capacity,
                                 int *num_units, int *num_pairs) {
    if (!qo_indptr || !kv_indptr || !req_pool_indices || !num_units || !num_pairs || batch < 0 || num_q_tiles < 0 ||
        q_tile < 1 || workgroups_per_tile < 1 || num_cus < kPlanXcds || capacity < 0 ||
        (num_q_tiles > 0 && (!q_tile_to_batch || !q_tile_to_index || !units)))
        return astr::fail(ASTR_E_INVAL, "prefill_plan: bad argument");
    // key steps seen by each tile (0 for a tile the kernel skips), and its
    // request row, first query row, rows and first row's position
    std::vector<int> steps(num_q_tiles, 0), group(num_q_tiles, -1);
    std::vector<std::array<int32_t, 4>> rows_of(num_q_tiles, {0, 0, 0, 0});
    int max_steps = 0;
    for (int t = 0; t < num_q_tiles; ++t) {
        const int b = q_tile_to_batch[t];
        const int64_t idx = q_tile_to_index[t];
        if (b < 0 || b >= batch || idx < 0) continue;
        const int64_t e = static_cast<int64_t>(qo_indptr[b + 1]) - qo_indptr[b];
        const int64_t p = static_cast<int64_t>(kv_indptr[b + 1]) - kv_indptr[b] - e;
        const int64_t row0 = idx * q_tile;
        if (e <= 0 || p < 0 || row0 >= e) continue;
        const int64_t rows = std::min<int64_t>(q_tile, e - row0);
        const int64_t kv_end = p + row0 + rows;
        const int64_t q_row = qo_indptr[b] + row0;
        if (kv_end > INT32_MAX || q_row > INT32_MAX) continue;
        steps[t] = static_cast<int>((kv_end + kPlanStep - 1) / kPlanStep);
        group[t] = b;
        rows_of[t] = {req_pool_indices[b], static_cast<int32_t>(q_row), static_cast<int32_t>(rows),
                      static_cast<int32_t>(p + row0)};
        max_steps = std::max(max_steps, steps[t]);
    }
    const int cus_per_xcd = num_cus / kPlanXcds;
    // candidate split sets: every tile above a fraction of the longest, cut
    // in the middle, and the N longest tiles, cut at 3/10 of their steps
    std::vector<int> by_len(num_q_tiles);
    for (int t = 0; t < num_q_tiles; ++t) by_len[t] = t;
    std::stable_sort(by_len.begin(), by_len.end(), [&](int a, int b) { return steps[a] > steps[b]; });
    struct Candidate {
        std::vector<char> split;
        int num, den;
    };
    std::vector<Candidate> cands;
    for (int k = 9; k >= 3; --k) {
        const int64_t thr = static_cast<int64_t>(max_steps) * k / 10;
        Candidate c{std::vector<char>(num_q_tiles, 0), 1, 2};
        for (int t = 0; t < num_q_tiles; ++t) c.split[t] = steps[t] > thr;
        cands.push_back(std::move(c));
    }
    for (int top : {1, 2, 3, 4, 5, 6, 8, 10, 12, 16}) {
        if (top >= num_q_tiles) break;
        Candidate c{std::vector<char>(num_q_tiles, 0), 3, 10};
        for (int i = 0; i < top; ++i) c.split[by_len[i]] = 1;
        cands.push_back(std::move(c));
    }
    std::vector<std::vector<int>> queue, cand_queue;
    std::vector<PlanUnit> best = plan_units(steps, group, std::vector<char>(num_q_tiles, 0), 1, 2);
    const double base_end = deal(best, workgroups_per_tile, cus_per_xcd, batch, queue);
    double best_end = base_end;
    std::vector<PlanUnit> chosen;
    std::vector<std::vector<int>> chosen_queue;
    for (const Candidate &c : cands) {
        std::vector<PlanUnit> cand = plan_units(steps, group, c.split, c.num, c.den);
        const double end = deal(cand, workgroups_per_tile, cus_per_xcd, batch, cand_queue);
        if (end < best_end) {
            best_end = end;
            chosen.swap(cand);
            chosen_queue.swap(cand_queue);
        }
    }
    if (!chosen.empty() && best_end <= 0.90 * base_end) {
        best.swap(chosen);
        queue.swap(chosen_queue);
    }
    // position 8k + x holds the k-th unit of XCD x; shorter queues are padded
    size_t len = 0;
    for (const auto &q : queue) len = std::max(len, q.size());
    const int64_t n = static_cast<int64_t>(len) * kPlanXcds;
    if (n > capacity)
        return astr::fail(ASTR_E_INVAL, "prefill_plan: %lld units, capacity %d", static_cast<long long>(n), capacity);
    std::vector<int> pair_of(num_q_tiles, -1);
    int pairs = 0;
    for (size_t k = 0; k < len; ++k) {
        for (int x = 0; x < kPlanXcds; ++x) {
            int32_t *row = units + 8 * (kPlanXcds * k + x);
            if (k >= queue[x].size()) {
                row[0] = -1, row[1] = 0, row[2] = 0, row[3] = -1;
                row[4] = row[5] = row[6] = row[7] = 0;
                continue;
            }
            const PlanUnit &u = best[queue[x][k]];
            int pw = -1;
            if (u.piece >= 0) {
                if (pair_of[u.tile] < 0) pair_of[u.tile] = pairs++;
                pw = 2 * pair_of[u.tile] + u.piece;
            }
            row[0] = u.tile, row[1] = u.lo, row[2] = u.hi, row[3] = pw;
            for (int f = 0; f < 4; ++f) row[4 + f] = rows_of[u.tile][f];
        }
    }
    *num_units = static_cast<int>(n);
    *num_pairs = pairs;
    return ASTR_OK;
}
