"""Attention over a paged KV pool, float64.

Definitions followed:

* AstrAI docs/developer/internals.md, "Autoregression & Causal Masking":
  a lower-triangular mask, 0 where query position i may attend key position
  j <= i and -inf elsewhere (the page prints the 5 x 5 case).
* internals.md, "KV Cache Mathematics" (and docs/guides/inference.md, "KV
  Cache"): the decode output o_n = sum_j softmax(q_n k_j / sqrt(d_k)) v_j over
  every cached key of the request.
* internals.md, "Attention Backend": scale 1/sqrt(head_dim); the plain
  backend writes K/V to the cache, gathers them through ``req_to_token`` and
  runs dense scaled-dot-product attention -- the semantics written out here.
* inference.md, "KVCache System": pools ``k_buffer``/``v_buffer`` of shape
  [n_layers, size, n_kv_heads, head_dim], ``req_to_token[req, pos]`` -> slot,
  ``kv_indptr``/``qo_indptr`` prefix sums of the KV and query lengths, and the
  split-K decode partial output and max/log-sum buffers.
* AstrAI paper, "Model Architecture": grouped-query attention, fewer KV heads
  than query heads.

Readings where the pages are silent: query head h reads KV head
h // (n_heads / n_kv_heads); a request whose KV length L exceeds its query
count e has a cached prefix p = L - e and its query i (0-based) sits at
position p + i and sees keys j <= p + i; split s of a decode covers positions
[s*C, min((s+1)*C, L)) and stores the normalised partial output and the
natural-log log-sum-exp of its scaled scores.  A table entry outside the
pool names no key (the pages never produce one): that key takes no part in
the softmax, and a query with no key left gets zeros.
"""

import math

import numpy as np


# -- the mask ------------------------------------------------------------------

def causal_mask(q_len: int, prefix_len: int = 0) -> np.ndarray:
    """Additive mask [q_len, prefix_len + q_len]: 0 where key j <= prefix_len + i."""
    i = np.arange(q_len)[:, None]
    j = np.arange(prefix_len + q_len)[None, :]
    return np.where(j <= prefix_len + i, 0.0, -np.inf)


# -- dense attention -------------------------------------------------------------

def attend(q, k, v, scale: float, mask=None) -> np.ndarray:
    """softmax(q k^T * scale + mask) v for one head.

    q [M, D], k [N, D], v [N, D] -> [M, D], float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = (q @ k.T) * scale
    if mask is not None:
        s = s + mask
    mx = s.max(axis=1, keepdims=True)
    empty = np.isneginf(mx)                      # every key masked: the row is 0
    s = s - np.where(empty, 0.0, mx)
    p = np.exp(s)
    p = p / np.where(empty, 1.0, p.sum(axis=1, keepdims=True))
    return p @ v


def kv_head_of(h: int, n_heads: int, n_kv_heads: int) -> int:
    """KV head read by query head h: consecutive groups of n_heads/n_kv_heads."""
    return h // (n_heads // n_kv_heads)


def _absent(key_ok, n: int) -> np.ndarray:
    """Additive row [n]: -inf for keys that take no part (key_ok False)."""
    if key_ok is None:
        return np.zeros(n)
    return np.where(np.asarray(key_ok, dtype=bool), 0.0, -np.inf)


def decode_dense(q, k, v, scale: float, key_ok=None) -> np.ndarray:
    """One decode query per head against a request's whole KV.

    q [Hq, D], k/v [L, Hkv, D] -> [Hq, D]; key_ok [L] (default all True).
    """
    hq, hkv = q.shape[0], k.shape[1]
    mask = _absent(key_ok, k.shape[0])[None, :]
    out = np.empty(q.shape, dtype=np.float64)
    for h in range(hq):
        g = kv_head_of(h, hq, hkv)
        out[h] = attend(q[h][None, :], k[:, g], v[:, g], scale, mask)[0]
    return out


def prefill_dense(q, k, v, scale: float, key_ok=None) -> np.ndarray:
    """Causal attention of e queries over a request's L = p + e keys.

    q [e, Hq, D], k/v [L, Hkv, D] -> [e, Hq, D]; query i sees keys j <= p + i
    (and only keys with key_ok, default all).
    """
    e, hq, _ = q.shape
    L, hkv = k.shape[0], k.shape[1]
    mask = causal_mask(e, L - e) + _absent(key_ok, L)[None, :]
    out = np.empty(q.shape, dtype=np.float64)
    for h in range(hq):
        g = kv_head_of(h, hq, hkv)
        out[:, h] = attend(q[:, h], k[:, g], v[:, g], scale, mask)
    return out


# -- split-K decode and its merge ------------------------------------------------

def decode_split(q, k, v, scale: float, chunk: int):
    """Split-K partials of one decode query per head.

    q [Hq, D], k/v [L, Hkv, D] -> (o_part [Hq, S, D], lse [Hq, S]) with
    S = ceil(L / chunk).  Split s covers positions [s*chunk, min((s+1)*chunk, L)):
    its scores s_j = q.k_j * scale have maximum m and l = sum exp(s_j - m); the
    stored output is sum exp(s_j - m) v_j / l and lse = m + ln l.
    """
    hq, d = q.shape
    L, hkv = k.shape[0], k.shape[1]
    n_split = -(-L // chunk)
    o = np.zeros((hq, n_split, d))
    lse = np.full((hq, n_split), -np.inf)
    for h in range(hq):
        g = kv_head_of(h, hq, hkv)
        for s in range(n_split):
            lo, hi = s * chunk, min((s + 1) * chunk, L)
            sc = (k[lo:hi, g] @ q[h]) * scale
            m = sc.max()
            w = np.exp(sc - m)
            l_ = w.sum()
            o[h, s] = (w @ v[lo:hi, g]) / l_
            lse[h, s] = m + math.log(l_)
    return o, lse


def merge_splits(o_part, lse) -> np.ndarray:
    """Log-sum-exp merge: M = max_s lse_s, w_s = exp(lse_s - M),
    o = sum_s w_s o_s / sum_s w_s.  Splits with lse = -inf carry no weight.

    o_part [..., S, D], lse [..., S] -> [..., D].
    """
    lse = np.asarray(lse, dtype=np.float64)
    m = lse.max(axis=-1, keepdims=True)
    w = np.where(np.isneginf(lse), 0.0, np.exp(lse - m))
    return (w[..., None] * o_part).sum(axis=-2) / w.sum(axis=-1)[..., None]


# -- the paged forms: gather through req_to_token, then the dense definition ------

def gather(pool, layer: int, req_to_token, req: int, length: int):
    """(pool[layer, req_to_token[req, 0:length]] -> [length, Hkv, D], key_ok
    [length]); an entry outside the pool gathers a zero row and key_ok False."""
    slots = np.asarray(req_to_token)[req, :length].astype(np.int64)
    size = np.shape(pool)[1]
    ok = (slots >= 0) & (slots < size)
    rows = np.zeros((length,) + tuple(np.shape(pool)[2:]), dtype=np.float64)
    rows[ok] = np.asarray(pool[layer][slots[ok]], dtype=np.float64)
    return rows, ok


def paged_decode(q, k_pool, v_pool, layer: int, req_to_token, req_pool_indices,
                 kv_indptr, scale: float) -> np.ndarray:
    """Decode attention for a batch: q [B, Hq, D] -> [B, Hq, D]."""
    out = np.empty(np.shape(q), dtype=np.float64)
    for b in range(len(req_pool_indices)):
        L = int(kv_indptr[b + 1] - kv_indptr[b])
        r = int(req_pool_indices[b])
        k, ok = gather(k_pool, layer, req_to_token, r, L)
        v, _ = gather(v_pool, layer, req_to_token, r, L)
        out[b] = decode_dense(np.asarray(q[b], dtype=np.float64), k, v, scale, ok)
    return out


def paged_prefill(q, k_pool, v_pool, layer: int, req_to_token, req_pool_indices,
                  qo_indptr, kv_indptr, scale: float) -> np.ndarray:
    """Ragged causal prefill: q [sum e_b, Hq, D] in qo_indptr order -> same shape."""
    out = np.empty(np.shape(q), dtype=np.float64)
    for b in range(len(req_pool_indices)):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        L = int(kv_indptr[b + 1] - kv_indptr[b])
        r = int(req_pool_indices[b])
        k, ok = gather(k_pool, layer, req_to_token, r, L)
        v, _ = gather(v_pool, layer, req_to_token, r, L)
        out[q0:q1] = prefill_dense(np.asarray(q[q0:q1], dtype=np.float64), k, v, scale, ok)
    return out
