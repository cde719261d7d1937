"""Pins for the oracle's attention (CPU only).

Facts used: the printed 5x5 causal mask and the decode formula
o_n = sum_j softmax(q_n k_j / sqrt(d_k)) v_j (AstrAI docs/developer/internals.md,
"Autoregression & Causal Masking" and "KV Cache Mathematics"); scale
1/sqrt(head_dim) and the gather-then-dense-attention semantics of the plain
backend (internals.md, "Attention Backend").  Independent routes: brute-force
Python loops on tiny inputs, torch's scaled_dot_product_attention on the CPU in
float64 (with its grouped-query expansion and its lower-right causal bias),
scipy's logsumexp, closed forms.
"""

import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp
from torch.nn.attention.bias import causal_lower_right

from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "causal_mask_5x5.txt")


def _golden_mask():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    return np.array([[float(t) for t in r] for r in rows])


def test_causal_mask_equals_printed_5x5():
    g = _golden_mask()
    assert g.shape == (5, 5)
    assert np.array_equal(A.causal_mask(5, 0), g)


def test_causal_mask_with_prefix_is_bottom_right_aligned():
    m = A.causal_mask(5, 3)
    assert m.shape == (5, 8)
    assert np.all(m[:, :3] == 0)                 # the whole cached prefix is visible
    assert np.array_equal(m[:, 3:], _golden_mask())
    lib = causal_lower_right(5, 8)._materialize().numpy()
    assert np.array_equal(m == 0, lib)


def _brute_attend(q, k, v, scale, visible):
    """Pure-Python softmax attention, one query row."""
    s = [sum(q[d] * k[j][d] for d in range(len(q))) * scale if visible(j) else None
         for j in range(len(k))]
    m = max(x for x in s if x is not None)
    w = [math.exp(x - m) if x is not None else 0.0 for x in s]
    tot = sum(w)
    return [sum(w[j] * v[j][d] for j in range(len(k))) / tot for d in range(len(v[0]))]


def test_decode_dense_brute_force():
    rng = np.random.default_rng(10)
    hq, hkv, d, L = 4, 2, 8, 7
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    scale = 1 / math.sqrt(d)
    got = A.decode_dense(q, k, v, scale)
    for h in range(hq):
        g = h // (hq // hkv)
        want = _brute_attend(q[h], k[:, g].tolist(), v[:, g].tolist(), scale, lambda j: True)
        np.testing.assert_allclose(got[h], want, rtol=0, atol=1e-13)


def test_prefill_dense_brute_force_with_prefix():
    rng = np.random.default_rng(11)
    e, p, hq, hkv, d = 5, 3, 2, 1, 4
    q = rng.standard_normal((e, hq, d))
    k = rng.standard_normal((p + e, hkv, d))
    v = rng.standard_normal((p + e, hkv, d))
    scale = 1 / math.sqrt(d)
    got = A.prefill_dense(q, k, v, scale)
    for i in range(e):
        for h in range(hq):
            want = _brute_attend(q[i, h], k[:, 0].tolist(), v[:, 0].tolist(), scale,
                                 lambda j: j <= p + i)
            np.testing.assert_allclose(got[i, h], want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("hq,hkv,e,p", [(16, 4, 37, 0), (8, 2, 20, 48), (6, 1, 9, 16)])
def test_prefill_matches_torch_sdpa(hq, hkv, e, p):
    rng = np.random.default_rng(12)
    d = 64
    q = rng.standard_normal((e, hq, d))
    k = rng.standard_normal((p + e, hkv, d))
    v = rng.standard_normal((p + e, hkv, d))
    got = A.prefill_dense(q, k, v, 1 / math.sqrt(d))
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    mask = causal_lower_right(e, p + e) if p else None
    want = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, is_causal=(p == 0),
                                          enable_gqa=True)
    np.testing.assert_allclose(got, want[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_decode_matches_torch_sdpa_gqa():
    rng = np.random.default_rng(13)
    hq, hkv, d, L = 16, 4, 128, 300
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    got = A.decode_dense(q, k, v, 1 / math.sqrt(d))
    want = F.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None], torch.from_numpy(k).permute(1, 0, 2)[None],
        torch.from_numpy(v).permute(1, 0, 2)[None], enable_gqa=True)
    np.testing.assert_allclose(got, want[0, :, 0].numpy(), rtol=0, atol=1e-12)


def test_special_cases():
    rng = np.random.default_rng(14)
    d = 16
    q = rng.standard_normal((4, d))
    v0 = rng.standard_normal((1, 2, d))
    k0 = rng.standard_normal((1, 2, d))
    out = A.decode_dense(q, k0, v0, 0.25)
    assert np.array_equal(out, v0[0][[0, 0, 1, 1]])          # one key: o = v_0 exactly
    kk = np.repeat(rng.standard_normal((1, 2, d)), 9, axis=0)  # identical keys: mean of V
    vv = rng.standard_normal((9, 2, d))
    np.testing.assert_allclose(A.decode_dense(q, kk, vv, 0.25), vv.mean(axis=0)[[0, 0, 1, 1]],
                               atol=1e-13)
    ones = np.ones((9, 2, d))                                  # weights sum to one
    np.testing.assert_allclose(A.decode_dense(q, rng.standard_normal((9, 2, d)), ones, 0.25),
                               1.0, atol=1e-14)
    # row 0 of a prefill with no prefix sees only key 0
    qp = rng.standard_normal((3, 2, d))
    kp, vp = rng.standard_normal((3, 1, d)), rng.standard_normal((3, 1, d))
    assert np.array_equal(A.prefill_dense(qp, kp, vp, 0.25)[0], vp[0][[0, 0]])


@pytest.mark.parametrize("L", [1, 5, 256, 700])
def test_split_merge_invariant_to_chunk(L):
    rng = np.random.default_rng(15 + L)
    hq, hkv, d = 8, 2, 32
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    scale = 1 / math.sqrt(d)
    ref = A.decode_dense(q, k, v, scale)
    for c in sorted({1, 3, 16, 256, L}):
        o, lse = A.decode_split(q, k, v, scale, c)
        assert o.shape == (hq, -(-L // c), d)
        np.testing.assert_allclose(A.merge_splits(o, lse), ref, rtol=0, atol=1e-12)
    # one split's lse is the log-sum-exp of its scores
    o, lse = A.decode_split(q, k, v, scale, L)
    s = np.einsum("ld,d->l", k[:, 0], q[0]) * scale
    np.testing.assert_allclose(lse[0, 0], logsumexp(s), rtol=1e-14)


def test_merge_skips_empty_splits():
    rng = np.random.default_rng(16)
    o = rng.standard_normal((3, 4))
    lse = np.array([0.3, -np.inf, 1.1])
    got = A.merge_splits(o, lse)
    w = np.exp([0.3, 1.1])
    np.testing.assert_allclose(got, (w[0] * o[0] + w[1] * o[2]) / w.sum(), atol=1e-15)


def test_paged_forms_gather_through_the_table():
    rng = np.random.default_rng(17)
    n_layers, slots, hkv, hq, d = 3, 64, 2, 4, 16
    kp = rng.standard_normal((n_layers, slots, hkv, d))
    vp = rng.standard_normal((n_layers, slots, hkv, d))
    perm = rng.permutation(slots)
    table = np.full((2, 32), -1)
    table[0, :20] = perm[:20]
    table[1, :30] = perm[20:50]
    lens = [20, 30]
    # decode with the requests in swapped batch order
    q = rng.standard_normal((2, hq, d))
    got = A.paged_decode(q, kp, vp, 2, table, [1, 0], [0, lens[1], lens[1] + lens[0]], 0.25)
    for b, r in enumerate([1, 0]):
        sl = table[r, :lens[r]]
        np.testing.assert_allclose(got[b], A.decode_dense(q[b], kp[2, sl], vp[2, sl], 0.25),
                                   atol=1e-14)
    # prefill of the last 7 / 4 tokens
    qo = [0, 7, 11]
    qq = rng.standard_normal((11, hq, d))
    got = A.paged_prefill(qq, kp, vp, 1, table, [0, 1], qo, [0, 20, 50], 0.25)
    np.testing.assert_allclose(got[:7], A.prefill_dense(qq[:7], kp[1, perm[:20]],
                                                        vp[1, perm[:20]], 0.25), atol=1e-14)


def test_last_prefill_row_equals_decode_and_prefix_reuse():
    rng = np.random.default_rng(18)
    p, e, hq, hkv, d = 24, 10, 4, 2, 32
    q = rng.standard_normal((p + e, hq, d))
    k = rng.standard_normal((p + e, hkv, d))
    v = rng.standard_normal((p + e, hkv, d))
    full = A.prefill_dense(q, k, v, 0.2)
    part = A.prefill_dense(q[p:], k, v, 0.2)
    np.testing.assert_allclose(part, full[p:], atol=1e-13)
    np.testing.assert_allclose(full[-1], A.decode_dense(q[-1], k, v, 0.2), atol=1e-13)


def _brute_attend_or_zero(q, k, v, scale, visible):
    """_brute_attend, but a row with no visible key is all zeros."""
    if not any(visible(j) for j in range(len(k))):
        return [0.0] * len(v[0])
    return _brute_attend(q, k, v, scale, visible)


def test_absent_keys_take_no_part_brute_force():
    # table entries outside the pool (-1, pool size, beyond) name no key
    rng = np.random.default_rng(19)
    n_layers, slots, hkv, hq, d = 2, 40, 2, 4, 8
    kp = rng.standard_normal((n_layers, slots, hkv, d))
    vp = rng.standard_normal((n_layers, slots, hkv, d))
    table = np.full((2, 16), -1)
    table[0, :9] = rng.permutation(slots)[:9]
    table[0, [1, 4]] = [-1, slots]                  # positions 1 and 4: no key
    table[1, :3] = [slots + 3, -7, slots]           # request 1: no key at all
    scale = 1 / math.sqrt(d)
    ok0 = [j not in (1, 4) for j in range(9)]
    # decode, both requests
    q = rng.standard_normal((2, hq, d))
    got = A.paged_decode(q, kp, vp, 1, table, [0, 1], [0, 9, 12], scale)
    for h in range(hq):
        g = h // (hq // hkv)
        k0 = [kp[1, table[0, j], g].tolist() if ok0[j] else None for j in range(9)]
        v0 = [vp[1, table[0, j], g].tolist() if ok0[j] else [0.0] * d for j in range(9)]
        want = _brute_attend(q[0, h], [x or [0.0] * d for x in k0], v0, scale, lambda j: ok0[j])
        np.testing.assert_allclose(got[0, h], want, rtol=0, atol=1e-13)
    assert np.array_equal(got[1], np.zeros((hq, d)))
    # prefill of the last 5 tokens of request 0: causal and present
    qq = rng.standard_normal((5, hq, d))
    got = A.paged_prefill(qq, kp, vp, 0, table, [0], [0, 5], [0, 9], scale)
    for i in range(5):
        for h in range(hq):
            g = h // (hq // hkv)
            kk = [kp[0, table[0, j], g].tolist() if ok0[j] else [0.0] * d for j in range(9)]
            vv = [vp[0, table[0, j], g].tolist() if ok0[j] else [0.0] * d for j in range(9)]
            want = _brute_attend_or_zero(qq[i, h], kk, vv, scale, lambda j: ok0[j] and j <= 4 + i)
            np.testing.assert_allclose(got[i, h], want, rtol=0, atol=1e-13)


def test_key_mask_default_and_all_absent():
    rng = np.random.default_rng(20)
    q = rng.standard_normal((3, 4, 8))
    k = rng.standard_normal((7, 2, 8))
    v = rng.standard_normal((7, 2, 8))
    np.testing.assert_array_equal(A.prefill_dense(q, k, v, 0.3),
                                  A.prefill_dense(q, k, v, 0.3, np.ones(7, bool)))
    got = A.prefill_dense(q, k, v, 0.3, np.zeros(7, bool))
    assert np.array_equal(got, np.zeros_like(got))
    # the first query sees keys 0..4; with those absent it gets zeros, the others do not
    ok = np.array([False] * 5 + [True] * 2)
    got = A.prefill_dense(q, k, v, 0.3, ok)
    assert np.array_equal(got[0], np.zeros((4, 8)))
    assert np.all(np.abs(got[1:]).sum(axis=-1) > 0)
