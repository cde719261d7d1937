"""Oracle-side expected values for the GPU parity tests.

Built only from ``workloads`` (the shared seeded inputs) and ``oracle``: each
request's keys and values are assembled in position order (history or cached
prefix first, then the new tokens rotated and rounded by the oracle), and the
oracle's dense definitions give the expected outputs.  Tolerances are the
ones fixed for this path: float32 max-abs 1e-5; bf16 max-abs 2e-2 and
relative L2 1e-2; rotated keys within 1 bf16 ulp.
"""

import math

import numpy as np

from oracle import attention as A
from oracle import bf16, rope


def round_store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Value as stored in the pool: bf16 nearest-even, or float32 kept exact."""
    return bf16.round_bf16(x) if dtype == "bf16" else np.asarray(x, dtype=np.float64)


def new_positions(cs) -> np.ndarray:
    return np.concatenate([np.arange(int(s) - int(n), int(s)) for s, n in zip(cs.seq_lens, cs.new_lens)])


def new_offsets(cs) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(cs.new_lens)]).astype(np.int64)


def table(cs) -> np.ndarray:
    """The float32 cos/sin table the method stores, built by the oracle."""
    return rope.freqs_cis_f32(cs.max_ctx_len, cs.head_dim, cs.theta)


def rotated_exact(cs, tab=None):
    """(q, k) of the new tokens rotated by the stored table, before rounding."""
    tab = table(cs) if tab is None else tab
    pos = new_positions(cs)[:, None]
    return (rope.rotate_with_table(cs.q.astype(np.float64), pos, tab),
            rope.rotate_with_table(cs.k.astype(np.float64), pos, tab))


def rotated_new(cs):
    """(q, k) of the new tokens rotated at their positions, rounded as stored."""
    q, k = rotated_exact(cs)
    return round_store(q, cs.dtype), round_store(k, cs.dtype)


def request_kv(cs, b: int, k_rot: np.ndarray):
    """Keys/values of request b in position order, float64 [L_b, Hkv, D]."""
    off = new_offsets(cs)
    kn, vn = k_rot[off[b]:off[b + 1]], cs.v[off[b]:off[b + 1]].astype(np.float64)
    if cs.kind == "decode":
        kh, vh = cs.history(b)
    else:
        p = int(cs.prefix_lens[b])
        if p:
            kh, vh = cs.group_history(int(cs.group_of[b]))
            kh, vh = kh[:p], vh[:p]
        else:
            kh = vh = np.zeros((0,) + cs.k.shape[1:], dtype=np.float32)
    return (np.concatenate([kh.astype(np.float64), kn]), np.concatenate([vh.astype(np.float64), vn]))


def expected_decode(cs, sample=None, rot=None, key_ok=None, workers: int = 1):
    """{b: [Hq, D]} for the newest token of each sampled request (key_ok:
    {b: bool [L_b]} marks the keys that take part, default all).  With
    workers > 1 the requests are spread over that many threads (the oracle's
    NumPy work releases the interpreter lock; BLAS runs one thread each)."""
    q_rot, k_rot = rot if rot is not None else rotated_new(cs)
    off = new_offsets(cs)
    scale = 1.0 / math.sqrt(cs.head_dim)
    todo = list(range(cs.batch) if sample is None else sample)

    def one(b):
        K, V = request_kv(cs, b, k_rot)
        ok = None if key_ok is None else key_ok.get(b)
        return b, A.decode_dense(q_rot[off[b + 1] - 1], K, V, scale, ok)

    if workers <= 1:
        return dict(one(b) for b in todo)
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    # longest first, so that no long request starts last
    todo.sort(key=lambda b: -int(cs.seq_lens[b]))
    with threadpool_limits(1), ThreadPoolExecutor(max_workers=workers) as ex:
        return dict(ex.map(one, todo))


def expected_prefill(cs, sample=None, rot=None, key_ok=None):
    """{b: [e_b, Hq, D]} for the new rows of each sampled request (key_ok as
    for expected_decode)."""
    q_rot, k_rot = rot if rot is not None else rotated_new(cs)
    off = new_offsets(cs)
    scale = 1.0 / math.sqrt(cs.head_dim)
    out = {}
    for b in (range(cs.batch) if sample is None else sample):
        K, V = request_kv(cs, b, k_rot)
        ok = None if key_ok is None else key_ok.get(b)
        out[b] = A.prefill_dense(q_rot[off[b]:off[b + 1]], K, V, scale, ok)
    return out


def assert_close(got, want, dtype: str, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    mx = float(err.max()) if err.size else 0.0
    if dtype == "f32":
        assert mx <= 1e-5, f"{what}: max-abs {mx:.3e} > 1e-5"
        return mx, 0.0
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    assert mx <= 2e-2 and rel <= 1e-2, f"{what}: max-abs {mx:.3e}, rel-L2 {rel:.3e}"
    return mx, rel


def assert_within_ulp(got, exact, what: str = ""):
    """|got - exact| <= one bf16 ulp of the rounded exact value."""
    got = np.asarray(got, dtype=np.float64)
    exact = np.asarray(exact, dtype=np.float64)
    tol = bf16.ulp_bf16(bf16.round_bf16(exact))
    bad = np.abs(got - exact) > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} values beyond 1 bf16 ulp"
