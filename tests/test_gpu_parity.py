"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Every case is drawn by ``workloads`` with a fixed seed; the GPU side is staged
by ``staging`` (library page tables, torch-allocated pool pre-filled with a
NaN canary), the expected side by ``expect`` (oracle only).  Bars: page
tables bit-exact (covered on the CPU in test_native_host), rotated K within
1 bf16 ulp, V copied bit-exactly, outputs within max-abs 1e-5 (float32) or
max-abs 2e-2 and rel-L2 1e-2 (bf16).
"""

import math

import numpy as np
import pytest
import torch

import expect as E
import paged_gqa_attention_rope_amd as astr
import staging
from oracle import attention as A
from oracle import rope
from workloads import make_case
from workloads.gen import bf16_storage, decode_case, prefill_case

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.fixture(autouse=True)
def _cleanup():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# cases
# ---------------------------------------------------------------------------

def _dec(seed, **kw):
    base = dict(batch=6, n_heads=16, n_kv_heads=4, head_dim=128, dtype="bf16", mode=1,
                page_size=16, split_chunk=256, len_lo=1, len_hi=1500, shuffle_pages=True)
    base.update(kw)
    return decode_case(seed, **base)


def _pre(seed, **kw):
    base = dict(batch=5, n_heads=16, n_kv_heads=4, head_dim=128, dtype="bf16", mode=0,
                page_size=1, q_tile=64, ext_lo=1, ext_hi=200)
    base.update(kw)
    return prefill_case(seed, **base)


DECODE = {
    "decode-contig-f32-b2": lambda: make_case(1),
    "decode-page1-b8": lambda: make_case(2),
    "decode-page1-b8-seed101": lambda: make_case(2, 101),
    "page16-3layers-chunk512": lambda: _dec(11, batch=12, split_chunk=512, len_hi=3000,
                                            log_uniform=True, n_layers=3, random_layer=True),
    "single-split-direct": lambda: _dec(12, batch=5, split_chunk=256, len_hi=256, page_size=1,
                                        pool_slots=4096),
    "length-one-and-two": lambda: _dec(13, lens=[1, 1, 2, 3, 300, 257], split_chunk=128),
    "g1-d64-contig": lambda: _dec(14, batch=4, n_heads=8, n_kv_heads=8, head_dim=64, mode=0,
                                  split_chunk=128, len_lo=100, len_hi=700, shuffle_pages=False),
    "g6-d64": lambda: _dec(15, n_heads=24, n_kv_heads=4, head_dim=64, split_chunk=300),
    "g8-d128": lambda: _dec(16, n_heads=16, n_kv_heads=2, split_chunk=200),
    "g2-d128-f32": lambda: _dec(17, n_heads=8, n_kv_heads=4, dtype="f32", split_chunk=100),
    "g4-d64-f32-page1": lambda: _dec(18, head_dim=64, dtype="f32", page_size=1, pool_slots=20000),
}

def _pre_random(s):
    """Random batch under the library's work plan: extends of 1-700 rows behind
    shared page-aligned prefixes of up to 1600 tokens; even seeds draw 1-4
    requests (long tiles dominate and the plan splits them), odd ones 5-24."""
    rng = np.random.default_rng(900 + s)
    batch = int(rng.integers(1, 5) if s % 2 == 0 else rng.integers(5, 25))
    return _pre(500 + s, batch=batch, mode=1, page_size=16, pool_slots=1 << 16, n_groups=3,
                prefix_pages_hi=100, ext_lo=1, ext_hi=700, shuffle_pages=True)


PREFILL = {
    **{f"plan-random-{s}": (lambda s=s: _pre_random(s)) for s in range(6)},
    "prefill-contig-b4": lambda: make_case(3),
    "prefill-radix-b16": lambda: make_case(4),
    "prefill-radix-b16-seed101": lambda: make_case(4, 101),
    "tiny-extends": lambda: _pre(21, batch=7, ext_lo=1, ext_hi=3),
    "ragged-65-129": lambda: _pre(22, batch=3, ext_lo=63, ext_hi=130),
    "prefix-page16-g1-d64": lambda: _pre(23, n_heads=4, n_kv_heads=4, head_dim=64, mode=1,
                                         page_size=16, pool_slots=16384, n_groups=2,
                                         prefix_pages_hi=20, ext_lo=1, ext_hi=150,
                                         max_ctx_len=480),
    "prefix-g6-d64": lambda: _pre(24, n_heads=24, n_kv_heads=4, head_dim=64, mode=1,
                                  page_size=16, pool_slots=16384, n_groups=3, prefix_pages_hi=30,
                                  ext_lo=10, ext_hi=140, max_ctx_len=640),
    "prefix-g8-d128": lambda: _pre(25, n_heads=16, n_kv_heads=2, mode=1, page_size=16,
                                   pool_slots=16384, n_groups=2, prefix_pages_hi=12, ext_hi=100,
                                   max_ctx_len=300),
    "g2-f32-d128": lambda: _pre(26, n_heads=8, n_kv_heads=4, dtype="f32", ext_hi=150),
    # 64 KV heads x 128: a slot is wider than a buffer record stride can express
    "wide-slot-g1-kv64-d128": lambda: _pre(28, batch=3, n_heads=64, n_kv_heads=64, mode=1,
                                           page_size=16, pool_slots=4096, n_groups=2,
                                           prefix_pages_hi=6, ext_lo=20, ext_hi=90, max_ctx_len=200),
    # 4 query heads per KV head with slots wider than a record stride
    "wide-slot-g4-kv64-d128": lambda: _pre(29, batch=2, n_heads=256, n_kv_heads=64, mode=1,
                                           page_size=16, pool_slots=2048, n_groups=2,
                                           prefix_pages_hi=4, ext_lo=30, ext_hi=70, max_ctx_len=160),
    "prefix-f32-d64": lambda: _pre(27, head_dim=64, dtype="f32", mode=1, page_size=16,
                                   pool_slots=8192, n_groups=2, prefix_pages_hi=10, ext_hi=90,
                                   max_ctx_len=260),
}


# ---------------------------------------------------------------------------
# rotary table and fused write
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
def test_rope_table_matches_oracle(d):
    say(f"rope_table d={d} max_pos=32768")
    t = astr.rope_table(32768, d, 10000.0, "cuda")
    torch.cuda.synchronize()
    got = t.cpu().numpy().astype(np.float64)
    want = rope.freqs_cis(32768, d)
    ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - want) <= ulp)


@pytest.mark.parametrize("name", ["decode-contig-f32-b2", "prefill-contig-b4", "decode-page1-b8", "g6-d64", "prefix-f32-d64", "prefill-radix-b16"])
def test_rope_kv_write(name):
    cs = (DECODE.get(name) or PREFILL.get(name))()
    say(f"rope_kv_write case={name} seed={cs.seed} tokens={cs.n_new}")
    st = staging.stage(cs)
    staging.run_write(st)
    torch.cuda.synchronize()
    exact_q, exact_k = E.rotated_exact(cs)
    loc = torch.from_numpy(st.write_meta["out_cache_loc"].astype(np.int64)).cuda()
    L = cs.layer_id
    gk = to_np(st.k_buffer[L].index_select(0, loc))
    gv = to_np(st.v_buffer[L].index_select(0, loc))
    gq = to_np(st.q)
    if cs.dtype == "bf16":
        E.assert_within_ulp(gk, exact_k, "rotated k")
        E.assert_within_ulp(gq, exact_q, "rotated q")
    else:
        assert np.abs(gk - exact_k).max() <= 1e-5
        assert np.abs(gq - exact_q).max() <= 1e-5
    assert np.array_equal(gv, cs.v.astype(np.float64)), "v must be copied bit-exactly"
    # canary: only history and written slots of the attended layer hold numbers
    touched = np.zeros(cs.pool_slots, dtype=bool)
    touched[st.write_meta["out_cache_loc"]] = True
    table = st.pool.table()
    for b, r in enumerate(st.reqs):
        hist = int(cs.seq_lens[b] - cs.new_lens[b])
        touched[table[r, :hist]] = True
    for buf in (st.k_buffer, st.v_buffer):
        finite = (~torch.isnan(buf.float()).all(dim=3).all(dim=2)).cpu().numpy()
        assert np.array_equal(finite[L], touched), "a slot outside out_cache_loc changed"
        assert not np.delete(finite, L, axis=0).any(), "another layer changed"


def test_rope_kv_write_skips_out_of_range_tokens():
    cs = _pre(31, batch=2, ext_lo=5, ext_hi=5)
    say("rope_kv_write out-of-range slots and positions are skipped")
    st = staging.stage(cs)
    loc = st.write_cache.out_cache_loc.clone()
    loc[0] = -1
    loc[1] = cs.pool_slots                      # one past the end
    pos = st.positions.clone()
    pos[2] = st.freqs.shape[0]                  # position outside the table
    q0 = st.q.clone()
    astr.rope_kv_write(st.q, st.k, st.v, pos, loc, st.freqs, st.write_cache, 0)
    torch.cuda.synchronize()
    finite = (~torch.isnan(st.k_buffer[0].float()).all(dim=2).all(dim=1)).cpu().numpy()
    good = st.write_meta["out_cache_loc"][3:]
    assert finite.sum() == len(good) and finite[good].all()
    assert torch.equal(st.q[:3], q0[:3]), "skipped tokens keep their q"


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_rope_backward_matches_oracle(dtype, d):
    # gradient rows of 24 heads at positions spread over a 32k table, plus
    # out-of-range positions that must leave their rows unchanged
    say(f"rope_backward dtype={dtype} d={d}")
    n, h, max_pos = 3000, 24, 32768
    rng = np.random.default_rng(40 + d)
    g = rng.standard_normal((n, h, d)).astype(np.float32)
    if dtype == "bf16":
        g = bf16_storage(g)
    pos = rng.integers(0, max_pos, size=n).astype(np.int32)
    pos[:3] = [-1, max_pos, 0]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    table = astr.rope_table(max_pos, d, 10000.0, "cuda")
    gt = torch.from_numpy(g).to(tdt).cuda()
    astr.rope_backward(gt, torch.from_numpy(pos).cuda(), table)
    torch.cuda.synchronize()
    got = gt.float().cpu().numpy().astype(np.float64)
    tab = rope.freqs_cis_f32(max_pos, d, 10000.0)         # the oracle's stored float32 table
    ok = (pos >= 0) & (pos < max_pos)
    want = rope.rotate_backward_with_table(g[ok].astype(np.float64), pos[ok][:, None], tab)
    assert np.array_equal(got[~ok], g[~ok].astype(np.float64)), "out-of-range rows must be unchanged"
    if dtype == "bf16":
        E.assert_within_ulp(got[ok], want, "rope gradient")
    else:
        ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got[ok] - want) <= ulp), "rope gradient beyond 1 float32 ulp"


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(DECODE))
def test_decode_parity(name):
    cs = DECODE[name]()
    say(f"decode case={name} seed={cs.seed} B={cs.batch} Hq={cs.n_heads} Hkv={cs.n_kv_heads} "
        f"D={cs.head_dim} {cs.dtype} lens={cs.seq_lens.min()}..{cs.seq_lens.max()} C={cs.split_chunk}")
    st = staging.stage(cs)
    staging.run_write(st)
    out = staging.run_decode(st)
    torch.cuda.synchronize()
    want = E.expected_decode(cs)
    got = to_np(out)
    for b in range(cs.batch):
        E.assert_close(got[b], want[b], cs.dtype, f"{name} request {b} (L={cs.seq_lens[b]})")


@pytest.mark.parametrize("name", ["decode-contig-f32-b2", "decode-page1-b8", "g2-d128-f32", "g8-d128"])
def test_decode_work_items_equal_full_grid(name):
    """The work-item grid (one workgroup per split that holds keys) gives the
    same bits as the full (entry, split) grid, also with the items listed in
    another order."""
    cs = DECODE[name]()
    say(f"decode work items case={name} B={cs.batch} C={cs.split_chunk}")
    st = staging.stage(cs)
    staging.run_write(st)
    q = staging.decode_query(st)
    c = st.attn_cache
    assert c.num_split_items > 0
    full = astr.KVCache(**{**c.__dict__, "split_item_batch": None, "split_item_index": None,
                           "num_split_items": 0, "split_item_chunk": 0})
    perm = torch.randperm(c.num_split_items, generator=torch.Generator().manual_seed(3)).to(q.device)
    shuf = astr.KVCache(**{**c.__dict__, "split_item_batch": c.split_item_batch[perm].contiguous(),
                           "split_item_index": c.split_item_index[perm].contiguous()})
    outs = [astr.decode_attn(q, cc, cs.layer_id, cs.split_chunk) for cc in (c, full, shuf)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    want = E.expected_decode(cs)
    got = to_np(outs[0])
    for b in range(cs.batch):
        E.assert_close(got[b], want[b], cs.dtype, f"{name} request {b}")


FUSED = [n for n in DECODE if n not in ("decode-contig-f32-b2", "g2-d128-f32", "g4-d64-f32-page1")]   # bf16, one new token each


@pytest.mark.parametrize("name", FUSED)
def test_decode_attn_write_equals_write_then_decode(name):
    # the fused call must store the same pool bits and produce the same output
    # bits as the rotary write followed by the plain decode, on two separately
    # staged copies of the workload (NaN canary everywhere else in the pools)
    cs = DECODE[name]()
    say(f"fused decode write case={name} seed={cs.seed} B={cs.batch} C={cs.split_chunk}")
    assert cs.dtype == "bf16" and np.all(cs.new_lens == 1)
    two = staging.stage(cs)
    staging.run_write(two)
    want_out = staging.run_decode(two)
    one = staging.stage(cs)
    got_out = astr.decode_attn_write(one.q, one.k, one.v, one.attn_cache, cs.layer_id, one.freqs,
                                     cs.split_chunk)
    torch.cuda.synchronize()
    assert torch.equal(got_out.view(torch.int16), want_out.view(torch.int16)), "output bits differ"
    for a, b in ((one.k_buffer, two.k_buffer), (one.v_buffer, two.v_buffer)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "pool bits differ"
    want = E.expected_decode(cs)
    got = to_np(got_out)
    for b in range(cs.batch):
        E.assert_close(got[b], want[b], cs.dtype, f"{name} request {b}")


def test_decode_step_graph_replays_equal_eager():
    # a 4-layer step (history in one layer, zeros elsewhere) run eagerly on one
    # staging and captured + replayed three times on another, with unrelated
    # eager work between replays: outputs and pools must match bit for bit;
    # the layer holding the history also matches the oracle
    from paged_gqa_attention_rope_amd.step import DecodeStep
    cs = _dec(51, batch=6, len_hi=1200, n_layers=4, random_layer=True, split_chunk=256)
    say(f"graph-captured 4-layer decode step, history in layer {cs.layer_id}")
    nl, b, hq, hk, d = cs.n_layers, cs.batch, cs.n_heads, cs.n_kv_heads, cs.head_dim
    rng = np.random.default_rng(52)
    inp = [bf16_storage(rng.standard_normal((nl, b, n, d)).astype(np.float32)) for n in (hq, hk, hk)]
    inp[0][cs.layer_id], inp[1][cs.layer_id], inp[2][cs.layer_id] = cs.q, cs.k, cs.v
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in inp)
    eager = staging.stage(cs, canary=False)
    want = DecodeStep(eager.attn_cache, eager.freqs, q, k, v, cs.split_chunk).run().clone()
    graphed = staging.stage(cs, canary=False)
    step = DecodeStep(graphed.attn_cache, graphed.freqs, q, k, v, cs.split_chunk)
    step.capture()
    scratch = torch.zeros(1 << 20, device="cuda")
    for r in range(3):
        step.out.fill_(float("nan"))
        got = step.replay()
        scratch.add_(1.0)                           # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"replay {r} output differs"
        for a_, b_ in ((graphed.k_buffer, eager.k_buffer), (graphed.v_buffer, eager.v_buffer)):
            assert torch.equal(a_.view(torch.int16), b_.view(torch.int16)), f"replay {r} pool differs"
    ref = E.expected_decode(cs)
    got = to_np(want[cs.layer_id])
    for i in range(b):
        E.assert_close(got[i], ref[i], cs.dtype, f"layer {cs.layer_id} request {i}")


def test_decode_split_partials_match_oracle():
    cs = _dec(41, batch=4, len_lo=100, len_hi=900, split_chunk=128)
    say("decode split partials chunk=128")
    st = staging.stage(cs)
    staging.run_write(st)
    o_part, lse = astr.decode_workspace(st.attn_cache, cs.n_heads, cs.split_chunk)
    staging.run_decode(st, o_part=o_part, lse_part=lse)
    torch.cuda.synchronize()
    q_rot, k_rot = E.rotated_new(cs)
    off = E.new_offsets(cs)
    go, gl = to_np(o_part), to_np(lse)
    for b in range(cs.batch):
        K, V = E.request_kv(cs, b, k_rot)
        wo, wl = A.decode_split(q_rot[off[b + 1] - 1], K, V, 1 / math.sqrt(cs.head_dim), cs.split_chunk)
        ns = wo.shape[1]
        E.assert_close(go[b, :, :ns], wo, "bf16", f"o_part request {b}")
        assert np.abs(gl[b, :, :ns] - wl).max() <= 1e-2


def test_decode_zero_length_request_gives_zero():
    cs = _dec(42, lens=[40, 70], split_chunk=32)
    say("decode with a zero-length entry")
    st = staging.stage(cs)
    staging.run_write(st)
    kv = st.attn_cache.kv_indptr.clone()
    kv[1] = kv[0]                                   # entry 0 now has no keys
    kv[2] = kv[1] + 70
    c2 = astr.KVCache(**{**st.attn_cache.__dict__, "kv_indptr": kv})
    out = astr.decode_attn(staging.decode_query(st), c2, cs.layer_id, cs.split_chunk)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[0]) == 0
    want = E.expected_decode(cs, sample=[1])
    E.assert_close(to_np(out[1]), want[1], "bf16", "request 1")


def test_decode_request_row_outside_table_gives_zero():
    """A batch entry whose request row lies outside req_to_token counts as a
    request without keys: the kernels never read that row (its output is
    zero) and the other entry is unaffected."""
    cs = _dec(43, lens=[40, 70], split_chunk=32)
    say("decode with a request row outside the table")
    st = staging.stage(cs)
    staging.run_write(st)
    rpi = st.attn_cache.req_pool_indices.clone()
    rpi[0] = st.attn_cache.req_to_token.shape[0] + 1000
    c2 = astr.KVCache(**{**st.attn_cache.__dict__, "req_pool_indices": rpi})
    out = astr.decode_attn(staging.decode_query(st), c2, cs.layer_id, cs.split_chunk)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[0]) == 0
    want = E.expected_decode(cs, sample=[1])
    E.assert_close(to_np(out[1]), want[1], "bf16", "request 1")


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_parity(name):
    cs = PREFILL[name]()
    say(f"prefill case={name} seed={cs.seed} B={cs.batch} Hq={cs.n_heads} Hkv={cs.n_kv_heads} "
        f"D={cs.head_dim} {cs.dtype} ext={cs.new_lens.min()}..{cs.new_lens.max()} "
        f"prefix<={cs.prefix_lens.max()}")
    st = staging.stage(cs)
    assert st.cached == list(cs.prefix_lens), "radix hit must equal the drawn prefix"
    staging.run_write(st)
    out = staging.run_prefill(st)
    torch.cuda.synchronize()
    want = E.expected_prefill(cs)
    got = to_np(out)
    off = E.new_offsets(cs)
    for b in range(cs.batch):
        E.assert_close(got[off[b]:off[b + 1]], want[b], cs.dtype, f"{name} request {b}")


def _corrupt_table(st, cs, rng, per_request=6):
    """Point some table entries of every request outside the pool; returns
    {b: bool [L_b]} of the keys that still take part."""
    bad_values = [-1, cs.pool_slots, cs.pool_slots + 4097, 2 ** 31 - 1]
    t = st.attn_cache.req_to_token
    key_ok = {}
    for b, r in enumerate(st.reqs):
        L = int(cs.seq_lens[b])
        ok = np.ones(L, dtype=bool)
        if b == 0 and L <= 40:
            ok[:] = False                        # a request with no key left at all
        else:
            pos = rng.choice(L, size=min(per_request, L - 1), replace=False)
            ok[pos] = False
        for j in np.nonzero(~ok)[0]:
            t[r, int(j)] = int(bad_values[int(j) % len(bad_values)])
        key_ok[b] = ok
    return key_ok


@pytest.mark.parametrize("name", ["prefill-radix-b16", "ragged-65-129", "tiny-extends", "prefix-g8-d128",
                                  "prefix-g6-d64", "prefix-page16-g1-d64", "prefix-f32-d64"])
def test_prefill_keys_outside_pool_take_no_part(name):
    cs = PREFILL[name]()
    say(f"prefill with table entries outside the pool, case={name} seed={cs.seed}")
    st = staging.stage(cs)
    staging.run_write(st)
    key_ok = _corrupt_table(st, cs, np.random.default_rng(cs.seed + 7))
    out = staging.run_prefill(st)
    torch.cuda.synchronize()
    want = E.expected_prefill(cs, key_ok=key_ok)
    got = to_np(out)
    off = E.new_offsets(cs)
    for b in range(cs.batch):
        E.assert_close(got[off[b]:off[b + 1]], want[b], cs.dtype, f"{name} request {b}")


def _with_score_jumps(cs, rng):
    """Scale two cached prefix keys of every prefix group by 2^4 and 2^7
    (exact in bf16), at random positions past the first quarter of the
    prefix: rows that reach them see their running maximum jump by tens to
    hundreds in the exponent, past the range of a float exponential."""
    orig = cs._group_hist
    picks = {}
    for grp, toks in enumerate(cs.group_tokens):
        n = len(toks)
        if n >= 8:
            picks[grp] = rng.choice(np.arange(n // 4, n), size=2, replace=False)

    def hist(grp):
        k, v = orig(grp)
        if grp in picks:
            k = k.copy()
            k[picks[grp][0]] *= 16.0
            k[picks[grp][1]] *= 128.0
        return k, v
    cs._group_hist = hist
    return sum(len(p) for p in picks.values())


@pytest.mark.parametrize("name", ["prefill-radix-b16", "prefix-g8-d128", "prefix-g6-d64", "prefix-page16-g1-d64"])
def test_prefill_score_jumps_raise_the_max(name):
    # The lazily raised running max (softmax over the visible keys, AstrAI
    # docs/guides/inference.md, 'Attention Backend') must follow scores that
    # jump far past it midway through a row.  The bf16 kernels take
    # q * scale * log2(e) rounded to bf16 as the product operand; with a
    # 2^7-scaled key that rounding alone moves a score by ~0.2 in the
    # exponent, so this test uses the softmax scale for which that factor is
    # 1/8 (exact); the query operand is the oracle's stored rotation (a
    # 1-ulp rounding difference of the rotation would be scaled by 2^7 as
    # well), so the comparison checks the running max.
    cs = PREFILL[name]()
    n = _with_score_jumps(cs, np.random.default_rng(cs.seed + 11))
    assert n > 0
    scale = float(np.float32(0.125 / math.log2(math.e)))
    say(f"prefill with score jumps, case={name} seed={cs.seed} scaled keys={n} scale={scale:.8f}")
    st = staging.stage(cs)
    staging.run_write(st)
    q_rot, k_rot = E.rotated_new(cs)
    q_in = torch.from_numpy(q_rot.astype(np.float32)).to(st.q.dtype).cuda()
    assert q_in.shape == st.q.shape
    out = astr.prefill_attn(q_in, st.attn_cache, cs.layer_id, sm_scale=scale)
    torch.cuda.synchronize()
    got = to_np(out)
    off = E.new_offsets(cs)
    for b in range(cs.batch):
        K, V = E.request_kv(cs, b, k_rot)
        want = A.prefill_dense(q_rot[off[b]:off[b + 1]], K, V, scale, None)
        assert np.all(np.isfinite(want))
        E.assert_close(got[off[b]:off[b + 1]], want, cs.dtype, f"{name} request {b}")


@pytest.mark.parametrize("name", ["decode-page1-b8", "page16-3layers-chunk512", "g8-d128", "g6-d64"])
def test_decode_score_jumps_across_splits(name):
    # Split-K partials whose log-sum-exps differ by up to ~185 in the
    # exponent must merge to the direct softmax (AstrAI
    # docs/guides/inference.md, 'KVCache System': partial outputs with their
    # max and sum).  Two cached keys per request are scaled by 2^4 and 2^7
    # (exact in bf16).  The query operand is the oracle's stored rotation (a
    # 1-ulp difference of the rotation would be scaled by 2^7); the softmax
    # scale is the prefill test's (this kernel scales its float32 scores, so
    # any scale would do).
    cs = DECODE[name]()
    rng = np.random.default_rng(cs.seed + 11)
    orig = cs._hist
    picks = {}
    for b in range(cs.batch):
        n = int(cs.hist_lens[b])
        if n >= 8:
            picks[b] = rng.choice(np.arange(n // 4, n), size=2, replace=False)

    def hist(b):
        k, v = orig(b)
        if b in picks:
            k = k.copy()
            k[picks[b][0]] *= 16.0
            k[picks[b][1]] *= 128.0
        return k, v
    cs._hist = hist
    assert picks
    scale = float(np.float32(0.125 / math.log2(math.e)))
    say(f"decode with score jumps, case={name} seed={cs.seed} requests with scaled keys={len(picks)}")
    st = staging.stage(cs)
    staging.run_write(st)
    q_rot, k_rot = E.rotated_new(cs)
    off = E.new_offsets(cs)
    last = [int(off[b + 1]) - 1 for b in range(cs.batch)]
    q_in = torch.from_numpy(q_rot[last].astype(np.float32)).to(st.q.dtype).cuda()
    out = astr.decode_attn(q_in, st.attn_cache, cs.layer_id, cs.split_chunk, sm_scale=scale)
    torch.cuda.synchronize()
    got = to_np(out)
    for b in range(cs.batch):
        K, V = E.request_kv(cs, b, k_rot)
        want = A.decode_dense(q_rot[last[b]], K, V, scale, None)
        assert np.all(np.isfinite(want))
        E.assert_close(got[b], want, cs.dtype, f"{name} request {b} (L={cs.seq_lens[b]})")


@pytest.mark.parametrize("name", ["decode-page1-b8", "g8-d128", "g6-d64", "g2-d128-f32", "length-one-and-two"])
def test_decode_keys_outside_pool_take_no_part(name):
    cs = DECODE[name]()
    say(f"decode with table entries outside the pool, case={name} seed={cs.seed}")
    st = staging.stage(cs)
    staging.run_write(st)
    key_ok = _corrupt_table(st, cs, np.random.default_rng(cs.seed + 7))
    out = staging.run_decode(st)
    torch.cuda.synchronize()
    want = E.expected_decode(cs, key_ok=key_ok)
    got = to_np(out)
    for b in range(cs.batch):
        E.assert_close(got[b], want[b], cs.dtype, f"{name} request {b}")


@pytest.mark.parametrize("name", ["prefill-radix-b16", "prefix-g6-d64", "prefix-f32-d64"])
def test_last_prefill_row_equals_decode(name):
    cs = PREFILL[name]()
    say(f"prefill last row vs decode, case={name}")
    st = staging.stage(cs)
    staging.run_write(st)
    pre = staging.run_prefill(st)
    dmeta = st.pool.bind(st.reqs, np.ones(cs.batch, dtype=np.int32), 64)
    dcache = astr.cache_from_bind(st.k_buffer, st.v_buffer, st.pool.table(), dmeta)
    last = torch.from_numpy((E.new_offsets(cs)[1:] - 1).astype(np.int64)).cuda()
    q_last = st.q.index_select(0, last).contiguous()
    dec = astr.decode_attn(q_last, dcache, cs.layer_id, 128)
    torch.cuda.synchronize()
    E.assert_close(to_np(dec), to_np(pre.index_select(0, last)), cs.dtype, "decode vs prefill")


# ---------------------------------------------------------------------------
# every supported (dtype, head_dim, query heads per KV head), small shapes
# ---------------------------------------------------------------------------

SHAPES = [(dt, d, g) for dt in ("bf16", "f32") for d in (64, 128) for g in (1, 2, 4, 6, 8)]


@pytest.mark.parametrize("dtype,d,g", SHAPES, ids=[f"{dt}-d{d}-g{g}" for dt, d, g in SHAPES])
def test_decode_every_supported_shape(dtype, d, g):
    # 2 KV heads, lengths 1..700 over page-16 shuffled pages, chunk 128
    # (several splits and a ragged last split per request)
    cs = _dec(300 + 10 * g + d // 64, batch=4, n_heads=2 * g, n_kv_heads=2, head_dim=d, dtype=dtype,
              split_chunk=128, len_lo=1, len_hi=700)
    say(f"decode shape sweep {dtype} d={d} G={g} lens={cs.seq_lens.tolist()}")
    st = staging.stage(cs)
    staging.run_write(st)
    out = staging.run_decode(st)
    torch.cuda.synchronize()
    want = E.expected_decode(cs)
    got = to_np(out)
    for b in range(cs.batch):
        E.assert_close(got[b], want[b], dtype, f"{dtype} d{d} G{g} request {b} (L={cs.seq_lens[b]})")


@pytest.mark.parametrize("dtype,d,g", SHAPES, ids=[f"{dt}-d{d}-g{g}" for dt, d, g in SHAPES])
def test_prefill_every_supported_shape(dtype, d, g):
    # 2 KV heads, 3 requests behind radix prefixes of up to 160 positions,
    # extends 1..150 (a full tile and a ragged one, or a single partial tile)
    cs = _pre(400 + 10 * g + d // 64, batch=3, n_heads=2 * g, n_kv_heads=2, head_dim=d, dtype=dtype,
              mode=1, page_size=16, pool_slots=8192, n_groups=2, prefix_pages_hi=10, ext_lo=1,
              ext_hi=150, max_ctx_len=320)
    say(f"prefill shape sweep {dtype} d={d} G={g} ext={cs.new_lens.tolist()} pre={cs.prefix_lens.tolist()}")
    st = staging.stage(cs)
    staging.run_write(st)
    out = staging.run_prefill(st)
    torch.cuda.synchronize()
    want = E.expected_prefill(cs)
    got = to_np(out)
    off = E.new_offsets(cs)
    for b in range(cs.batch):
        E.assert_close(got[off[b]:off[b + 1]], want[b], dtype, f"{dtype} d{d} G{g} request {b}")


# ---------------------------------------------------------------------------
# the large decode workload at full size, every request
# ---------------------------------------------------------------------------

def test_decode_full_size_all_requests():
    """The 256-request, 24-layer decode workload exactly as bench.py runs it
    (work-item grid, split 512): every request's output against the oracle,
    and every other layer of both pools still holds the NaN canary."""
    cs = make_case(5)
    free, total = torch.cuda.mem_get_info()
    say(f"decode full size: B={cs.batch} pool_slots={cs.pool_slots} layers={cs.n_layers} "
        f"layer_id={cs.layer_id} free={free / 2**30:.0f} GiB")
    st = staging.stage(cs, canary=True)
    staging.run_write(st)
    out = staging.run_decode(st)
    torch.cuda.synchronize()
    got = to_np(out)
    say("decode full size: oracle over all requests")
    want = E.expected_decode(cs, workers=16)
    worst = (0.0, 0.0)
    for b in range(cs.batch):
        mx, rel = E.assert_close(got[b], want[b], "bf16", f"request {b} (L={cs.seq_lens[b]})")
        worst = (max(worst[0], mx), max(worst[1], rel))
    say(f"decode full size: worst max-abs {worst[0]:.2e}, worst rel-L2 {worst[1]:.2e}")
    nan_bits = torch.tensor(float("nan"), dtype=torch.bfloat16).view(torch.int16).item()
    chunk = 1 << 28
    for buf in (st.k_buffer, st.v_buffer):
        for layer in range(cs.n_layers):
            if layer == cs.layer_id:
                continue
            flat = buf[layer].view(-1).view(torch.int16)
            for lo in range(0, flat.numel(), chunk):
                assert bool((flat[lo:lo + chunk] == nan_bits).all()), f"layer {layer} changed"


# ---------------------------------------------------------------------------
# prefill work plans: split tiles merged by the half that finishes second
# ---------------------------------------------------------------------------

def _tile_steps(meta):
    qo, kv, qt = meta["qo_indptr"], meta["kv_indptr"], meta["q_tile"]
    out = []
    for b, i in zip(meta["q_tile_to_batch"], meta["q_tile_to_index"]):
        e = int(qo[b + 1] - qo[b])
        p = int(kv[b + 1] - kv[b]) - e
        out.append(-(-(p + int(i) * qt + min(qt, e - int(i) * qt)) // 32))
    return out


def _forced_plan(meta, cut, upper_first):
    """Every tile split at key step cut(n); halves listed upper first where
    upper_first(t) holds."""
    qo, kv, rpi = meta["qo_indptr"], meta["kv_indptr"], meta["req_pool_indices"]
    rows = []
    for t, n in enumerate(_tile_steps(meta)):
        b, i = int(meta["q_tile_to_batch"][t]), int(meta["q_tile_to_index"][t])
        e = int(qo[b + 1] - qo[b])
        p = int(kv[b + 1] - kv[b]) - e
        desc = [int(rpi[b]), int(qo[b]) + 64 * i, min(64, e - 64 * i), p + 64 * i]
        lo, hi = [t, 0, cut(n), 2 * t] + desc, [t, cut(n), 2 ** 31 - 1, 2 * t + 1] + desc
        rows += [hi, lo] if upper_first(t) else [lo, hi]
    return np.array(rows, np.int32), meta["num_q_tiles"]


def _with_plan(cache, units, pairs, n_heads, workspace=None):
    import dataclasses
    need = astr.prefill_workspace_bytes(pairs, n_heads, int(cache.k_buffer.shape[3]))
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=cache.k_buffer.device)
    return dataclasses.replace(cache, prefill_units=torch.from_numpy(units).cuda(), num_prefill_pairs=pairs,
                               prefill_workspace=workspace), workspace


@pytest.mark.parametrize("name", ["prefill-radix-b16", "ragged-65-129", "tiny-extends", "prefix-g8-d128",
                                  "wide-slot-g4-kv64-d128"])
def test_prefill_forced_split_matches_oracle(name):
    cs = PREFILL[name]()
    st = staging.stage(cs, plan=False)
    staging.run_write(st)
    want = E.expected_prefill(cs)
    off = E.new_offsets(cs)
    meta = st.attn_meta
    variants = [
        ("half, lower first", lambda n: n // 2, lambda t: False),
        ("half, upper first", lambda n: n // 2, lambda t: True),
        ("one step, alternating", lambda n: min(1, n), lambda t: t % 2 == 1),
        ("empty lower half", lambda n: 0, lambda t: t % 3 == 0),
        ("empty upper half", lambda n: n + 3, lambda t: t % 2 == 0),
    ]
    ws = None
    for label, cut, upper in variants:
        units, pairs = _forced_plan(meta, cut, upper)
        cache, ws = _with_plan(st.attn_cache, units, pairs, cs.n_heads, ws)
        for rep in range(2):                    # the counts are left at zero for the next call
            say(f"prefill forced split case={name} {label} call {rep}")
            out = astr.prefill_attn(st.q, cache, cs.layer_id)
            torch.cuda.synchronize()
            got = to_np(out)
            for b in range(cs.batch):
                E.assert_close(got[off[b]:off[b + 1]], want[b], cs.dtype, f"{name} {label} request {b}")
        slots = pairs * cs.n_heads // 4
        counts = ws[:4 * slots].view(torch.int32)
        assert int(counts.abs().sum()) == 0, "completion counts must be zero after a call"


@pytest.mark.parametrize("name", ["prefill-radix-b16", "prefill-radix-b16-seed101", "prefill-contig-b4", "prefix-g8-d128"])
def test_prefill_plan_matches_unplanned(name):
    cs = PREFILL[name]()
    st = staging.stage(cs)
    staging.run_write(st)
    c = st.attn_cache
    say(f"prefill library plan case={name} units={0 if c.prefill_units is None else len(c.prefill_units)} "
        f"pairs={c.num_prefill_pairs}")
    planned = staging.run_prefill(st)
    import dataclasses
    plain = astr.prefill_attn(st.q, dataclasses.replace(c, prefill_units=None, num_prefill_pairs=0,
                                                        prefill_workspace=None), cs.layer_id)
    torch.cuda.synchronize()
    want = E.expected_prefill(cs)
    off = E.new_offsets(cs)
    a, b_ = to_np(planned), to_np(plain)
    for b in range(cs.batch):
        E.assert_close(a[off[b]:off[b + 1]], want[b], cs.dtype, f"{name} planned request {b}")
        E.assert_close(b_[off[b]:off[b + 1]], want[b], cs.dtype, f"{name} unplanned request {b}")
    # the two differ only in the order of the softmax sums
    assert np.linalg.norm(a - b_) <= 2e-3 * np.linalg.norm(b_)


@pytest.mark.parametrize("plan", [False, True])
def test_prefill_tiles_past_total_q_are_skipped(plan):
    # q and out hold fewer rows than qo_indptr asks for: a tile whose rows
    # fall outside [0, total_q) is skipped (its rows stay as they were), every
    # other tile is computed as usual
    cs = PREFILL["ragged-65-129"]()
    off = E.new_offsets(cs)
    b = next(i for i in range(cs.batch) if cs.new_lens[i] >= 75)
    cut = int(off[b]) + 64 + 5                   # request b keeps its first tile, loses the rest
    say(f"prefill with total_q {cut} of {int(off[-1])} rows, plan={plan}")
    st = staging.stage(cs, plan=plan)
    staging.run_write(st)
    q = st.q[:cut].contiguous()
    out = torch.full_like(q, float("nan"))
    astr.prefill_attn(q, st.attn_cache, cs.layer_id, out=out)
    torch.cuda.synchronize()
    want = E.expected_prefill(cs)
    got = to_np(out)
    for r in range(cs.batch):
        for t in range(-(-int(cs.new_lens[r]) // 64)):
            lo, hi = int(off[r]) + 64 * t, min(int(off[r]) + 64 * (t + 1), int(off[r + 1]))
            if hi <= cut:
                E.assert_close(got[lo:hi], want[r][lo - int(off[r]):hi - int(off[r])], cs.dtype,
                               f"request {r} tile {t}")
            elif lo < cut:
                assert np.isnan(got[lo:cut]).all(), f"request {r} tile {t} crosses total_q and must be skipped"
