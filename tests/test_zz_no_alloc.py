"""The allocation-free decode entry point (astr_decode_attn_noalloc) on the
GPU: on two calls in a row, the second with a smaller batch, its output must
equal astr_decode_attn's bit for bit (same kernels, scratch in the library's
static array instead of a caller workspace) and match the float64 oracle."""

import numpy as np
import pytest
import torch

import expect as E
import paged_gqa_attention_rope_amd as astr
import staging
from workloads.gen import decode_case

pytestmark = pytest.mark.gpu


def _case(seed, **kw):
    base = dict(n_heads=16, n_kv_heads=4, head_dim=128, dtype="bf16", mode=1, page_size=16,
                shuffle_pages=True)
    base.update(kw)
    return decode_case(seed, **base)


CALLS = [
    ("8 requests, lengths to 3000, chunk 256",
     lambda: _case(61, batch=8, split_chunk=256, len_lo=200, len_hi=3000, log_uniform=True)),
    ("3 requests, lengths to 700, chunk 128",
     lambda: _case(62, batch=3, split_chunk=128, len_lo=1, len_hi=700)),
]


def test_noalloc_decode_equals_decode_attn_on_two_calls():
    for label, make in CALLS:
        cs = make()
        print(f"[no-alloc] {label}: lens={cs.seq_lens.tolist()}", flush=True)
        st = staging.stage(cs)
        staging.run_write(st)
        q = staging.decode_query(st)
        want = staging.run_decode(st)
        got = torch.full_like(q, float("nan"))
        astr.decode_attn_noalloc(q, st.attn_cache, cs.layer_id, cs.split_chunk, out=got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{label}: output bits differ"
        ref = E.expected_decode(cs)
        g = got.float().cpu().numpy().astype(np.float64)
        for b in range(cs.batch):
            E.assert_close(g[b], ref[b], cs.dtype, f"{label} request {b}")
