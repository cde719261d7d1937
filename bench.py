"""Benchmark of the paged GQA attention path on one MI355X.

One step = one pass of the whole path over one batch of each headline
workload, inputs already resident in HBM:
  decode  (256 requests, page 16, shuffled pages, 24-layer bf16 pool, 16/4
           heads, d 128, KV lengths log-uniform in [1024, 32768], split 512):
           rotary write of the new tokens + split-K decode + merge;
  prefill (16 requests, page 16, radix-cached prefixes 0..2048, extends
           32..512, 16/4 heads, d 128, bf16):
           rotary write of the extend tokens + causal prefill.
The page tables are built once, before timing (they are per-step host
metadata shared by all layers); their host cost is reported separately.

value = decode KV GB/s: algorithmic bytes (every cached K/V row read once,
its slot index, q read and output written) / the decode call's mean device
time over the timed steps (split-K pass + merge), from HIP events recorded
on the stream the kernels run on; the median is reported beside it.  The
prefill figure (TFLOP/s over unmasked (query, key) pairs) is in "prefill".
"configs" holds the other workloads: the tiny float32 decode, the
cache-resident 8-request decode and the 4-request contiguous prefill, each
the median of 50 calls with warm caches and with the caches flushed (a
512 MB write between calls).  "ceilings" holds what a plain streaming read
and a matrix-core loop attain on the same device.  cpu_baseline times the
float64 oracle on a bounded sample of the decode workload (and, under
"prefill", of the prefill workload) on the host cores.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak


def decode_bytes(cs) -> int:
    """Algorithmic bytes of one decode call: K and V rows (all KV heads) of every
    cached position, its 4-byte slot index, q read and output written."""
    esz = 2 if cs.dtype == "bf16" else 4
    row = cs.n_kv_heads * cs.head_dim * esz * 2 + 4
    return int(cs.seq_lens.sum()) * row + cs.batch * cs.n_heads * cs.head_dim * esz * 2


def prefill_flops(cs) -> int:
    """4*D*Hq per unmasked (query, key) pair: QK^T and PV, 2 flop per MAC."""
    e, p = cs.new_lens.astype(np.int64), cs.prefix_lens.astype(np.int64)
    pairs = int((e * p + e * (e + 1) // 2).sum())
    return 4 * cs.head_dim * cs.n_heads * pairs


PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_JSON = os.path.join(PROFILES, "hbm_traffic.json")
# sources whose change invalidates a call's counter figures (the prefill's
# traffic also depends on how its work plan places tiles on the XCDs)
KERNEL_SOURCES = {"decode": ("paged_gqa_attention_rope_amd/csrc/decode.hip",),
                  "prefill": ("paged_gqa_attention_rope_amd/csrc/prefill.hip",
                              "paged_gqa_attention_rope_amd/csrc/pagepool.cpp")}
# kernels (name prefixes in the rocprofv3 counter CSV) that make up each call
CALL_KERNELS = {"decode": ("decode_mfma_kernel<128, 4, false>", "decode_merge_kernel<astr::bf16_t, 128>"),
                "prefill": ("prefill_rs_kernel<4, false>",)}


def _sha(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        h.update(open(os.path.join(ROOT, path), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(call: str):
    """HBM bytes per call from the committed counter summary, or None when the
    kernel source has changed since the counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_JSON))[call]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != _sha(KERNEL_SOURCES[call]):
        return None
    return int(rec["fetch_bytes"] + rec["write_bytes"])


def summarize_pmc(fetch_dir: str, write_dir: str):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)
    into bytes per call, scaled by what each counter reads for the 1 GiB
    device copy of the same run (--copy-probe)."""
    import csv
    import glob

    def per_kernel(d, counter):
        # (kernel, grid in work-items) -> counter values: the same kernel runs
        # on the headline workloads and on smaller ones in one bench run
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    vals.setdefault((_short_name(r["Kernel_Name"]), int(r["Grid_Size"])), []).append(
                        float(r["Counter_Value"]))
        return vals

    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        v = per_kernel(d, counter)
        copy = max([max(x) for (name, _), x in v.items() if name.startswith("__amd_rocclr_copyBuffer")] or [0.0])
        if copy <= 0:
            raise SystemExit(f"no copy-probe dispatch in {d}")
        scale = 2 ** 30 / (copy * 1024.0)          # bytes per counter KiB
        for call, kernels in CALL_KERNELS.items():
            rec = out.setdefault(call, {"source_sha": _sha(KERNEL_SOURCES[call]), "kernels": {}})
            total = 0.0
            for k in kernels:
                # the headline workload is the largest launch of each kernel
                match = sorted(((grid, x) for (name, grid), x in v.items() if name.startswith(k)),
                               key=lambda gx: gx[0])
                if not match:
                    raise SystemExit(f"no {k} dispatch in {d}")
                grid, x = match[-1]
                kib = float(np.median(x))
                rec["kernels"].setdefault(k, {})[counter] = {"kib_per_dispatch": round(kib, 1),
                                                              "bytes": int(kib * 1024 * scale),
                                                              "grid": grid, "dispatches": len(x)}
                total += kib * 1024 * scale
            rec["fetch_bytes" if counter == "FETCH_SIZE" else "write_bytes"] = int(total)
            rec[f"{counter.lower()}_scale"] = round(scale, 5)
    os.makedirs(PROFILES, exist_ok=True)
    json.dump(out, open(TRAFFIC_JSON, "w"), indent=1)
    print(json.dumps(out, indent=1))


def _host_cores() -> int:
    return len(os.sched_getaffinity(0))


def cpu_baseline(cs, budget_s: float = 15.0):
    """The oracle, as it stands, on a bounded sample of the decode workload:
    requests in batch order until budget_s has passed, BLAS on every core
    this process may run on."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import expect as E
    from threadpoolctl import threadpool_limits
    cores = _host_cores()
    rot = E.rotated_new(cs)
    done, nbytes = [], 0
    esz = 2
    with threadpool_limits(cores):
        t0 = time.perf_counter()
        for b in range(cs.batch):
            E.expected_decode(cs, sample=[b], rot=rot)
            done.append(b)
            nbytes += int(cs.seq_lens[b]) * (cs.n_kv_heads * cs.head_dim * esz * 2 + 4) + \
                cs.n_heads * cs.head_dim * esz * 2
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"float64 decode of the first {len(done)} of {cs.batch} requests "
                      f"({int(cs.seq_lens[done].sum())} KV positions, history regenerated "
                      f"from the seeded streams), {dt:.1f} s"}


def cpu_baseline_prefill(cs, budget_s: float = 10.0):
    """The oracle on a bounded sample of the prefill workload: whole requests
    in batch order until budget_s has passed, in GFLOP/s over the same
    unmasked-pair count as the device figure."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import expect as E
    from threadpoolctl import threadpool_limits
    cores = _host_cores()
    rot = E.rotated_new(cs)
    done, flops = [], 0
    with threadpool_limits(cores):
        t0 = time.perf_counter()
        for b in range(cs.batch):
            E.expected_prefill(cs, sample=[b], rot=rot)
            done.append(b)
            e, p = int(cs.new_lens[b]), int(cs.prefix_lens[b])
            flops += 4 * cs.head_dim * cs.n_heads * (e * p + e * (e + 1) // 2)
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e9, 4), "unit": "GFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 causal prefill of the first {len(done)} of {cs.batch} requests "
                      f"({int(cs.new_lens[done].sum())} query rows, {flops / 1e9:.2f} GFLOP), {dt:.1f} s"}


def _time_ms(fn, stream, reps: int = 10, warm: int = 2) -> float:
    """Mean duration of fn() in ms over `reps` back-to-back calls, from two HIP
    events on `stream`.  A ~5 ms spin kernel goes first, so that every call
    is queued before the first one starts and host launch time stays out of
    the interval."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(10_000_000)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _rep_ms(fn, stream, reps: int = 50, warm: int = 3, flush=None) -> np.ndarray:
    """Durations (ms) of `reps` separate calls of fn(), each bracketed by its
    own pair of HIP events on `stream`.  With flush, flush() runs between
    calls, outside the brackets.  A spin kernel goes first so that the calls
    are queued ahead of the device and host launch time stays out."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda._sleep(40_000_000)
    for a, b in ev:
        if flush is not None:
            flush()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def _stats(ms: np.ndarray) -> dict:
    return {"median_us": round(float(np.median(ms)) * 1e3, 2), "mean_us": round(float(ms.mean()) * 1e3, 2),
            "min_us": round(float(ms.min()) * 1e3, 2), "reps": int(ms.size)}


def measure_small_configs(stream, dev):
    """The workloads other than the two headline batches, each measured on its
    own: median of 50 calls with warm caches, and with a 512 MB write
    between calls (which evicts the 256 MB last-level cache)."""
    import torch
    import paged_gqa_attention_rope_amd as astr
    import staging
    from workloads import make_case
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush = lambda: scratch.fill_(1)
    out = {}
    n_cus = torch.cuda.get_device_properties(dev).multi_processor_count

    # 1: tiny float32 decode, every position through the rotary write
    cs = make_case(1)
    st = staging.stage(cs, device=dev, canary=False)
    q_dec = staging.decode_query(st)
    res = {"workload": cs.name, "bound": "launch latency (50 tokens, 2 requests)"}
    for label, fl in (("hot", None), ("flushed", flush)):
        w = _rep_ms(lambda: staging.run_write(st), stream, flush=fl)
        d = _rep_ms(lambda: staging.run_decode(st, q_dec), stream, flush=fl)
        res[label] = {"rope_kv_write": _stats(w), "decode_attn": _stats(d)}
    out["1"] = res
    del st

    # 2: 8-request decode whose whole working set fits the last-level cache
    cs = make_case(2)
    st = staging.stage(cs, device=dev, canary=False)
    staging.run_write(st)
    q_dec = staging.decode_query(st)
    o_part, lse_part = astr.decode_workspace(st.attn_cache, cs.n_heads, cs.split_chunk)
    outd = torch.empty_like(q_dec)
    nbytes = decode_bytes(cs)
    res = {"workload": cs.name, "bytes_per_launch": nbytes,
           "bound": f"HBM in principle; the {nbytes / 1e6:.1f} MB working set fits the 256 MB last-level "
                    "cache, so warm calls read it from there"}
    for label, fl in (("hot", None), ("flushed", flush)):
        d = _rep_ms(lambda: staging.run_decode(st, q_dec, out=outd, o_part=o_part, lse_part=lse_part), stream,
                    flush=fl)
        gbs = nbytes / (float(np.median(d)) * 1e-3) / 1e9
        res[label] = {**_stats(d), "GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    out["2"] = res
    del st

    # 3: 4-request contiguous prefill, no prefix
    cs = make_case(3)
    st = staging.stage(cs, device=dev, canary=False)
    staging.run_write(st)
    outp = torch.empty_like(st.q)
    flops = prefill_flops(cs)
    c = st.attn_cache
    units = int(c.prefill_units.shape[0]) if c.prefill_units is not None else c.num_q_tiles
    real = int((c.prefill_units[:, 6] > 0).sum()) if c.prefill_units is not None else c.num_q_tiles
    wgs = real * (cs.n_heads // 4)
    steps = [(-(-(int(p) + min(64 * (t + 1), int(e))) // 32)) for e, p in zip(cs.new_lens, cs.prefix_lens)
             for t in range(-(-int(e) // 64))]
    res = {"workload": cs.name, "flops_per_launch": flops,
           "occupancy": {"query_tiles": c.num_q_tiles, "plan_units": units, "split_tiles": c.num_prefill_pairs,
                         "workgroups": wgs, "compute_units": n_cus, "waves_per_workgroup": 8,
                         "busy_cu_frac": round(min(wgs, n_cus) / n_cus, 3),
                         "longest_tile_key_steps": max(steps), "mean_tile_key_steps": round(float(np.mean(steps)), 1)},
           "bound": f"latency / occupancy: {wgs} workgroups (one per compute unit) for {n_cus} compute units, "
                    f"and the longest tile walks {max(steps)} steps of 32 keys against a mean of "
                    f"{np.mean(steps):.1f}"}
    for label, fl in (("hot", None), ("flushed", flush)):
        w = _rep_ms(lambda: staging.run_write(st), stream, flush=fl)
        p = _rep_ms(lambda: staging.run_prefill(st, out=outp), stream, flush=fl)
        tfs = flops / (float(np.median(p)) * 1e-3) / 1e12
        res[label] = {"rope_kv_write": _stats(w), "prefill_attn": {**_stats(p), "TFLOPs": round(tfs, 1),
                                                                  "frac_of_bf16_peak": round(tfs / BF16_PEAK_TFLOPS, 4)}}
    out["3"] = res
    del st, scratch
    torch.cuda.empty_cache()
    return out


def measure_ceilings(stream, dev):
    """What a plain streaming read (4 GiB of random bits, 16-byte loads) and a
    loop of independent matrix-core products attain on this device.  The read
    is timed at several grid sizes and the fastest is reported: the rate
    depends on the grid (8 workgroups per compute unit reads ~10% slower than
    24 on MI355X), and a ceiling should be the best the chip does."""
    import torch
    import paged_gqa_attention_rope_amd as astr
    n_cus = torch.cuda.get_device_properties(dev).multi_processor_count
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    # random bits, as the attention reads (HBM reads of constant data run ~4% faster)
    buf = torch.randn(1 << 30, dtype=torch.float32, device=dev, generator=gen)   # 4 GiB
    nbytes = buf.numel() * 4
    res = {}
    for nt in (True, False):
        best = None
        for per_cu in (8, 16, 24, 32):
            wg = per_cu * n_cus
            sink = torch.empty(wg, dtype=torch.int32, device=dev)
            ms = _rep_ms(lambda: astr.ceiling_stream_read(buf, wg, nt, sink), stream, reps=20)
            gbps = nbytes / (float(np.median(ms)) * 1e-3) / 1e9
            if best is None or gbps > best["GBps"]:
                best = {"GBps": round(gbps, 1), "bytes": nbytes, "workgroups": wg, **_stats(ms)}
        res["stream_read_nt" if nt else "stream_read"] = best
    del buf
    wg, iters = 4 * n_cus, 4096                                           # 4 waves per SIMD
    sink = torch.empty(256 * wg, dtype=torch.float32, device=dev)
    flops = astr.ceiling_mfma_loop(wg, iters, sink)
    ms = _rep_ms(lambda: astr.ceiling_mfma_loop(wg, iters, sink), stream, reps=20)
    res["mfma_bf16_16x16x32"] = {"TFLOPs": round(flops / (float(np.median(ms)) * 1e-3) / 1e12, 1),
                                 "flops": flops, "waves_per_simd": 4, **_stats(ms)}
    torch.cuda.empty_cache()
    return res


def measure_next_rows(st_d, cs_d, st_p, q_unrot, out_d, o_part, lse_part, stream, dbytes):
    """The adjacent rows: the fused decode write on the decode workload, and
    the rotary gradient on a gradient of the prefill batch's q shape."""
    import paged_gqa_attention_rope_amd as astr
    import staging
    write_then_decode_ms = _time_ms(lambda: (staging.run_write(st_d), staging.run_decode(
        st_d, out=out_d, o_part=o_part, lse_part=lse_part)), stream)
    fused_ms = _time_ms(lambda: astr.decode_attn_write(
        q_unrot, st_d.k, st_d.v, st_d.attn_cache, cs_d.layer_id, st_d.freqs, cs_d.split_chunk,
        out=out_d, o_part=o_part, lse_part=lse_part), stream)
    # the whole step over all layers: one metadata build, every layer's fused
    # decode write, eager and as one replayed HIP graph
    from paged_gqa_attention_rope_amd.step import DecodeStep
    nl = int(st_d.k_buffer.shape[0])
    lay = DecodeStep(st_d.attn_cache, st_d.freqs, q_unrot.expand(nl, *q_unrot.shape).contiguous(),
                     st_d.k.expand(nl, *st_d.k.shape).contiguous(),
                     st_d.v.expand(nl, *st_d.v.shape).contiguous(), cs_d.split_chunk)
    eager_ms = _time_ms(lay.run, stream, reps=3, warm=1)
    lay.capture()
    graph_ms = _time_ms(lay.replay, stream, reps=3, warm=1)
    del lay
    g = st_p.q.clone()
    t, h, d = (int(x) for x in g.shape)
    rb_bytes = 2 * g.numel() * g.element_size() + t * (d // 2) * 8    # grad read + written, table rows
    rb_ms = _time_ms(lambda: astr.rope_backward(g, st_p.positions, st_p.freqs), stream)
    return {
        "pagepool_lifecycle": measure_pagepool_lifecycle(),
        "decode_attn_write": {
            "workload": cs_d.name, "ms_per_launch": round(fused_ms, 5),
            "write_then_decode_ms": round(write_then_decode_ms, 5),
            "achieved_GBps": round(dbytes / (fused_ms * 1e-3) / 1e9, 2),
            "frac": round(dbytes / (fused_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "decode_step_all_layers": {
            "layers": nl, "eager_ms_per_step": round(eager_ms, 4), "graph_ms_per_step": round(graph_ms, 4),
            "graph_ms_per_layer": round(graph_ms / nl, 5),
            "achieved_GBps": round(nl * dbytes / (graph_ms * 1e-3) / 1e9, 2)},
        "rope_backward": {
            "shape": [t, h, d], "dtype": "bf16", "bytes_per_launch": rb_bytes,
            "ms_per_launch": round(rb_ms, 5),
            "achieved_GBps": round(rb_bytes / (rb_ms * 1e-3) / 1e9, 2),
            "frac": round(rb_bytes / (rb_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }


def measure_pagepool_lifecycle(n_requests=1536, batch=16, decode_steps=8, seed=6):
    """Host cost of the page-table builder's whole request lifecycle, through
    the Python binding, on a pool shaped like the prefill workload (page 16,
    65 536 slots) and too small to keep every finished prompt: batches of 16
    requests, each a prompt of one of 4 shared prefixes (16 * U{0..128}
    tokens) plus its own U{32..512} tokens, are admitted (radix lookup),
    extended, bound as one prefill step, run 8 decode steps (extend by one and
    bind each), then completed (cache the pages with KV, release)."""
    import paged_gqa_attention_rope_amd as astr
    rng = np.random.default_rng(seed)
    ps, slots, max_ctx = 16, 65536, 2560
    pp = astr.PagePool(1, slots, ps, batch, max_ctx)
    prefixes = [rng.integers(0, 32000, size=2048).astype(np.int32) for _ in range(4)]
    admitted = cached = 0
    t0 = time.perf_counter()
    t_bind = 0.0
    n_bind = 0
    for first in range(0, n_requests, batch):
        reqs, toks, lens, new = [], [], [], []
        for _ in range(min(batch, n_requests - first)):
            pre = prefixes[rng.integers(0, 4)][:ps * int(rng.integers(0, 129))]
            own = rng.integers(0, 32000, size=int(rng.integers(32, 513))).astype(np.int32)
            t = np.concatenate([pre, own, rng.integers(0, 32000, size=decode_steps).astype(np.int32)])
            n = len(pre) + len(own)
            r, c = pp.admit(t, n)
            pp.extend(r, n - c)
            reqs.append(r); toks.append(t); lens.append(n); new.append(n - c)
            admitted += n
            cached += c
        tb = time.perf_counter()
        pp.bind(reqs, new, 64)
        t_bind += time.perf_counter() - tb
        n_bind += 1
        for _ in range(decode_steps):
            for r in reqs:
                pp.extend(r, 1)
            tb = time.perf_counter()
            pp.bind(reqs, [1] * len(reqs), 64)
            t_bind += time.perf_counter() - tb
            n_bind += 1
        for r, t, n in zip(reqs, toks, lens):
            pp.complete(r, t, n + decode_steps)
    total = time.perf_counter() - t0
    return {"requests": n_requests, "batch": batch, "decode_steps": decode_steps,
            "pool_pages": slots // ps, "us_per_request": round(total / n_requests * 1e6, 2),
            "us_per_bind": round(t_bind / n_bind * 1e6, 2),
            "prefix_hit_frac": round(cached / admitted, 4), "pages_evicted": pp.evicted_pages(),
            "pages_cached_at_end": pp.cached_pages()}


def _short_name(kernel_name: str) -> str:
    return kernel_name.replace("void ", "", 1).replace("astr::(anonymous namespace)::", "", 1).split("(")[0]


def summarize_trace(trace_dir: str):
    """Per-kernel call count, mean and median duration (us) from a rocprofv3
    --kernel-trace run (its kernel_trace.csv), one row per kernel and launch
    size (workgroups), as a markdown table."""
    import csv
    import glob
    rows = {}
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            name = _short_name(r["Kernel_Name"])
            if not any(k in name for k in ("decode", "prefill", "rope", "stream_read", "mfma_loop")):
                continue
            wgs = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) // max(
                1, int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"]))
            rows.setdefault((name, wgs), []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print("| kernel | workgroups | calls | mean | median | min | max |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for name, wgs in sorted(rows):
        v = np.array(rows[(name, wgs)])
        print(f"| `{name}` | {wgs} | {v.size} | {v.mean():.2f} | {np.median(v):.2f} | {v.min():.2f} | {v.max():.2f} |")


def _gpu_agent(pmc_dir: str):
    """(compute units, XCDs) of the GPU agent from rocprofv3's agent-info file."""
    import csv
    import glob
    for f in glob.glob(os.path.join(pmc_dir, "**", "*agent_info.csv"), recursive=True):
        for a in csv.DictReader(open(f)):
            if a.get("Agent_Type", "").upper() == "GPU":
                return int(a["Cu_Count"]), int(a["Num_Xcc"])
    return None


def summarize_counters(pmc_dir: str):
    """Mean of every counter per kernel and launch size (workgroups) from a
    rocprofv3 --pmc run, as a markdown table (attention-path kernels only).
    Derived columns where their counters were taken: the L2 hit rate
    TCC_HIT / (TCC_HIT + TCC_MISS), and the mean waves resident per SIMD,
    SQ_WAVE_CYCLES (quad-cycles summed over all waves) x 4 over the dispatch's
    active cycles per XCD (GRBM_GUI_ACTIVE, summed over the XCDs) x 4 SIMDs x
    compute units (rocprof's OccupancyPercent is the same ratio over 32 waves
    per compute unit)."""
    import csv
    import glob
    vals, names = {}, []
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            name = _short_name(r["Kernel_Name"])
            if not any(k in name for k in ("decode", "prefill", "rope")):
                continue
            wgs = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
            c = r["Counter_Name"]
            if c not in names:
                names.append(c)
            vals.setdefault((name, wgs), {}).setdefault(c, {})[int(r["Dispatch_Id"])] = float(r["Counter_Value"])
    agent = _gpu_agent(pmc_dir)
    hit = "TCC_HIT_sum" in names and "TCC_MISS_sum" in names
    occ = "SQ_WAVE_CYCLES" in names and "GRBM_GUI_ACTIVE" in names and agent is not None
    extra = (["L2 hit %"] if hit else []) + (["waves per SIMD"] if occ else [])
    print("| kernel | workgroups | dispatches | " + " | ".join(names + extra) + " |")
    print("|---|---:|---:|" + "---:|" * (len(names) + len(extra)))
    for key in sorted(vals):
        per = vals[key]
        n = max(len(per.get(c, {})) for c in names)
        mean = {c: float(np.mean(list(per[c].values()))) for c in names if c in per}
        cells = [f"{mean[c]:,.0f}" if c in mean else "" for c in names]
        if hit:
            h, m = mean.get("TCC_HIT_sum", 0.0), mean.get("TCC_MISS_sum", 0.0)
            cells.append(f"{100.0 * h / (h + m):.1f}" if h + m > 0 else "")
        if occ:
            cus, xcds = agent
            active = mean.get("GRBM_GUI_ACTIVE", 0.0) / xcds
            cells.append(f"{mean.get('SQ_WAVE_CYCLES', 0.0) / (active * cus):.2f}" if active > 0 else "")
        print(f"| `{key[0]}` | {key[1]} | {n} | " + " | ".join(cells) + " |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline steps (no other workloads, ceilings or adjacent rows)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one 1 GiB device-to-device copy (a reference dispatch of "
                         "known size for calibrating HBM byte counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/hbm_traffic.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-counters", metavar="PMC_DIR",
                    help="print the mean of each counter per kernel and launch size of a rocprofv3 "
                         "--pmc run and exit")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="print per-kernel call counts, mean and median durations of a rocprofv3 "
                         "--kernel-trace run and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(requests shard across GPUs with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import staging
    from workloads import make_case

    def say(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    t_stage = time.perf_counter()
    cs_d = make_case(5, args.seed)
    cs_p = make_case(4, args.seed)
    st_p = staging.stage(cs_p, device=dev, canary=False)
    st_d = staging.stage(cs_d, device=dev, canary=False)
    say(f"staged decode ({cs_d.pool_slots} slots x {cs_d.n_layers} layers) and prefill "
        f"in {time.perf_counter() - t_stage:.1f} s")
    # host cost of one step's metadata build (decode: every request appends a token)
    t0 = time.perf_counter()
    st_d.pool.bind(st_d.reqs, np.ones(cs_d.batch, dtype=np.int32), 64)
    bind_ms = (time.perf_counter() - t0) * 1e3
    # and of the prefill work plan (built once per step, shared by all layers;
    # median of 5 builds, as a serving loop builds one per step)
    import paged_gqa_attention_rope_amd as astr
    n_cus = torch.cuda.get_device_properties(dev).multi_processor_count
    plan_times = []
    for _ in range(5):
        t0 = time.perf_counter()
        astr.prefill_plan(st_p.attn_meta, cs_p.n_heads, n_cus)
        plan_times.append((time.perf_counter() - t0) * 1e3)
    plan_ms = float(np.median(plan_times))

    q_dec = staging.decode_query(st_d)
    q_unrot = q_dec.clone()                     # the fused decode takes q before rotation
    out_d = torch.empty_like(q_dec)
    o_part, lse_part = astr.decode_workspace(st_d.attn_cache, cs_d.n_heads, cs_d.split_chunk)
    out_p = torch.empty_like(st_p.q)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        staging.run_write(st_d)
        if ev:
            ev[1].record(stream)
        staging.run_decode(st_d, q_dec, out=out_d, o_part=o_part, lse_part=lse_part)
        if ev:
            ev[2].record(stream)
        staging.run_write(st_p)
        if ev:
            ev[3].record(stream)
        staging.run_prefill(st_p, out=out_p)
        if ev:
            ev[4].record(stream)

    if args.copy_probe:
        src = torch.ones(2 ** 28, dtype=torch.float32, device=dev)     # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    say(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    parts = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(4)]
                      for i in range(args.steps)])             # ms
    t_wd, t_dec, t_wp, t_pre = parts.mean(axis=0)
    m_wd, m_dec, m_wp, m_pre = np.median(parts, axis=0)
    dbytes = decode_bytes(cs_d)
    pflops = prefill_flops(cs_p)
    dec_gbs = dbytes / (t_dec * 1e-3) / 1e9
    pre_tfs = pflops / (t_pre * 1e-3) / 1e12

    nxt = configs = ceilings = back = None
    if not args.no_extras:
        # the prefill alone, warm: 20 groups of 5 back-to-back calls, one event
        # pair per group (in the step, the decode's 4.7 GB stream has just
        # evicted the prefill's keys and values from the caches)
        say("prefill back to back")
        groups = _rep_ms(lambda: [staging.run_prefill(st_p, out=out_p) for _ in range(5)], stream, reps=20) / 5
        back = {"what": "prefill_attn alone, warm caches, 5 calls per event pair", **_stats(groups),
                "TFLOPs": round(pflops / (float(np.median(groups)) * 1e-3) / 1e12, 1),
                "frac_of_bf16_peak": round(pflops / (float(np.median(groups)) * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        say("adjacent rows")
        nxt = measure_next_rows(st_d, cs_d, st_p, q_unrot, out_d, o_part, lse_part, stream, dbytes)
        del st_d, o_part, lse_part
        torch.cuda.empty_cache()
        say("other workloads")
        configs = measure_small_configs(stream, dev)
        say("ceilings")
        ceilings = measure_ceilings(stream, dev)

    cpu = cpu_p = None
    if not args.no_cpu_baseline:
        say("oracle baselines")
        cpu = cpu_baseline(cs_d)
        cpu_p = cpu_baseline_prefill(cs_p)

    def attainable(rate, key, unit):
        if not ceilings:
            return None
        return {"ceiling": key, "attainable": ceilings[key][unit], "unit": "GB/s" if unit == "GBps" else "TFLOP/s",
                "frac": round(rate / ceilings[key][unit], 4)}

    line = {
        "metric": "decode attn KV GB/s (% HBM peak) + prefill attn TFLOP/s (% bf16 MFMA peak)",
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": cs_d.name,
            "prefill_workload": cs_p.name,
            "decode_batch": cs_d.batch, "decode_kv_positions": int(cs_d.seq_lens.sum()),
            "decode_split_chunk": cs_d.split_chunk, "layer_id": cs_d.layer_id,
            "prefill_batch": cs_p.batch, "prefill_rows": int(cs_p.new_lens.sum()),
            "prefill_cached_prefix": int(cs_p.prefix_lens.sum()),
        },
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("decode"),
                     "kernel": "decode_attn (split-K pass + merge)",
                     "bytes_per_launch": dbytes, "ms_per_launch": round(float(t_dec), 5),
                     "median_ms_per_launch": round(float(m_dec), 5),
                     "attainable": attainable(dec_gbs, "stream_read_nt", "GBps")},
        "prefill": {"value": round(pre_tfs, 2), "unit": "TFLOP/s",
                    "roofline": {"bound": "mfma", "achieved": round(pre_tfs, 2),
                                 "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(pre_tfs / BF16_PEAK_TFLOPS, 4),
                                 "traffic": measured_traffic("prefill"),
                                 "kernel": "prefill_attn", "flops_per_launch": pflops,
                                 "ms_per_launch": round(float(t_pre), 5),
                                 "median_ms_per_launch": round(float(m_pre), 5),
                                 "attainable": attainable(pre_tfs, "mfma_bf16_16x16x32", "TFLOPs")},
                    "back_to_back": back,
                    "plan": {"units": 0 if st_p.attn_cache.prefill_units is None
                             else int(st_p.attn_cache.prefill_units.shape[0]),
                             "split_tiles": int(st_p.attn_cache.num_prefill_pairs)},
                    "cpu_baseline": cpu_p},
        "parts_ms": {"rope_kv_write_decode": round(float(t_wd), 5), "decode_attn": round(float(t_dec), 5),
                     "rope_kv_write_prefill": round(float(t_wp), 5), "prefill_attn": round(float(t_pre), 5),
                     "median": {"rope_kv_write_decode": round(float(m_wd), 5), "decode_attn": round(float(m_dec), 5),
                                "rope_kv_write_prefill": round(float(m_wp), 5),
                                "prefill_attn": round(float(m_pre), 5)},
                     "host_bind_decode": round(bind_ms, 3), "host_plan_prefill": round(plan_ms, 3)},
        "configs": configs,
        "ceilings": ceilings,
        "next": nxt,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
