"""CPU checks of bench.py's rocprofv3 summarizers on small synthetic CSV
files: the tables under profiles/ and the bench line's `traffic` field come
from them, so a wrong pick of the headline launch, a wrong calibration or a
stale figure would misreport the measurements."""

import csv
import json
import os

import pytest

import bench

NS = "void astr::(anonymous namespace)::"


def _csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _counters(d, rows):
    """rows: (dispatch, kernel, grid work-items, workgroup size, counter, value)."""
    _csv(os.path.join(d, "run_counter_collection.csv"),
         ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Workgroup_Size", "Counter_Name", "Counter_Value"],
         [(i, g, k, wg, c, v) for i, k, g, wg, c, v in rows])


def _pmc_case(tmp_path, counter, copy_kib, vals):
    """One counter pass: a staging copy, the 1 GiB copy probe, then each
    (kernel, grid, values) as that many dispatches."""
    d = str(tmp_path / counter)
    rows = [(1, "__amd_rocclr_copyBuffer", 131072, 256, counter, 100.0),
            (2, "__amd_rocclr_copyBuffer", 131072, 256, counter, copy_kib)]
    for name, grid, v in vals:
        for x in v:
            rows.append((len(rows) + 1, NS + name + "(int, float*)", grid, 256, counter, x))
    _counters(d, rows)
    return d


@pytest.fixture
def sources(tmp_path, monkeypatch):
    """Point the hashed sources and the traffic record at temporary files."""
    srcs = {}
    for call in ("decode", "prefill"):
        p = tmp_path / f"{call}.src"
        p.write_text(f"// {call} kernel source\n")
        srcs[call] = (str(p),)
    monkeypatch.setattr(bench, "KERNEL_SOURCES", srcs)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "profiles" / "hbm_traffic.json"))
    return srcs


def test_summarize_pmc_picks_headline_launch_and_calibrates(tmp_path, sources, capsys):
    dec, mrg, pre = bench.CALL_KERNELS["decode"][0], bench.CALL_KERNELS["decode"][1], bench.CALL_KERNELS["prefill"][0]
    # FETCH_SIZE reads half a copy's bytes (scale 2), WRITE_SIZE all of them (scale 1)
    fetch = [(dec, 4096, [7.0, 7.0]), (dec, 4702208, [1000.0, 1004.0, 1001.0]),
             (mrg, 262144, [20.0]), (pre, 212992, [300.0, 302.0, 301.0]), (pre, 65536, [5.0])]
    write = [(dec, 4702208, [40.0, 40.0, 40.0]), (dec, 4096, [1.0]),
             (mrg, 262144, [1.0]), (pre, 212992, [21.0, 21.0, 21.0])]
    fd = _pmc_case(tmp_path, "FETCH_SIZE", 524288.0, fetch)
    wd = _pmc_case(tmp_path, "WRITE_SIZE", 1048576.0, write)
    bench.summarize_pmc(fd, wd)
    rec = json.load(open(bench.TRAFFIC_JSON))
    kd = rec["decode"]["kernels"][dec]
    assert kd["FETCH_SIZE"]["grid"] == 4702208 and kd["FETCH_SIZE"]["dispatches"] == 3
    assert kd["FETCH_SIZE"]["kib_per_dispatch"] == 1001.0                       # median, largest launch
    assert rec["decode"]["fetch_size_scale"] == 2.0 and rec["decode"]["write_size_scale"] == 1.0
    assert rec["decode"]["fetch_bytes"] == int((1001.0 + 20.0) * 1024 * 2.0)
    assert rec["decode"]["write_bytes"] == int((40.0 + 1.0) * 1024)
    assert rec["prefill"]["fetch_bytes"] == int(301.0 * 1024 * 2.0)
    assert rec["prefill"]["kernels"][pre]["FETCH_SIZE"]["grid"] == 212992
    # the bench reports the figure while the sources match, and drops it after a change
    assert bench.measured_traffic("decode") == rec["decode"]["fetch_bytes"] + rec["decode"]["write_bytes"]
    with open(sources["decode"][0], "a") as f:
        f.write("// changed\n")
    assert bench.measured_traffic("decode") is None
    assert bench.measured_traffic("prefill") is not None


def test_summarize_pmc_requires_the_copy_probe(tmp_path, sources):
    dec = bench.CALL_KERNELS["decode"][0]
    d = str(tmp_path / "nocopy")
    _counters(d, [(1, NS + dec + "(int)", 64, 64, "FETCH_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(d, d)


def test_summarize_trace_rows_per_kernel_and_launch_size(tmp_path, capsys):
    hdr = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z",
           "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z"]
    k = NS + "decode_mfma_kernel<128, 4, false>(int, float*)"
    rows = [(k, 0, 700_000, 4702208, 1, 1, 256, 1, 1),        # 18368 workgroups, 700 us
            (k, 0, 710_000, 4702208, 1, 1, 256, 1, 1),
            (k, 0, 760_000, 4702208, 1, 1, 256, 1, 1),
            (k, 0, 9_000, 32768, 1, 1, 256, 1, 1),            # 128 workgroups, 9 us
            ("void at::native::vectorized_elementwise_kernel<4>(int)", 0, 5_000, 1024, 1, 1, 256, 1, 1)]
    _csv(str(tmp_path / "trace" / "run_kernel_trace.csv"), hdr, rows)
    bench.summarize_trace(str(tmp_path / "trace"))
    out = capsys.readouterr().out.strip().splitlines()
    assert out[0].startswith("| kernel | workgroups | calls |")
    body = {tuple(c.strip() for c in line.strip("|").split("|")[:3]): line for line in out[2:]}
    assert len(out) == 4                                      # torch's kernel is not listed
    big = body[("`decode_mfma_kernel<128, 4, false>`", "18368", "3")]
    cells = [c.strip() for c in big.strip("|").split("|")]
    assert cells[3:] == ["723.33", "710.00", "700.00", "760.00"]   # mean, median, min, max (us)
    assert ("`decode_mfma_kernel<128, 4, false>`", "128", "1") in body


def test_summarize_counters_means_per_launch_size(tmp_path, capsys):
    k = NS + "prefill_rs_kernel<4, false>(int)"
    rows = [(1, k, 212992, 512, "SQ_INSTS_MFMA", 100.0), (1, k, 212992, 512, "GRBM_GUI_ACTIVE", 10.0),
            (2, k, 212992, 512, "SQ_INSTS_MFMA", 300.0), (2, k, 212992, 512, "GRBM_GUI_ACTIVE", 30.0),
            (3, k, 98304, 512, "SQ_INSTS_MFMA", 7.0), (3, k, 98304, 512, "GRBM_GUI_ACTIVE", 1.0)]
    _counters(str(tmp_path / "pmc"), rows)
    bench.summarize_counters(str(tmp_path / "pmc"))
    out = capsys.readouterr().out.strip().splitlines()
    assert out[0] == "| kernel | workgroups | dispatches | SQ_INSTS_MFMA | GRBM_GUI_ACTIVE |"
    assert "| `prefill_rs_kernel<4, false>` | 416 | 2 | 200 | 20 |" in out
    assert "| `prefill_rs_kernel<4, false>` | 192 | 1 | 7 | 1 |" in out


def test_summarize_counters_derives_l2_hits_and_waves_per_simd(tmp_path, capsys):
    # 2 XCDs of 4 compute units: GRBM_GUI_ACTIVE 400 summed = 200 active cycles
    # per XCD; SQ_WAVE_CYCLES 1600 quad-cycles = 6400 wave-cycles over
    # 200 cycles x 16 SIMDs = 2 waves per SIMD; 30 hits of 40 requests = 75%
    d = str(tmp_path / "pmc")
    k = NS + "prefill_rs_kernel<4, false>(int)"
    rows = [(1, k, 212992, 512, "TCC_HIT_sum", 30.0), (1, k, 212992, 512, "TCC_MISS_sum", 10.0),
            (1, k, 212992, 512, "SQ_WAVE_CYCLES", 1600.0), (1, k, 212992, 512, "GRBM_GUI_ACTIVE", 400.0)]
    _counters(d, rows)
    _csv(os.path.join(d, "run_agent_info.csv"), ["Agent_Type", "Cu_Count", "Num_Xcc"],
         [("CPU", "0", "0"), ("GPU", "4", "2")])
    bench.summarize_counters(d)
    out = capsys.readouterr().out.strip().splitlines()
    assert out[0].endswith("| L2 hit % | waves per SIMD |")
    assert out[2].endswith("| 75.0 | 2.00 |")


def test_summarize_counters_omits_occupancy_without_agent_info(tmp_path, capsys):
    d = str(tmp_path / "pmc")
    k = NS + "prefill_rs_kernel<4, false>(int)"
    _counters(d, [(1, k, 212992, 512, "SQ_WAVE_CYCLES", 1600.0), (1, k, 212992, 512, "GRBM_GUI_ACTIVE", 400.0)])
    bench.summarize_counters(d)
    out = capsys.readouterr().out.strip().splitlines()
    assert "waves per SIMD" not in out[0]
