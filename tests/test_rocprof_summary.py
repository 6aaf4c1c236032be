"""The rocprofv3 summaries behind the committed profiles, on small synthetic
CSV files in rocprofv3's column layout (no GPU): kernel names, per-kernel and
per-launch-shape times, counter averages, the HBM-traffic scaling by a copy
of known size, and the engine figures (matrix-core busy fraction, L2 hit
rate, VALU instructions per MFMA)."""
from __future__ import annotations

import csv
import json
import os

import pytest

from paged_kv_attention_kvcache_amd import rocprof_summary as rs

DECODE = "void pkv::decode_whole<pkv::BF16, pkv::ValuFold<pkv::BF16, 128, 2, false>, 8>(uint4 const*, int)"
COPY = "void at::native::copy_kernel<float>(float*, float const*)"


def _write(path, header, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def _counters(d, rows):
    """rows: (dispatch, kernel, grid, counter, value, start_ns, end_ns)."""
    os.makedirs(d, exist_ok=True)
    hdr = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value",
           "Start_Timestamp", "End_Timestamp"]
    _write(os.path.join(d, "run_counter_collection.csv"), hdr, rows)


def test_short_name_keeps_templates_drops_arguments():
    assert rs.short_name(DECODE) == \
        "pkv::decode_whole<pkv::BF16, pkv::ValuFold<pkv::BF16, 128, 2, false>, 8>"
    assert rs.short_name("void k(int)") == "k"
    assert len(rs.short_name("x" * 300)) == 110


def test_kernel_and_shape_stats(tmp_path):
    d = str(tmp_path)
    _write(os.path.join(d, "run_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
           [[DECODE, 4, 240000, 60000, 75.0, 58000, 62000]])
    _write(os.path.join(d, "run_kernel_trace.csv"),
           ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp",
            "End_Timestamp"],
           [[DECODE, 131072, 1, 1, 0, 58000], [DECODE, 131072, 1, 1, 100000, 162000],
            [DECODE, 65536, 1, 1, 200000, 230000]])
    st = rs.kernel_stats(d)
    assert st == [{"name": rs.short_name(DECODE), "calls": 4, "avg_us": 60.0, "min_us": 58.0,
                   "max_us": 62.0, "pct": 75.0}]
    sh = {r["grid"]: r for r in rs.shape_stats(d)}
    assert sh[(131072, 1, 1)]["calls"] == 2 and sh[(131072, 1, 1)]["avg_us"] == 60.0
    assert sh[(65536, 1, 1)]["min_us"] == 30.0


def test_traffic_scales_by_the_copy_probe(tmp_path):
    # a copy of 1 MiB reads 512 KiB of FETCH_SIZE (scale 2) and writes 1024
    # KiB (scale 1); the kernel reads 1000 KiB and writes 10 KiB per dispatch
    base = str(tmp_path)
    _counters(os.path.join(base, "cf"), [[1, 256, COPY, "FETCH_SIZE", 512.0, 0, 10]])
    _counters(os.path.join(base, "cw"), [[1, 256, COPY, "WRITE_SIZE", 1024.0, 0, 10]])
    _counters(os.path.join(base, "kf"), [[1, 131072, DECODE, "FETCH_SIZE", 1000.0, 0, 10],
                                         [2, 131072, DECODE, "FETCH_SIZE", 1000.0, 20, 30]])
    _counters(os.path.join(base, "kw"), [[1, 131072, DECODE, "WRITE_SIZE", 10.0, 0, 10]])
    out = os.path.join(base, "t.json")
    rs.main(["traffic", "--fetch", os.path.join(base, "kf"), "--write", os.path.join(base, "kw"),
             "--copy-fetch", os.path.join(base, "cf"), "--copy-write", os.path.join(base, "cw"),
             "--kernel", "decode_whole", "--copy-bytes", str(1 << 20), "--json", out])
    res = json.load(open(out))
    assert res["fetch_scale"] == 2.0 and res["write_scale"] == 1.0
    assert res["hbm_read_bytes_per_launch"] == 2000 * 1024
    assert res["hbm_write_bytes_per_launch"] == 10 * 1024
    assert res["kernel_source_hash"] == rs.kernel_source_hash()


def test_engine_figures(tmp_path):
    # one dispatch of 100 us: 1024 SIMDs x 2.4 GHz x 100 us = 245.76 M SIMD
    # clocks, of which 61.44 M busy -> 25%; 300 of 400 L2 requests hit
    d = str(tmp_path / "e")
    rows = [[1, 524288, DECODE, c, v, 1000, 101000] for c, v in (
        ("SQ_VALU_MFMA_BUSY_CYCLES", 61.44e6), ("SQ_INSTS_VALU", 390.0), ("SQ_INSTS_MFMA", 100.0),
        ("TCC_HIT_sum", 300.0), ("TCC_MISS_sum", 100.0))]
    _counters(d, rows)
    (r,) = rs.engine_counters(d, "decode_whole")
    assert r["grid"] == 524288 and r["dispatches"] == 1 and r["us"] == pytest.approx(100.0)
    assert r["mfma_busy"] == pytest.approx(0.25)
    assert r["l2_hit"] == pytest.approx(0.75)
    assert r["valu_per_mfma"] == pytest.approx(3.9)
    assert rs.engine_counters(d, "prefill") == []


def test_source_hash_covers_every_library_source(tmp_path, monkeypatch):
    h = rs.kernel_source_hash()
    assert len(h) == 16 and h == rs.kernel_source_hash()
    # a change to any source (a prefill kernel, the host code) changes the hash
    import shutil

    fake = tmp_path / "pkg"
    shutil.copytree(os.path.join(rs.HERE, "csrc"), fake / "csrc")
    monkeypatch.setattr(rs, "HERE", str(fake))
    assert rs.kernel_source_hash() == h
    for name in ("prefill_mfma.hip", "pagedkv.cpp", "span.hpp"):
        p = fake / "csrc" / name
        old = p.read_text()
        p.write_text(old + "\n")
        assert rs.kernel_source_hash() != h, name
        p.write_text(old)


def test_workload_figures(tmp_path):
    # Two workloads in one trace: the long-context call (stream kernel 3200 us
    # + combine 13 us) and the 8 x 2048 prefill (grid 524288; the 131072-grid
    # prefill calls belong to another workload). Copy probe: scales 2 and 1.
    base = str(tmp_path)
    stream = "void pkv::decode_stream<pkv::BF16, pkv::MfmaFold<8, false, false> >(uint4 const*)"
    comb = "void pkv::decode_stream_combine<pkv::BF16, 8>(int)"
    pre = "void pkv::prefill_mfma<4, 2, 2048>(uint4 const*)"
    st = os.path.join(base, "st")
    os.makedirs(st)
    _write(os.path.join(st, "run_kernel_trace.csv"),
           ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp",
            "End_Timestamp"],
           [[stream, 262144, 1, 1, 0, 3200000], [stream, 262144, 1, 1, 0, 3210000],
            [comb, 524288, 1, 1, 0, 13000], [pre, 524288, 1, 1, 0, 330000],
            [pre, 131072, 1, 1, 0, 39000]])
    _counters(os.path.join(base, "cf"), [[1, 256, COPY, "FETCH_SIZE", 512.0, 0, 10]])
    _counters(os.path.join(base, "cw"), [[1, 256, COPY, "WRITE_SIZE", 1024.0, 0, 10]])
    _counters(os.path.join(base, "kf"), [[1, 262144, stream, "FETCH_SIZE", 1000.0, 0, 10],
                                         [2, 524288, comb, "FETCH_SIZE", 10.0, 0, 10],
                                         [3, 524288, pre, "FETCH_SIZE", 300.0, 0, 10],
                                         [4, 131072, pre, "FETCH_SIZE", 99.0, 0, 10]])
    _counters(os.path.join(base, "kw"), [[1, 262144, stream, "WRITE_SIZE", 4.0, 0, 10],
                                         [2, 524288, comb, "WRITE_SIZE", 2.0, 0, 10],
                                         [3, 524288, pre, "WRITE_SIZE", 100.0, 0, 10],
                                         [4, 131072, pre, "WRITE_SIZE", 9.0, 0, 10]])
    out = os.path.join(base, "w.json")
    rs.main(["workloads", "--stats", st, "--fetch", os.path.join(base, "kf"),
             "--write", os.path.join(base, "kw"), "--copy-fetch", os.path.join(base, "cf"),
             "--copy-write", os.path.join(base, "cw"), "--copy-bytes", str(1 << 20),
             "--json", out])
    res = json.load(open(out))
    assert res["kernel_source_hash"] == rs.kernel_source_hash()
    w = res["workloads"]
    assert set(w) == {"longctx", "prefill_8x2048", "prefill_cold2048"}
    assert w["longctx"]["us_per_call"] == pytest.approx(3205.0 + 13.0)
    assert w["longctx"]["hbm_bytes_per_call"] == (1010 * 2 + 6) * 1024
    assert w["prefill_8x2048"]["us_per_call"] == pytest.approx(330.0)
    assert w["prefill_8x2048"]["hbm_bytes_per_call"] == (300 * 2 + 100) * 1024
    assert w["prefill_cold2048"]["us_per_call"] == pytest.approx(39.0)


def test_write_profiles_from_a_collection(tmp_path):
    # every summary collect_profiles.sh asks for, from minimal runs of each kind
    out = tmp_path / "out"
    ouro = "void pkv::decode_whole<pkv::BF16, pkv::ValuFold<pkv::BF16, 128, 2, false>, 8>(int)"
    pre = "void pkv::prefill_mfma<4, 2, 2048>(uint4 const*)"
    st = out / "stats_default"
    st.mkdir(parents=True)
    _write(str(st / "run_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
           [[ouro, 2, 120000, 60000, 50.0, 59000, 61000], [pre, 1, 330000, 330000, 50.0,
                                                           330000, 330000]])
    _write(str(st / "run_kernel_trace.csv"),
           ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp",
            "End_Timestamp"],
           [[ouro, 131072, 1, 1, 0, 59000], [ouro, 131072, 1, 1, 0, 61000],
            [pre, 524288, 1, 1, 0, 330000]])
    _counters(str(out / "copy_fetch"), [[1, 256, COPY, "FETCH_SIZE", 512.0, 0, 10]])
    _counters(str(out / "copy_write"), [[1, 256, COPY, "WRITE_SIZE", 1024.0, 0, 10]])
    _counters(str(out / "all_fetch"), [[1, 131072, ouro, "FETCH_SIZE", 100.0, 0, 10],
                                      [2, 524288, pre, "FETCH_SIZE", 300.0, 0, 10]])
    _counters(str(out / "all_write"), [[1, 131072, ouro, "WRITE_SIZE", 1.0, 0, 10],
                                      [2, 524288, pre, "WRITE_SIZE", 100.0, 0, 10]])
    _counters(str(out / "prefill_engine"), [[1, 524288, pre, "SQ_VALU_MFMA_BUSY_CYCLES", 1e6,
                                             0, 100000]])
    _counters(str(out / "prefill_pipeline"),
              [[1, 524288, pre, "SQ_BUSY_CU_CYCLES", 256 * 2e5, 0, 100000],
               [1, 524288, pre, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 8e4, 0, 100000],
               [1, 524288, pre, "SQ_INSTS_LDS_LOAD_BANDWIDTH", 256 * 2e5 / 64 * 50, 0, 100000],
               [1, 524288, pre, "SQ_WAIT_ANY", 30.0, 0, 100000],
               [1, 524288, pre, "SQ_WAVE_CYCLES", 100.0, 0, 100000]])
    _counters(str(out / "all_l2"), [[1, 131072, ouro, "TCC_HIT_sum", 10.0, 0, 10],
                                   [1, 131072, ouro, "TCC_MISS_sum", 90.0, 0, 10]])
    _counters(str(out / "decode_tcp"), [[1, 131072, ouro, "TCP_TCC_READ_REQ_LATENCY_sum", 5000.0,
                                         0, 10],
                                        [1, 131072, ouro, "TCP_TCC_READ_REQ_sum", 10.0, 0, 10]])
    _counters(str(out / "decode_tcc"), [[1, 131072, ouro, "TCC_EA0_RDREQ_LEVEL_sum", 1400.0, 0, 10],
                                        [1, 131072, ouro, "TCC_EA0_RDREQ_sum", 1.0, 0, 10]])
    _counters(str(out / "decode_sq"), [[1, 131072, ouro, "SQ_INSTS_VALU", 7.0, 0, 10]])
    prof = tmp_path / "profiles"
    rs.main(["write", str(out), "--profiles", str(prof)])
    names = sorted(os.listdir(prof))
    assert names == ["bench_default_kernel_stats.txt", "decode_memory_counters.txt",
                     "hbm_traffic.txt", "kernels.json", "l2_hit_rates.txt",
                     "prefill_engine_counters.txt"]
    k = json.load(open(prof / "kernels.json"))
    assert k["workloads"]["ouro"]["us_per_call"] == pytest.approx(60.0)
    # the copy probe of 1 GiB read 512 KiB of FETCH_SIZE and 1024 KiB of WRITE_SIZE
    assert k["workloads"]["prefill_8x2048"]["hbm_bytes_per_call"] == \
        300 * 1024 * 2048 + 100 * 1024 * 1024
    # 2e5 busy cycles per CU over a 100 us dispatch: 2 GHz; the matrix cores
    # 8e4 of them (40%); 50 B of LDS reads per CU-cycle; waves wait 30%
    pipe = (prof / "prefill_engine_counters.txt").read_text()
    for want in ("clock_ghz                    2", "mfma_busy_at_clock           0.4",
                 "lds_read_B_per_clk_cu        50", "wave_wait_frac               0.3"):
        assert want in pipe, want
    text = (prof / "decode_memory_counters.txt").read_text()
    assert "l1_to_l2_latency_clk     500" in text and "l2_to_mem_latency_clk    1400" in text
    for n in names:
        assert "collect_profiles.sh" in (prof / n).read_text()


def test_workload_kernels_name_kernels_of_the_library():
    # every kernel name the per-workload figures look for is the demangled
    # name of a kernel the built library holds (a renamed template would
    # otherwise drop its workload from the summaries without an error)
    import subprocess

    import paged_kv_attention_kvcache_amd as pkv

    if not os.path.exists(pkv.LIB_PATH):
        pytest.skip("library not built")
    out = subprocess.run(["nm", "-C", "--defined-only", pkv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    kernels = [ln.split(" ", 2)[2] for ln in out.splitlines()
               if " V void pkv::" in ln and "__device_stub__" not in ln]
    assert kernels
    for wl, ks in rs.WORKLOAD_KERNELS.items():
        for substr, _ in ks:
            assert any(substr in k for k in kernels), (wl, substr)
