"""Host-side rules of bench.py (no GPU): it measures one GPU and refuses
more with a message, and the roofline's counter-measured traffic is reported
only while the decode kernels' sources match the ones the counters were
taken on."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_profiles_follow_the_source_hash(monkeypatch):
    from paged_kv_attention_kvcache_amd import rocprof_summary

    path = os.path.join(ROOT, "profiles", "kernels.json")
    if os.path.exists(path):
        stored = json.load(open(path))
        if stored["kernel_source_hash"] == rocprof_summary.kernel_source_hash():
            assert bench.profile_for("ouro") == stored["workloads"]["ouro"]
    monkeypatch.setattr(rocprof_summary, "kernel_source_hash", lambda: "0" * 16)
    assert bench.profile_for("ouro") is None
    assert bench.profile_for("no_such_workload") is None


def test_roofline_prices_the_call_both_ways(monkeypatch):
    # 340 MB per call in 58 us live; the committed profile says 59 us and
    # 343 MB of counter-measured HBM traffic
    monkeypatch.setattr(bench, "profile_for", lambda w: {"us_per_call": 59.0,
                                                         "hbm_bytes_per_call": 343_000_000})
    r = bench.roofline("ouro", "k", 340e6 / 58e-6 / 1e9, 8000.0, "GB/s", "hbm", 340e6, 58e-6)
    assert r["frac"] == round(340e6 / 58e-6 / 1e9 / 8000.0, 4)
    assert r["traffic"] == 343_000_000 and r["profiled_us_per_call"] == 59.0
    assert r["achieved_profiled"] == round(340e6 / 59e-6 / 1e9, 2)
    assert r["hip_event_us_per_call"] == 58.0
    monkeypatch.setattr(bench, "profile_for", lambda w: None)
    r = bench.roofline("ouro", "k", 1.0, 8000.0, "GB/s", "hbm", 1.0, 1.0)
    assert r["traffic"] is None and "achieved_profiled" not in r


def test_workload_configs_name_the_shapes():
    for name in ("ouro", "huginn", "longctx"):
        cfg = bench.CONFIG_TEXT[name]
        assert cfg["workload"] and cfg["page_size"] == 16 and cfg["head_dim"] == 128


def test_kernel_labels_follow_the_split():
    # the label bench.py reports for each split, from an object holding only
    # the sizes kernel_for reads (no pool, no GPU)
    wl = bench.DecodeWorkload.__new__(bench.DecodeWorkload)
    wl.hq, wl.hkv, wl.D, wl.batch, wl.max_seq = 64, 8, 128, 256, 32768
    assert wl.kernel_for("balanced", 0).startswith("decode_stream<BF16, MfmaFold<8>>")
    assert wl.kernel_for("fixed", 512).startswith("decode_parts<BF16, MfmaFold<8>>")
    assert wl.kernel_for("fixed", 48).startswith("decode_block<BF16, MfmaFold<8>>")
    wl.hq = 16
    assert wl.kernel_for("fixed", 48).startswith("decode_parts<BF16, ValuFold<BF16, 128, 2>>")
    assert wl.kernel_for("whole", 0).startswith("decode_whole<")
