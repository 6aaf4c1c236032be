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


def test_traffic_follows_the_source_hash(monkeypatch):
    stored = json.load(open(os.path.join(ROOT, "profiles", "traffic_ouro.json")))
    from paged_kv_attention_kvcache_amd import rocprof_summary

    if stored["kernel_source_hash"] == rocprof_summary.kernel_source_hash():
        assert bench.traffic_from_profiles("ouro") == stored["hbm_bytes_per_launch"]
    monkeypatch.setattr(rocprof_summary, "kernel_source_hash", lambda: "0" * 16)
    assert bench.traffic_from_profiles("ouro") is None
    assert bench.traffic_from_profiles("no_such_workload") is None


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
