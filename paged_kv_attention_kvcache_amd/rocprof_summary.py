"""Summaries of rocprofv3 CSV output for this library's kernels.

    python -m paged_kv_attention_kvcache_amd.rocprof_summary stats DIR
        per-kernel calls / average / min / max duration from a
        `rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o run` run;
    python -m paged_kv_attention_kvcache_amd.rocprof_summary shapes DIR
        the same per launch shape (kernel, grid size) from the kernel trace of
        such a run, for kernels launched on inputs of several sizes;
    python -m paged_kv_attention_kvcache_amd.rocprof_summary pmc DIR
        per-kernel averages of every counter of a `--pmc` run;
    python -m paged_kv_attention_kvcache_amd.rocprof_summary traffic \\
            --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \\
            --kernel SUBSTR --copy-bytes N [--json OUT]
        HBM bytes per launch of the kernel whose name contains SUBSTR:
        FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by what the same
        counters read for a plain copy of N bytes (bytes read and written,
        divided by the counter's reading);
    python -m paged_kv_attention_kvcache_amd.rocprof_summary workloads \\
            --stats DIR --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \\
            --copy-bytes N --json OUT
        per bench.py workload (WORKLOAD_KERNELS): the average duration of
        each kernel one call launches (kernel trace of a default bench.py
        run), their sum per call, and the HBM bytes per call from the
        counter runs, with the hash of the sources they were taken on;
    python -m paged_kv_attention_kvcache_amd.rocprof_summary write OUT --profiles DIR
        every committed summary, from the runs collect_profiles.sh leaves in OUT.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


# The kernels one call of each bench.py workload launches, as (substring of
# the kernel's name, grid size in threads or None for any): the dominant
# kernel first, then the split-K combine where the split needs one.
WORKLOAD_KERNELS = {
    "ouro": [("decode_whole<pkv::BF16, pkv::ValuFold<pkv::BF16, 128, 2, false>", None)],
    "huginn": [("decode_whole<pkv::BF16, pkv::ValuFold<pkv::BF16, 128, 1, false>", None)],
    "longctx": [("decode_stream<pkv::BF16, pkv::MfmaFold<8, false, false>", None),
                ("decode_stream_combine<pkv::BF16, 8>", None)],
    "longctx_p512": [("decode_parts<pkv::BF16, pkv::MfmaFold<8, false, false>", None),
                     ("decode_parts_combine<pkv::BF16, 8>", None)],
    "prefill_cold2048": [("prefill_mfma", 131072)],
    "prefill_8x2048": [("prefill_mfma", 524288)],
}


def kernel_source_hash() -> str:
    """Hash of the library's sources (.hip, .hpp, .cpp), to tie timings and
    counter readings to the kernels they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".cpp")):
            h.update(name.encode())
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def _one(pattern: str) -> str:
    hits = glob.glob(pattern)
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def short_name(name: str) -> str:
    """Kernel name without the argument list (templates kept)."""
    depth, out = 0, []
    for ch in name:
        if ch == "(" and depth == 0 and out:
            break
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        out.append(ch)
    s = "".join(out).replace("void ", "").strip()
    return s if len(s) < 110 else s[:107] + "..."


def kernel_stats(d: str) -> list[dict]:
    rows = list(csv.DictReader(open(_one(os.path.join(d, "*kernel_stats.csv")))))
    out = []
    for r in rows:
        out.append({"name": short_name(r["Name"]), "calls": int(r["Calls"]),
                    "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                    "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    return out


def shape_stats(d: str) -> list[dict]:
    """Calls / average / min / max duration per (kernel, grid size)."""
    rows = csv.DictReader(open(_one(os.path.join(d, "*kernel_trace.csv"))))
    acc = collections.defaultdict(list)
    for r in rows:
        grid = (int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        acc[(short_name(r["Kernel_Name"]), grid)].append(dur)
    out = []
    for (name, grid), ds in sorted(acc.items()):
        out.append({"name": name, "grid": grid, "calls": len(ds), "avg_us": sum(ds) / len(ds),
                    "min_us": min(ds), "max_us": max(ds)})
    return out


def pmc_averages(d: str) -> dict:
    """{kernel short name: {counter: mean over dispatches}}."""
    rows = csv.DictReader(open(_one(os.path.join(d, "*counter_collection.csv"))))
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in rows:
        acc[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def _pick(avgs: dict, substr: str, counter: str) -> float:
    hits = [v[counter] for k, v in avgs.items() if substr in k and counter in v]
    if not hits:
        raise SystemExit(f"no kernel matching {substr!r} with {counter}")
    return max(hits)


def traffic(args) -> dict:
    cf = pmc_averages(args.copy_fetch)
    cw = pmc_averages(args.copy_write)
    # the copy probe's kernel is the one reading the most bytes
    copy_fetch = max(v.get("FETCH_SIZE", 0.0) for v in cf.values())
    copy_write = max(v.get("WRITE_SIZE", 0.0) for v in cw.values())
    fetch_scale = args.copy_bytes / (copy_fetch * 1024.0)
    write_scale = args.copy_bytes / (copy_write * 1024.0)
    f = _pick(pmc_averages(args.fetch), args.kernel, "FETCH_SIZE")
    w = _pick(pmc_averages(args.write), args.kernel, "WRITE_SIZE")
    res = {"kernel": args.kernel, "fetch_kib_raw": f, "write_kib_raw": w,
           "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
           "hbm_read_bytes_per_launch": round(f * 1024 * fetch_scale),
           "hbm_write_bytes_per_launch": round(w * 1024 * write_scale),
           "hbm_bytes_per_launch": round(f * 1024 * fetch_scale + w * 1024 * write_scale),
           "kernel_source_hash": kernel_source_hash()}
    return res


def pmc_by_shape(d: str) -> dict:
    """{(kernel short name, grid size): {counter: mean over dispatches}}."""
    rows = csv.DictReader(open(_one(os.path.join(d, "*counter_collection.csv"))))
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in rows:
        key = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]))
        acc[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def _match(name: str, grid: int, substr: str, want_grid) -> bool:
    return substr in name and (want_grid is None or grid == want_grid)


def workloads(stats_dir, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir,
              copy_bytes: float) -> dict:
    """Per workload of WORKLOAD_KERNELS: kernel averages from a kernel trace
    and HBM bytes per call from FETCH_SIZE / WRITE_SIZE runs, scaled by the
    counters' reading for a plain copy of copy_bytes bytes."""
    shapes = shape_stats(stats_dir)
    cf = pmc_averages(copy_fetch_dir)
    cw = pmc_averages(copy_write_dir)
    fetch_scale = copy_bytes / (max(v.get("FETCH_SIZE", 0.0) for v in cf.values()) * 1024.0)
    write_scale = copy_bytes / (max(v.get("WRITE_SIZE", 0.0) for v in cw.values()) * 1024.0)
    fetch = pmc_by_shape(fetch_dir)
    write = pmc_by_shape(write_dir)
    out = {"kernel_source_hash": kernel_source_hash(), "fetch_scale": round(fetch_scale, 4),
           "write_scale": round(write_scale, 4), "workloads": {}}
    for wl, kernels in WORKLOAD_KERNELS.items():
        ks, total_us, read_b, write_b, ok = [], 0.0, 0.0, 0.0, True
        for substr, grid in kernels:
            hits = [r for r in shapes if _match(r["name"], r["grid"][0], substr, grid)]
            if not hits:
                ok = False
                break
            calls = sum(r["calls"] for r in hits)
            avg = sum(r["avg_us"] * r["calls"] for r in hits) / calls
            f = [v["FETCH_SIZE"] for (n, g), v in fetch.items()
                 if _match(n, g, substr, grid) and "FETCH_SIZE" in v]
            w = [v["WRITE_SIZE"] for (n, g), v in write.items()
                 if _match(n, g, substr, grid) and "WRITE_SIZE" in v]
            rb = max(f) * 1024 * fetch_scale if f else None
            wb = max(w) * 1024 * write_scale if w else None
            ks.append({"kernel": hits[0]["name"], "grid": hits[0]["grid"][0], "calls": calls,
                       "avg_us": round(avg, 3), "hbm_read_bytes": None if rb is None else round(rb),
                       "hbm_write_bytes": None if wb is None else round(wb)})
            total_us += avg
            if rb is None or wb is None:
                read_b = write_b = None
            elif read_b is not None:
                read_b += rb
                write_b += wb
        if not ok:
            continue
        out["workloads"][wl] = {
            "kernels": ks, "us_per_call": round(total_us, 3),
            "hbm_bytes_per_call": None if read_b is None else round(read_b + write_b)}
    return out


def engine_counters(d: str, kernel: str, simds: int = 1024, clock_hz: float = 2.4e9,
                    cus: int = 256) -> list[dict]:
    """Per launch shape of the kernels matching `kernel`: the mean of each
    counter per dispatch and what follows from them. SQ_VALU_MFMA_BUSY_CYCLES
    sums matrix-core busy clocks over every SIMD, so mfma_busy = that / (SIMDs
    x dispatch time x the nominal 2.4 GHz engine clock), the fraction of the
    dense MFMA peak the busy time could deliver; l2_hit = TCC_HIT / (TCC_HIT +
    TCC_MISS), summed over the dies' L2 caches. With SQ_BUSY_CU_CYCLES (the
    busy cycles of the CUs, summed): clock_ghz = those of one CU / time (the
    engine clock, while every CU is busy for the whole dispatch);
    mfma_busy_at_clock = the matrix-core busy fraction at that clock;
    lds_read_B_per_clk_cu = SQ_INSTS_LDS_LOAD_BANDWIDTH (64-byte units) per
    CU-cycle; lds_active = SQ_LDS_IDX_ACTIVE per CU-cycle; wave_wait_frac =
    SQ_WAIT_ANY / SQ_WAVE_CYCLES."""
    rows = csv.DictReader(open(_one(os.path.join(d, "*counter_collection.csv"))))
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for r in rows:
        if kernel not in r["Kernel_Name"]:
            continue
        key = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]))
        acc[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
        dur[key][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    out = []
    for key, cs in sorted(acc.items()):
        m = {c: sum(v) / len(v) for c, v in cs.items()}
        t = sum(dur[key].values()) / len(dur[key])
        res = {"kernel": key[0], "grid": key[1], "dispatches": len(dur[key]), "us": t * 1e6, **m}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            res["mfma_busy"] = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * clock_hz * t)
        if m.get("TCC_HIT_sum", 0) + m.get("TCC_MISS_sum", 0) > 0:
            res["l2_hit"] = m["TCC_HIT_sum"] / (m["TCC_HIT_sum"] + m["TCC_MISS_sum"])
        if "SQ_INSTS_VALU" in m and m.get("SQ_INSTS_MFMA"):
            res["valu_per_mfma"] = m["SQ_INSTS_VALU"] / m["SQ_INSTS_MFMA"]
        busy = m.get("SQ_BUSY_CU_CYCLES", 0.0)
        if busy > 0:
            cu_cycles = busy / cus  # one CU's busy cycles
            res["clock_ghz"] = cu_cycles / t / 1e9
            if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                res["mfma_busy_at_clock"] = m["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / cu_cycles
            if "SQ_INSTS_LDS_LOAD_BANDWIDTH" in m:
                res["lds_read_B_per_clk_cu"] = m["SQ_INSTS_LDS_LOAD_BANDWIDTH"] * 64 / busy
            if "SQ_LDS_IDX_ACTIVE" in m:
                res["lds_active"] = m["SQ_LDS_IDX_ACTIVE"] / busy
        if m.get("SQ_WAVE_CYCLES") and "SQ_WAIT_ANY" in m:
            res["wave_wait_frac"] = m["SQ_WAIT_ANY"] / m["SQ_WAVE_CYCLES"]
        out.append(res)
    return out


COLLECT = "bash paged_kv_attention_kvcache_amd/collect_profiles.sh OUT"
PIPELINE_COUNTERS = ("SQ_BUSY_CU_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES "
                     "SQ_ACTIVE_INST_VALU SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS_LOAD_BANDWIDTH "
                     "SQ_WAIT_ANY SQ_WAVE_CYCLES")


def _stats_text(d: str) -> str:
    lines = [f"{'kernel':110s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} "
             f"{'%':>6s}"]
    for r in kernel_stats(d):
        if "pkv::" in r["name"]:
            lines.append(f"{r['name']:110s} {r['calls']:6d} {r['avg_us']:10.2f} "
                         f"{r['min_us']:10.2f} {r['max_us']:10.2f} {r['pct']:6.2f}")
    return "\n".join(lines) + "\n"


def _shapes_text(d: str) -> str:
    lines = [f"{'kernel':80s} {'grid (threads)':>15s} {'calls':>6s} {'avg_us':>10s} "
             f"{'min_us':>10s} {'max_us':>10s}"]
    for r in shape_stats(d):
        if "pkv::" in r["name"]:
            lines.append(f"{r['name'][:80]:80s} {r['grid'][0]:15d} {r['calls']:6d} "
                         f"{r['avg_us']:10.2f} {r['min_us']:10.2f} {r['max_us']:10.2f}")
    return "\n".join(lines) + "\n"


def write_profiles(out: str, profiles: str) -> None:
    """The committed summaries, from the runs of collect_profiles.sh in out."""
    j = lambda name: os.path.join(out, name)
    os.makedirs(profiles, exist_ok=True)
    res = workloads(j("stats_default"), j("all_fetch"), j("all_write"), j("copy_fetch"),
                    j("copy_write"), float(1 << 30))
    res["produced_by"] = COLLECT
    with open(os.path.join(profiles, "kernels.json"), "w") as fh:
        fh.write(json.dumps(res, indent=1) + "\n")
    h = res["kernel_source_hash"]
    hdr = f"""# rocprofv3 kernel statistics of the default benchmark (python3 bench.py: the Ouro
# headline step, then every other workload under "configs"), library sources {h}.
# Produced from the repository root by {COLLECT}, whose run is
#   rocprofv3 --kernel-trace --stats --output-format csv -d OUT/stats_default -o run -- python3 bench.py
# and summarised with
#   python -m paged_kv_attention_kvcache_amd.rocprof_summary stats OUT/stats_default
#   python -m paged_kv_attention_kvcache_amd.rocprof_summary shapes OUT/stats_default
# Durations in microseconds; % = share of all GPU kernel time in the run (the rest is
# the seeded input generation, done before each timed region).
# Per kernel:
"""
    with open(os.path.join(profiles, "bench_default_kernel_stats.txt"), "w") as fh:
        fh.write(hdr + _stats_text(j("stats_default")) +
                 "\n# Per launch shape (grid in threads):\n" + _shapes_text(j("stats_default")))
    hdr = f"""# HBM traffic and kernel time per call of each benchmark workload, library sources {h}.
# Produced from the repository root by {COLLECT}, whose runs are
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/copy_fetch -o run -- python3 bench.py --probe copy
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/copy_write -o run -- python3 bench.py --probe copy
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/all_fetch -o run -- python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/all_write -o run -- python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline
# plus the kernel trace of bench_default_kernel_stats.txt, summarised with
#   python -m paged_kv_attention_kvcache_amd.rocprof_summary workloads --stats OUT/stats_default --fetch OUT/all_fetch --write OUT/all_write --copy-fetch OUT/copy_fetch --copy-write OUT/copy_write --copy-bytes 1073741824 --json profiles/kernels.json
# FETCH_SIZE and WRITE_SIZE are KiB per dispatch; the plain copy of 1 GiB (1 GiB read and
# written) reads fetch x {res['fetch_scale']} and write x {res['write_scale']}, the factors applied here.
"""
    lines = []
    for wl, r in res["workloads"].items():
        lines.append(f"{wl}: {r['us_per_call']:.2f} us per call, HBM bytes per call "
                     f"{r['hbm_bytes_per_call']}")
        for k in r["kernels"]:
            lines.append(f"    {k['kernel']}  grid {k['grid']}  calls {k['calls']}  avg_us "
                         f"{k['avg_us']:.2f}  read {k['hbm_read_bytes']}  write "
                         f"{k['hbm_write_bytes']}")
    with open(os.path.join(profiles, "hbm_traffic.txt"), "w") as fh:
        fh.write(hdr + "\n".join(lines) + "\n")
    counters = ("GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA "
                "SQ_INSTS_LDS SQ_WAIT_INST_ANY SQ_WAVE_CYCLES SQ_BUSY_CYCLES")
    hdr = f"""# rocprofv3 engine counters of the prefill kernels per launch shape (grid in threads, 256
# per workgroup), library sources {h}. Produced from the repository root by {COLLECT}:
#   rocprofv3 --pmc {counters} --output-format csv -d OUT/prefill_engine -o run -- python3 bench.py --prefill-only --no-cpu-baseline
#   python -m paged_kv_attention_kvcache_amd.rocprof_summary engine OUT/prefill_engine --kernel prefill
# us: mean dispatch time under counter collection; mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES /
# (1024 SIMDs x 2.4 GHz x time); valu_per_mfma = SQ_INSTS_VALU / SQ_INSTS_MFMA.
"""
    body = []
    for r in engine_counters(j("prefill_engine"), "prefill"):
        body.append(f"{r['kernel']}  grid {r['grid']}  ({r['dispatches']} dispatches)")
        for k, v in r.items():
            if k not in ("kernel", "grid", "dispatches"):
                body.append(f"    {k:28s} {v:.6g}")
    body.append(f"""
# Second pass, what the step's pipeline waits on:
#   rocprofv3 --pmc {PIPELINE_COUNTERS} --output-format csv -d OUT/prefill_pipeline -o run -- python3 bench.py --prefill-only --no-cpu-baseline
# clock_ghz = SQ_BUSY_CU_CYCLES / 256 CUs / time; mfma_busy_at_clock = SQ_VALU_MFMA_BUSY_CYCLES /
# 1024 SIMDs / the CU cycles; lds_read_B_per_clk_cu = SQ_INSTS_LDS_LOAD_BANDWIDTH x 64 B per
# CU-cycle (it matches the kernel's 32 KiB of LDS reads per wave-step to within 2%);
# lds_active = SQ_LDS_IDX_ACTIVE per CU-cycle; wave_wait_frac = SQ_WAIT_ANY / SQ_WAVE_CYCLES.""")
    if os.path.isdir(j("prefill_pipeline")):
        for r in engine_counters(j("prefill_pipeline"), "prefill"):
            body.append(f"{r['kernel']}  grid {r['grid']}  ({r['dispatches']} dispatches)")
            for k, v in r.items():
                if k not in ("kernel", "grid", "dispatches"):
                    body.append(f"    {k:28s} {v:.6g}")
    with open(os.path.join(profiles, "prefill_engine_counters.txt"), "w") as fh:
        fh.write(hdr + "\n".join(body) + "\n")
    hdr = f"""# L2 hit rates per kernel and launch shape, library sources {h}: TCC_HIT / (TCC_HIT +
# TCC_MISS) over the dies' L2 caches. Produced from the repository root by {COLLECT}:
#   rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum --output-format csv -d OUT/all_l2 -o run -- python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline
#   python -m paged_kv_attention_kvcache_amd.rocprof_summary engine OUT/all_l2 --kernel pkv::
"""
    body = [f"{r['kernel'][:80]:80s} grid {r['grid']:9d}  dispatches {r['dispatches']:5d}  "
            f"l2_hit {r.get('l2_hit', float('nan')):.3f}"
            for r in engine_counters(j("all_l2"), "pkv::")]
    with open(os.path.join(profiles, "l2_hit_rates.txt"), "w") as fh:
        fh.write(hdr + "\n".join(body) + "\n")
    hdr = f"""# Memory-pipeline counters of the decode kernels per launch shape, library sources {h}.
# Produced from the repository root by {COLLECT}, whose runs are (one counter set each)
#   rocprofv3 --pmc TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum TCP_UTCL1_TRANSLATION_MISS_sum TCP_UTCL1_REQUEST_sum --output-format csv -d OUT/decode_tcp -o run -- python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-prefill
#   rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_LEVEL_sum --output-format csv -d OUT/decode_tcc -o run -- (the same)
#   rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_VMEM_RD SQ_INST_LEVEL_VMEM SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_BUSY_CYCLES SQ_WAVES --output-format csv -d OUT/decode_sq -o run -- (the same)
# l1_to_l2_latency_clk = TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ (average clocks from an L1
# miss to its L2 data); l2_to_mem_latency_clk = TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ (average
# clocks an L2 read to the memory side is outstanding); counts are per dispatch. Kernel names
# separate the workloads: ValuFold<BF16, 128, 2> is the Ouro shape, ValuFold<BF16, 128, 1> the
# Huginn shape, MfmaFold<8> the long-context shape (balanced split and fixed partitions).
"""
    body = []
    for d in decode_memory(out):
        body.append(f"{d['kernel']}  grid {d['grid']}")
        for k, v in d.items():
            if k not in ("kernel", "grid") and v is not None:
                body.append(f"    {k:24s} {v:.6g}")
    with open(os.path.join(profiles, "decode_memory_counters.txt"), "w") as fh:
        fh.write(hdr + "\n".join(body) + "\n")


def decode_memory(out: str) -> list[dict]:
    """Per decode kernel and launch shape, from the decode_tcp / decode_tcc /
    decode_sq runs: the average L1->L2 read latency (TCP_TCC_READ_REQ_LATENCY
    / TCP_TCC_READ_REQ, clocks), the average L2->memory read latency
    (TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ, clocks), the L2 hit rate, TLB
    misses per dispatch, and VALU and vector-load instructions per dispatch."""
    rows = {}
    for run in ("decode_tcp", "decode_tcc", "decode_sq"):
        for r in engine_counters(os.path.join(out, run), "decode"):
            rows.setdefault((r["kernel"], r["grid"]), {}).update(r)
    res = []
    for (k, g), r in sorted(rows.items()):
        d = {"kernel": k, "grid": g, "us": r.get("us")}
        if r.get("TCP_TCC_READ_REQ_sum"):
            d["l1_to_l2_latency_clk"] = r["TCP_TCC_READ_REQ_LATENCY_sum"] / r["TCP_TCC_READ_REQ_sum"]
            d["l2_read_requests"] = r["TCP_TCC_READ_REQ_sum"]
        if "TCP_UTCL1_TRANSLATION_MISS_sum" in r:
            d["tlb_misses"] = r["TCP_UTCL1_TRANSLATION_MISS_sum"]
        if r.get("TCC_EA0_RDREQ_sum"):
            d["l2_to_mem_latency_clk"] = r["TCC_EA0_RDREQ_LEVEL_sum"] / r["TCC_EA0_RDREQ_sum"]
        if "l2_hit" in r:
            d["l2_hit"] = r["l2_hit"]
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
                  "SQ_WAVE_CYCLES", "SQ_WAVES"):
            if c in r:
                d[c] = r[c]
        res.append(d)
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--all", action="store_true", help="include kernels of other libraries")
    sh = sub.add_parser("shapes")
    sh.add_argument("dir")
    p = sub.add_parser("pmc")
    p.add_argument("dir")
    e = sub.add_parser("engine")
    e.add_argument("dir")
    e.add_argument("--kernel", required=True)
    t = sub.add_parser("traffic")
    for k in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--kernel"):
        t.add_argument(k, required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--json", default=None)
    w = sub.add_parser("workloads")
    for k in ("--stats", "--fetch", "--write", "--copy-fetch", "--copy-write", "--json"):
        w.add_argument(k, required=True)
    w.add_argument("--copy-bytes", type=float, required=True)
    wr = sub.add_parser("write")
    wr.add_argument("out")
    wr.add_argument("--profiles", required=True)
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print(f"{'kernel':110s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'%':>6s}")
        for r in kernel_stats(args.dir):
            if args.all or "pkv::" in r["name"]:
                print(f"{r['name']:110s} {r['calls']:6d} {r['avg_us']:10.2f} {r['min_us']:10.2f} "
                      f"{r['max_us']:10.2f} {r['pct']:6.2f}")
    elif args.cmd == "shapes":
        print(f"{'kernel':60s} {'grid (threads)':>22s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} "
              f"{'max_us':>10s}")
        for r in shape_stats(args.dir):
            if "pkv::" in r["name"]:
                g = "x".join(str(v) for v in r["grid"])
                print(f"{r['name'][:60]:60s} {g:>22s} {r['calls']:6d} {r['avg_us']:10.2f} "
                      f"{r['min_us']:10.2f} {r['max_us']:10.2f}")
    elif args.cmd == "pmc":
        for k, cs in pmc_averages(args.dir).items():
            print(k)
            for c, v in sorted(cs.items()):
                print(f"    {c:40s} {v:.6g}")
    elif args.cmd == "engine":
        for r in engine_counters(args.dir, args.kernel):
            print(f"{r['kernel']}  grid {r['grid']}  ({r['dispatches']} dispatches)")
            for k, v in r.items():
                if k not in ("kernel", "grid", "dispatches"):
                    print(f"    {k:28s} {v:.6g}")
    elif args.cmd == "write":
        write_profiles(args.out, args.profiles)
    elif args.cmd == "workloads":
        res = workloads(args.stats, args.fetch, args.write, args.copy_fetch, args.copy_write,
                        args.copy_bytes)
        text = json.dumps(res, indent=1)
        print(text)
        with open(args.json, "w") as fh:
            fh.write(text + "\n")
    else:
        res = traffic(args)
        text = json.dumps(res, indent=1)
        print(text)
        if args.json:
            with open(args.json, "w") as fh:
                fh.write(text + "\n")


if __name__ == "__main__":
    sys.exit(main())
