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
        divided by the counter's reading).
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


# Sources the decode kernels are built from (the counter readings stored
# for the decode workloads stay valid while these are unchanged).
NOT_DECODE = ("prefill.hip", "prefill_mfma.hip", "prefill_cols.hip", "kv_write.hip")


def kernel_source_hash() -> str:
    """Hash of the decode kernels' sources (.hip, .hpp), to tie counter
    readings to the kernels they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")) and name not in NOT_DECODE:
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


def engine_counters(d: str, kernel: str, simds: int = 1024, clock_hz: float = 2.4e9) -> list[dict]:
    """Per launch shape of the kernels matching `kernel`: the mean of each
    counter per dispatch and what follows from them. SQ_VALU_MFMA_BUSY_CYCLES
    sums matrix-core busy clocks over every SIMD, so mfma_busy = that / (SIMDs
    x dispatch time x the nominal 2.4 GHz engine clock), the fraction of the
    dense MFMA peak the busy time could deliver; l2_hit = TCC_HIT / (TCC_HIT +
    TCC_MISS), summed over the dies' L2 caches."""
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
        out.append(res)
    return out


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
    else:
        res = traffic(args)
        text = json.dumps(res, indent=1)
        print(text)
        if args.json:
            with open(args.json, "w") as fh:
                fh.write(text + "\n")


if __name__ == "__main__":
    sys.exit(main())
