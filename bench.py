#!/usr/bin/env python3
"""Benchmark of the paged-KV attention hot path on one MI355X.

A step is one decode step of a looped model through every (plane, layer) bank
in model order: for each bank, store_kv writes each request's newest token and
decode attention reads the whole context through the page table. By default
both happen in one call (paged_decode_append_attn); --separate-write issues
paged_kv_write then paged_decode_attn instead (same results, bit for bit).

The headline (the top-level value, ms_per_step, roofline and cpu_baseline) is
the Ouro-style fixed-depth step: 24 layers x 4 loop planes = 96 banks, batch
64, seq_lens uniform in [512, 2048], page size 16, 16 query / 8 KV heads,
head_dim 128, bf16, pages randomly permuted. The same run measures every
other workload under "configs", each with the roofline of its dominant kernel
and the fp64 oracle timed on a stated sample:
  tiny_decode                     fp32, 4 requests of 17-64 tokens (launch-bound)
  huginn_recurrent_depth_decode   132 packed banks, MHA 32 heads, 78% aliased
                                  prompt pages (logical and unique bytes)
  cached_prefix_prefill           8 x 512-token prompts: cold chunk 2048,
                                  cold chunk 128, 16-token suffix over 496
  long_context_decode             batch 256, 8k-32k contexts, GQA 8: the
                                  library's balanced split and the stated
                                  fixed 512-token partitions
  prefill_8x2048                  8 cold 2048-token prompts in one chunk
--workload huginn|longctx times one of the decode workloads alone (its own
headline line), --prefill-only the prefill cases alone.

`value` is logical KV bytes read by decode attention per second over the
whole step (write + attention for every bank), with all inputs resident in
HBM before the timed region starts.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "paged decode attention KV GB/s (% of HBM peak); prefill TFLOP/s (% MFMA)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def profile_for(workload: str):
    """The committed rocprofv3 figures of one workload (profiles/kernels.json):
    {"us_per_call": summed kernel averages of one call, "hbm_bytes_per_call":
    counter-measured HBM bytes, "kernels": [...]}, or None when they were
    taken on other sources than the ones built here."""
    from paged_kv_attention_kvcache_amd.rocprof_summary import kernel_source_hash

    path = os.path.join(ROOT, "profiles", "kernels.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("workloads", {}).get(workload)


def roofline(workload: str, kernel: str, achieved: float, peak: float, unit: str,
             bound: str, per_call: float, call_s: float, **extra) -> dict:
    """The roofline object of a workload's dominant kernel: `achieved` from
    the live HIP-event time of one call (per_call algorithmic bytes or flops /
    call_s); beside it the same call priced with the committed rocprofv3
    kernel averages, and the counter-measured HBM traffic, when those were
    taken on these sources."""
    prof = profile_for(workload)
    r = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4),
         "traffic": prof.get("hbm_bytes_per_call") if prof else None,
         "kernel": kernel, "hip_event_us_per_call": round(call_s * 1e6, 3)}
    if prof:
        us = prof["us_per_call"]
        scale = 1e9 if unit == "GB/s" else 1e12
        r["profiled_us_per_call"] = us
        r["achieved_profiled"] = round(per_call / (us * 1e-6) / scale, 2)
        r["frac_profiled"] = round(per_call / (us * 1e-6) / scale / peak, 4)
    r.update(extra)
    return r


# --------------------------------------------------------------------------- workloads

class DecodeWorkload:
    """A multi-plane pool and one decode step's inputs, all on the device."""

    def __init__(self, name, batch, seq_range, hq, hkv, D, planes, layers, rec_first,
                 rec_count, order, alias=0.0, partition=0, seed=0, snapshot_banks=0,
                 snapshot_rows=0):
        import torch

        import paged_kv_attention_kvcache_amd as pkv
        from paged_kv_attention_kvcache_amd import synth

        self.name, self.hq, self.hkv, self.D, self.batch = name, hq, hkv, D, batch
        self.partition = partition  # 0: the library's balanced split
        rng = np.random.default_rng(seed)
        if alias > 0:
            prompts = rng.integers(seq_range[0], seq_range[1] + 1, size=batch)
            self.seq = (prompts + 1).astype(np.int32)
            shared = synth.alias_pages(prompts, alias, 16)
        else:
            self.seq = rng.integers(seq_range[0], seq_range[1] + 1, size=batch).astype(np.int32)
            shared = None
        self.table, self.num_pages, _ = synth.allocate_pages(rng, self.seq, 16,
                                                             shared_pages=shared)
        self.shared = shared
        self.bank_of, self.nb = pkv.bank_map(planes, layers, rec_first, rec_count)
        self.order = order  # [(plane, layer)] in model order
        shape = (self.nb, self.num_pages, hkv, 16, D)
        gb = 2 * np.prod(shape) * 2 / 1e9
        log(f"[{name}] pool: {self.nb} banks x {self.num_pages} pages = {gb:.1f} GB")
        k = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        v = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        synth.device_normal_(k, seed + 1)
        synth.device_normal_(v, seed + 2)
        self.pool = pkv.Pool(torch.bfloat16, self.num_pages, hkv, D, self.bank_of, self.nb,
                             k=k, v=v)
        nbk = len(order)
        self.q = synth.device_normal_(torch.empty((nbk, batch, hq, D), dtype=torch.bfloat16,
                                                  device="cuda"), seed + 3)
        self.nk = synth.device_normal_(torch.empty((nbk, batch, hkv, D), dtype=torch.bfloat16,
                                                   device="cuda"), seed + 4)
        self.nv = synth.device_normal_(torch.empty((nbk, batch, hkv, D), dtype=torch.bfloat16,
                                                   device="cuda"), seed + 5)
        self.slots = torch.from_numpy(synth.slots_of_last(self.table, self.seq, 16)).cuda()
        self.table_d = torch.from_numpy(self.table).cuda()
        self.seq_d = torch.from_numpy(self.seq).cuda()
        self.max_seq = int(self.seq.max())
        self.out = torch.empty((batch, hq, D), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((batch, hq), dtype=torch.float32, device="cuda")
        wsb = pkv.workspace_bytes(self.pool, batch, hq, self.max_seq, self.partition)
        self.ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
        self.pkv = pkv
        self.separate_write = False
        self.split = pkv.split_mode(self.pool, batch, hq, self.max_seq, self.partition)
        self.kernel_name = self.kernel_for(self.split, self.partition)
        # algorithmic bytes: each request reads its whole context (K and V)
        self.kv_bytes_per_call = int(self.seq.astype(np.int64).sum()) * 2 * hkv * D * 2
        uniq_pages = len(np.unique(np.concatenate(
            [self.table[r, :-(-int(n) // 16)] for r, n in enumerate(self.seq)])))
        self.unique_bytes_per_call = uniq_pages * 2 * hkv * 16 * D * 2
        torch.cuda.synchronize()
        # Host copies for the CPU baseline, taken before any library kernel runs:
        # whole banks of the first calls of the step, or the pages of the first
        # snapshot_rows requests of the first call's bank (renumbered).
        hb = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        self.snap = []
        for i in range(min(snapshot_banks, len(order))):
            b = int(self.bank_of[order[i]])
            self.snap.append((hb(k[b])[None], hb(v[b])[None], hb(self.q[i]), self.table,
                              self.seq, self.kv_bytes_per_call))
        if snapshot_rows:
            rows = np.arange(min(snapshot_rows, batch))
            b = int(self.bank_of[order[0]])
            need = [self.table[r, :-(-int(self.seq[r]) // 16)] for r in rows]
            uniq = np.unique(np.concatenate(need))
            remap = np.zeros(self.num_pages, np.int32)
            remap[uniq] = np.arange(len(uniq), dtype=np.int32)
            idx = torch.from_numpy(uniq.astype(np.int64)).cuda()
            table = np.zeros((len(rows), self.table.shape[1]), np.int32)
            for i, r in enumerate(rows):
                table[i, :len(need[i])] = remap[need[i]]
            seq = self.seq[rows]
            self.snap.append((hb(k[b].index_select(0, idx))[None],
                              hb(v[b].index_select(0, idx))[None], hb(self.q[0][rows]), table,
                              seq, int(seq.astype(np.int64).sum()) * 2 * hkv * D * 2))

    def kernel_for(self, split, partition):
        """The decode kernels a call of this workload launches."""
        g = self.hq // self.hkv
        mfma = g in (4, 8) and self.D == 128
        fold = f"MfmaFold<{g}>" if mfma else f"ValuFold<BF16, {self.D}, {g}>"
        if split == "whole":
            return f"decode_whole<BF16, {fold}> (persistent, one launch per call)"
        if split == "balanced":
            return f"decode_stream<BF16, {fold}> + decode_stream_combine"
        pp = (partition or 512) // 16  # pages per partition (512 tokens by default)
        parts = -(-self.max_seq // (partition or 512))
        if parts > 1 and self.batch <= 4096 and pp % (2 if mfma else 1) == 0:
            return f"decode_parts<BF16, {fold}> (persistent) + decode_parts_combine"
        return f"decode_block<BF16, {fold}> + decode_reduce"

    def time_fixed_partitions(self, partition, steps, stream):
        """Decode calls (no fused append) on fixed partitions of `partition`
        tokens and the in-order reduction, back to back between two events."""
        import torch

        pkv = self.pkv
        wsb = pkv.workspace_bytes(self.pool, self.batch, self.hq, self.max_seq, partition)
        ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
        plane, layer = self.order[0]

        def call():
            pkv.decode(self.pool, plane, layer, self.q[0], self.table_d, self.seq_d,
                       self.max_seq, partition=partition, out=self.out, lse=self.lse,
                       workspace=ws)

        call()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        sec = a.elapsed_time(b) / 1e3 / steps
        gbs = self.kv_bytes_per_call / sec / 1e9
        return {"partition": partition, "us_per_call": round(sec * 1e6, 2),
                "kv_GBps": round(gbs, 2), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                "kernel": self.kernel_for("fixed", partition),
                "how": "paged_decode_attn alone (no fused append), back to back"}

    def use_exit_depths(self, lo, hi, seed=7):
        """Early exit: every context token halted at a depth drawn uniformly
        from [lo, hi]; recurrent-layer calls then read each token from plane
        min(plane, depth) (paged_decode_latest_attn)."""
        import torch

        rng = np.random.default_rng(seed)
        stride = (self.max_seq + 15) // 16 * 16
        depth = rng.integers(lo, hi + 1, size=(self.batch, stride)).astype(np.int8)
        self.exit_depth = torch.from_numpy(depth).cuda()

    def call(self, i, decode_only=False):
        plane, layer = self.order[i]
        pkv = self.pkv
        if getattr(self, "exit_depth", None) is not None and plane > 0:
            pkv.decode_latest(self.pool, plane, layer, self.exit_depth, self.q[i], self.table_d,
                              self.seq_d, self.max_seq, partition=self.partition, out=self.out,
                              lse=self.lse, workspace=self.ws, k_new=self.nk[i],
                              v_new=self.nv[i])
            return
        if self.separate_write:
            if not decode_only:
                pkv.kv_write(self.pool, plane, layer, self.nk[i], self.nv[i], self.slots)
            extra = {}
        else:
            extra = dict(k_new=self.nk[i], v_new=self.nv[i])
        pkv.decode(self.pool, plane, layer, self.q[i], self.table_d, self.seq_d, self.max_seq,
                   partition=self.partition, out=self.out, lse=self.lse, workspace=self.ws,
                   **extra)

    def step(self):
        for i in range(len(self.order)):
            self.call(i)

    def step_graph(self):
        """The same step (fused calls) captured once as one submission."""
        pkv, nb = self.pkv, len(self.order)
        return pkv.StepGraph(self.pool, self.order, self.q, self.table_d, self.seq_d,
                             self.max_seq, [self.out] * nb, [self.lse] * nb, workspace=self.ws,
                             k_new=self.nk, v_new=self.nv, partition=self.partition)


def make_workload(name, partition, snapshot_banks=0, snapshot_rows=0):
    kw = dict(partition=partition, snapshot_banks=snapshot_banks, snapshot_rows=snapshot_rows)
    if name == "ouro":
        order = [(t, l) for t in range(4) for l in range(24)]
        return DecodeWorkload("ouro", 64, (512, 2048), 16, 8, 128, 4, 24, 0, 24, order, **kw)
    if name == "huginn":
        order = [(0, 0), (0, 1)] + [(t, l) for t in range(32) for l in range(2, 6)] + \
                [(0, 6), (0, 7)]
        return DecodeWorkload("huginn", 16, (200, 2000), 32, 32, 128, 32, 8, 2, 4, order,
                              alias=0.78, **kw)
    if name == "longctx":
        return DecodeWorkload("longctx", 256, (8192, 32768), 64, 8, 128, 1, 1, 0, 1, [(0, 0)],
                              **kw)
    raise SystemExit(f"unknown workload {name}")


CONFIG_TEXT = {
    "ouro": dict(workload="ouro_fixed_depth_decode", batch=64, seq_lens="uniform[512,2048]",
                 planes=4, layers=24, banks=96, q_heads=16, kv_heads=8, head_dim=128,
                 page_size=16),
    "huginn": dict(workload="huginn_recurrent_depth_decode", batch=16,
                   prompts="uniform[200,2000]", planes=32, layers=8, banks=132, q_heads=32,
                   kv_heads=32, head_dim=128, page_size=16, aliased_prompt_pages=0.78),
    "longctx": dict(workload="long_context_decode", batch=256, seq_lens="uniform[8192,32768]",
                    planes=1, layers=1, banks=1, q_heads=64, kv_heads=8, head_dim=128,
                    page_size=16),
}


# --------------------------------------------------------------------------- prefill

class PrefillWorkload:
    """Chunked causal prefill: `prompts` prompts of `n` tokens, 32 MHA heads,
    head_dim 128, bf16, page size 16, written then attended chunk by chunk
    (paged_kv_write + paged_prefill_attn per chunk). Calls rotate over `banks`
    banks of one pool so that each call's K/V come from HBM, not cache."""

    def __init__(self, prompts=8, n=512, heads=32, D=128, banks=132, seed=0):
        import torch

        import paged_kv_attention_kvcache_amd as pkv
        from paged_kv_attention_kvcache_amd import synth

        self.pkv, self.n, self.prompts, self.heads, self.D = pkv, n, prompts, heads, D
        rng = np.random.default_rng(seed)
        lens = np.full(prompts, n, np.int32)
        self.table, self.num_pages, _ = synth.allocate_pages(rng, lens, 16)
        self.bank_of, self.nb = pkv.bank_map(banks, 1)
        shape = (self.nb, self.num_pages, heads, 16, D)
        k = synth.device_normal_(torch.empty(shape, dtype=torch.bfloat16, device="cuda"), seed + 1)
        v = synth.device_normal_(torch.empty(shape, dtype=torch.bfloat16, device="cuda"), seed + 2)
        self.pool = pkv.Pool(torch.bfloat16, self.num_pages, heads, D, self.bank_of, self.nb,
                             k=k, v=v)
        tokens = prompts * n
        self.q = synth.device_normal_(torch.empty((tokens, heads, D), dtype=torch.bfloat16,
                                                  device="cuda"), seed + 3)
        self.kn = synth.device_normal_(torch.empty((tokens, heads, D), dtype=torch.bfloat16,
                                                   device="cuda"), seed + 4)
        self.vn = synth.device_normal_(torch.empty((tokens, heads, D), dtype=torch.bfloat16,
                                                   device="cuda"), seed + 5)
        self.out = torch.empty_like(self.q)
        self.table_d = torch.from_numpy(self.table).cuda()
        self.synth = synth

    def schedule(self, chunk, start=0):
        """Per chunk: (slots, cu_q_lens, seq_lens, first row, rows, visible pairs)."""
        import torch

        out, lo = [], start
        while lo < self.n:
            hi = min(lo + chunk, self.n)
            q_len = hi - lo
            slots = np.concatenate([self.synth.slots_of(self.table, r, np.arange(lo, hi), 16)
                                    for r in range(self.prompts)])
            rows = np.concatenate([r * self.n + np.arange(lo, hi) for r in range(self.prompts)])
            pairs = self.prompts * sum(p + 1 for p in range(lo, hi))
            out.append(dict(start=start, slots=torch.from_numpy(slots).cuda(),
                            rows=torch.from_numpy(rows.astype(np.int64)).cuda(),
                            cu=torch.from_numpy(np.arange(0, self.prompts + 1, dtype=np.int32)
                                                * q_len).cuda(),
                            seq=torch.from_numpy(np.full(self.prompts, hi, np.int32)).cuda(),
                            q_len=q_len, hi=hi, pairs=pairs))
            lo = hi
        for c in out:  # gathered per chunk so the timed calls read packed inputs
            c["q"] = self.q[c["rows"]].contiguous()
            c["k"] = self.kn[c["rows"]].contiguous()
            c["v"] = self.vn[c["rows"]].contiguous()
            c["o"] = torch.empty_like(c["q"])
        return out

    def run(self, chunks, bank, write=True):
        """write=True: paged_kv_write then paged_prefill_attn per chunk; False:
        the attention alone; "extend": paged_extend_attn (one call);
        "store_only": the paged_kv_write calls alone."""
        pkv = self.pkv
        for c in chunks:
            if write == "store_only":
                pkv.kv_write(self.pool, bank, 0, c["k"], c["v"], c["slots"])
                continue
            if write == "extend":
                pkv.extend(self.pool, bank, 0, c["k"], c["v"], c["slots"], c["q"], c["cu"],
                           self.table_d, c["seq"], c["q_len"], c["hi"], out=c["o"],
                           with_lse=False)
                continue
            if write:
                pkv.kv_write(self.pool, bank, 0, c["k"], c["v"], c["slots"])
            pkv.prefill(self.pool, bank, 0, c["q"], c["cu"], self.table_d, c["seq"], c["q_len"],
                        c["hi"], out=c["o"], with_lse=False)


PREFILL_CASES = [
    # (name, prompts, tokens per prompt, chunk, cached prefix tokens)
    ("cold_chunk2048", 8, 512, 2048, 0),
    ("cold_chunk128", 8, 512, 128, 0),
    ("suffix16_over_496", 8, 512, 4096, 496),
]
SUPPLEMENTARY = ("cold_2048x8_chunk2048", 8, 2048, 2048, 0)


def time_prefill_case(wl, chunks, reps):
    """Per call of the case (all its chunks): write-then-attend, the one-call
    extend, the attention alone and the store_kv alone, each over reps rounds
    of the bank rotation, between HIP events on the stream the library
    launches on."""
    import torch

    stream = torch.cuda.current_stream()
    for b in range(2):
        wl.run(chunks, b)
    torch.cuda.synchronize()
    out = {}
    for write in (True, "extend", False, "store_only"):
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nbk = wl.nb
        a.record(stream)
        for i in range(reps * nbk):
            wl.run(chunks, i % nbk, write=write)
        e.record(stream)
        torch.cuda.synchronize()
        key = {True: "write_then_attend", "extend": "extend_one_call",
               False: "attend_only", "store_only": "store_kv_only"}[write]
        out[key] = a.elapsed_time(e) / 1e3 / (reps * nbk)
    return out


def cpu_prefill(wl, chunks, budget_s):
    """The fp64 oracle on the first chunk's call of a prefill case (all its
    prompts and heads), on host copies of the chunk's K/V/Q written into a
    pool of its own: TFLOP/s of the same algorithmic flops."""
    import oracle

    c = chunks[0]
    hb = lambda t: t.contiguous().view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    bank_of = np.zeros((1, 1), np.int32)
    op = oracle.Pool("bf16", 16, wl.num_pages, wl.heads, wl.D, bank_of, 1)
    if c["start"]:  # the cached prefix, as the generator left it in the pool
        op.k[0] = hb(wl.pool.k[0])
        op.v[0] = hb(wl.pool.v[0])
    oracle.kv_write(op, 0, 0, hb(c["k"]), hb(c["v"]), c["slots"].cpu().numpy())
    q, cu = hb(c["q"]), c["cu"].cpu().numpy()
    seq = c["seq"].cpu().numpy()
    flops = 4 * wl.D * wl.heads * c["pairs"]
    done, spent, calls = 0, 0.0, 0
    while spent < budget_s and (calls == 0 or spent + spent / calls <= budget_s):
        t0 = time.perf_counter()
        oracle.prefill(op, 0, 0, q, cu, wl.table, seq)
        spent += time.perf_counter() - t0
        done += flops
        calls += 1
    return {"value": round(done / spent / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(os.environ.get("OMP_NUM_THREADS", "1")), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{calls} x the first call of the case ({wl.prompts} prompts x "
                      f"{c['q_len']} query rows, {wl.heads} heads, fp64 oracle), {spent:.2f} s"}


def run_prefill(reps=3, supplementary=True, cpu_budget=0.0):
    """TFLOP/s of causal prefill: 4 * head_dim * heads * (visible query-key
    pairs) algorithmic flops per call, written then attended. The cached-prefix
    cases are calls over 8 x 512-token prompts, rotating over 132 banks; the
    supplementary case 8 cold 2048-token prompts, rotating over 24 banks."""
    res = {}
    cases = list(PREFILL_CASES) + ([SUPPLEMENTARY] if supplementary else [])
    wls = {}
    for name, prompts, n, chunk, start in cases:
        if (prompts, n) not in wls:
            wls[(prompts, n)] = PrefillWorkload(prompts, n, banks=132 if n <= 512 else 24)
        wl = wls[(prompts, n)]
        chunks = wl.schedule(chunk, start)
        flops = 4 * wl.D * wl.heads * sum(c["pairs"] for c in chunks)
        hbm = sum(c["hi"] * wl.prompts * 2 * wl.heads * wl.D * 2 + 2 * c["q"].numel() * 2
                  for c in chunks)
        t = time_prefill_case(wl, chunks, reps)
        # store_kv: the chunk's K and V read from the caller's buffers and
        # written to their slots
        kv = sum(c["k"].numel() + c["v"].numel() for c in chunks) * 2 * 2
        st = t.pop("store_kv_only")
        out = {"store_kv": {"us": round(st * 1e6, 2), "bytes": kv,
                            "GBps": round(kv / st / 1e9, 1),
                            "hbm_frac": round(kv / st / 1e9 / HBM_PEAK_GBS, 4),
                            "kernel": "kv_write_kernel (paged_kv_write per chunk)"}}
        for key, sec in t.items():
            out[key] = {"us": round(sec * 1e6, 2), "TFLOPs": round(flops / sec / 1e12, 2),
                        "mfma_frac": round(flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                        "hbm_GBps": round(hbm / sec / 1e9, 1),
                        "hbm_frac": round(hbm / sec / 1e9 / HBM_PEAK_GBS, 4)}
        out["calls_per_case"] = len(chunks)
        out["flops"] = flops
        out["algorithmic_bytes"] = hbm
        sec = t["attend_only"] / len(chunks)
        if name == "cold_chunk2048":
            out["roofline"] = roofline(
                "prefill_cold2048", "prefill_mfma<4, 2, 2048, 2> (8 x 512 rows, 4 tiles each)",
                flops / sec / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", "mfma", flops, sec,
                hbm_frac=round(hbm / sec / 1e9 / HBM_PEAK_GBS, 4),
                note="at the ridge: 128 flop per algorithmic byte; the HBM floor of the "
                     "call is 16.8 us")
        if name == SUPPLEMENTARY[0]:
            out["roofline"] = roofline(
                "prefill_8x2048", "prefill_mfma<4, 2, 2048, 2> (8 x 2048 rows, 16 tiles each)",
                flops / sec / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", "mfma", flops, sec)
        if cpu_budget > 0 and name in ("cold_chunk2048", "suffix16_over_496"):
            log(f"cpu baseline (oracle): prefill {name} ...")
            out["cpu_baseline"] = cpu_prefill(wl, chunks, cpu_budget)
        res[name] = out
        log(f"prefill {name}: {out}")
    return res


def run_lotus(prompts=8, prompt_len=512, block=64, loop_iters=4, heads=32, D=128, reps=20):
    """The LOTUS in-place loop: loop_iters + 1 passes over a fixed block of
    `block` latent positions after each cached prompt, each pass one
    paged_extend_attn (store_kv of the block to the same slots + extend-prefill
    of all block rows). Reports the time per pass and per loop, and TFLOP/s of
    4 * D * heads * (visible query-key pairs)."""
    import torch

    import paged_kv_attention_kvcache_amd as pkv
    from paged_kv_attention_kvcache_amd import synth

    rng = np.random.default_rng(0)
    lens = np.full(prompts, prompt_len + block, np.int32)
    table, num_pages, _ = synth.allocate_pages(rng, lens, 16)
    bank_of, nb = pkv.bank_map(1, 1)
    shape = (1, num_pages, heads, 16, D)
    k = synth.device_normal_(torch.empty(shape, dtype=torch.bfloat16, device="cuda"), 11)
    v = synth.device_normal_(torch.empty(shape, dtype=torch.bfloat16, device="cuda"), 12)
    pool = pkv.Pool(torch.bfloat16, num_pages, heads, D, bank_of, nb, k=k, v=v)
    lb = pkv.LotusBlock(pool, 0, 0, torch.from_numpy(table).cuda(), [prompt_len] * prompts,
                        block)
    rows = prompts * block
    mk = lambda s_: synth.device_normal_(torch.empty((loop_iters + 1, rows, heads, D),
                                                     dtype=torch.bfloat16, device="cuda"), s_)
    kp, vp, qp = mk(13), mk(14), mk(15)
    out = torch.empty((rows, heads, D), dtype=torch.bfloat16, device="cuda")

    def loop():
        for i in range(loop_iters + 1):
            lb.pass_(kp[i], vp[i], qp[i], out=out, with_lse=False)

    loop()
    torch.cuda.synchronize()
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        loop()
    e.record()
    torch.cuda.synchronize()
    loop_s = a.elapsed_time(e) / 1e3 / reps
    pairs = prompts * sum(prompt_len + j + 1 for j in range(block))
    flops = 4 * D * heads * pairs * (loop_iters + 1)
    res = {"prompts": prompts, "prompt_len": prompt_len, "block": block,
           "loop_iters": loop_iters, "heads": heads, "head_dim": D,
           "us_per_loop": round(loop_s * 1e6, 2),
           "us_per_pass": round(loop_s * 1e6 / (loop_iters + 1), 2),
           "TFLOPs": round(flops / loop_s / 1e12, 2),
           "how": "paged_extend_attn per pass (store_kv to the block's fixed slots + "
                  "extend-prefill of the block)"}
    log(f"lotus: {res}")
    return res


def run_latest_bank(wl, steps=10, warmup=2):
    """The Huginn-shaped step where context tokens halted early at depths
    uniform in [20, 31] and recurrent-layer calls read each token from its
    latest bank (paged_decode_latest_attn), timed on the same workload after
    its ordinary step. Logical KV bytes are the same in both."""
    import torch

    stream = torch.cuda.current_stream()
    wl.use_exit_depths(20, 31)
    for _ in range(warmup):
        wl.step()
    torch.cuda.synchronize()
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        wl.step()
    e.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(e) / steps
    wl.exit_depth = None
    return {"ms_per_step": round(ms, 4),
            "kv_GBps_logical": round(wl.kv_bytes_per_call * len(wl.order) / (ms / 1e3) / 1e9, 2),
            "exit_depths": "uniform[20,31] per context token",
            "how": "paged_decode_latest_attn for plane >= 1 (store_kv of the newest token fused)"}


def run_tiny(reps=500, cpu_budget=0.0):
    """The tiny decode shape (fp32, 4 requests of 17-64 tokens, 4 query / 2 kv
    heads, head_dim 64, a 64-page pool): the fused store_kv + attention call,
    timed per call. At about 166 KB of KV it measures launch latency, not
    bandwidth."""
    import torch

    import paged_kv_attention_kvcache_amd as pkv
    from paged_kv_attention_kvcache_amd import synth

    case = synth.make_decode_case(0, "f32", 4, (17, 64), 4, 2, 64, num_pages=64)
    bank_of, nb = pkv.bank_map(1, 1)
    shape = (nb, 64, 2, 16, 64)
    pool = pkv.Pool(torch.float32, 64, 2, 64, bank_of, nb,
                    k=torch.zeros(shape, device="cuda"), v=torch.zeros(shape, device="cuda"))
    bd = case.banks[(0, 0)]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    pkv.kv_write(pool, 0, 0, dev(bd.fill_k), dev(bd.fill_v), dev(bd.fill_slots))
    q, nk, nv = dev(bd.q), dev(bd.new_k), dev(bd.new_v)
    table, seq = dev(case.page_table), dev(case.seq_lens)
    mx = int(case.seq_lens.max())
    ws = torch.empty(max(pkv.workspace_bytes(pool, 4, 4, mx, 0), 1), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((4, 4, 64), device="cuda")
    lse = torch.empty((4, 4), device="cuda")
    call = lambda: pkv.decode(pool, 0, 0, q, table, seq, mx, out=out, lse=lse, workspace=ws,
                              k_new=nk, v_new=nv)
    for _ in range(20):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    kv = int(case.seq_lens.sum()) * 2 * 2 * 64 * 4
    res = {"config": dict(workload="tiny_decode", batch=4, seq_lens="uniform[17,64]",
                          q_heads=4, kv_heads=2, head_dim=64, dtype="fp32", num_pages=64),
           "us_per_call": round(us, 3), "kv_bytes": kv, "kv_GBps": round(kv / us / 1e3, 2),
           "how": "paged_decode_append_attn back to back on one stream (launch-bound; "
                  "not held to the HBM bar)"}
    if cpu_budget > 0:
        import oracle

        op = oracle.Pool("f32", 16, 64, 2, 64, bank_of, nb)
        oracle.kv_write(op, 0, 0, bd.fill_k, bd.fill_v, bd.fill_slots)
        oracle.kv_write(op, 0, 0, bd.new_k, bd.new_v, bd.new_slots)
        spent, calls = 0.0, 0
        while spent < cpu_budget:
            t0 = time.perf_counter()
            oracle.decode(op, 0, 0, bd.q, case.page_table, case.seq_lens)
            spent += time.perf_counter() - t0
            calls += 1
        res["cpu_baseline"] = {
            "value": round(spent / calls * 1e6, 3), "unit": "us per call",
            "cores": int(os.environ.get("OMP_NUM_THREADS", "1")), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{calls} calls of the whole tiny decode (4 requests, 4 heads; the "
                      f"oracle's attention alone, its store_kv done once), {spent:.2f} s"}
    return res


def run_page_mgr(reps=200):
    """Host bookkeeping of the page manager for one Huginn-shaped decode step
    (16 requests, 132 bank writes of one token each, then a publication
    check of every request's page-table row over 32 planes), and the cost
    of allocating and releasing pages."""
    import paged_kv_attention_kvcache_amd as pkv

    bank_of, _ = pkv.bank_map(32, 8, 2, 4)
    order = [(0, 0), (0, 1)] + [(t, l) for t in range(32) for l in range(2, 6)] + \
            [(0, 6), (0, 7)]
    B, pages_per_req = 16, 126  # 2000-token prompts
    m = pkv.PageManager(B * pages_per_req + 64, bank_of)
    rows = [m.alloc(pages_per_req) for _ in range(B)]
    slots = np.array([r[-1] * 16 + 3 for r in rows], np.int32)
    t0 = time.perf_counter()
    for _ in range(reps):
        for (p, l) in order:
            m.note_write(p, l, slots)
        for r in rows:
            m.published_prefix(32, r)
    step_us = (time.perf_counter() - t0) / reps * 1e6
    t0 = time.perf_counter()
    for _ in range(reps):
        ids = m.alloc(64)
        m.release(ids)
    pair_us = (time.perf_counter() - t0) / reps * 1e6
    m.close()
    return {"host_us_per_huginn_step": round(step_us, 2),
            "host_us_alloc_release_64_pages": round(pair_us, 2),
            "how": "pkv_mgr_note_write per bank call + pkv_mgr_published_prefix per request, "
                   "through the Python binding (host only)"}


# --------------------------------------------------------------------------- CPU baseline

def cpu_model() -> str:
    """The host CPU's model name (as /proc/cpuinfo states it)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads() -> int:
    """Threads the oracle runs with: every core this process may use."""
    threads = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(threads))
    return int(os.environ["OMP_NUM_THREADS"])


def cpu_baseline(wl: DecodeWorkload, budget_s: float = 8.0):
    """The fp64 oracle, as it stands, on the workload's host snapshots (whole
    banks of the step, or a subset of the requests of one bank, copied before
    any library kernel ran) until about budget_s of CPU time; scaled to
    logical KV GB/s like the GPU value."""
    import oracle

    cores = cpu_threads()
    done_bytes, spent, calls = 0, 0.0, 0
    bank_of = np.zeros((1, 1), np.int32)
    pools = [(oracle.Pool("bf16", 16, k.shape[1], wl.hkv, wl.D, bank_of, 1, k, v), q, t, n, b)
             for k, v, q, t, n, b in wl.snap]
    while pools and spent < budget_s:
        for op, q, table, seq, nbytes in pools:
            t0 = time.perf_counter()
            oracle.decode(op, 0, 0, q, table, seq)
            spent += time.perf_counter() - t0
            done_bytes += nbytes
            calls += 1
            if spent >= budget_s:
                break
    rows = len(wl.snap[0][4]) if wl.snap else 0
    what = (f"{len(wl.snap)} distinct banks of the {len(wl.order)} in one {wl.name} step, "
            f"{wl.batch} requests, all heads" if rows == wl.batch else
            f"the first {rows} of the {wl.batch} requests of one call, all heads")
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{calls} oracle decode calls over {what}; logical KV bytes of those "
                      f"calls / {spent:.1f} s (fp64)"}


# --------------------------------------------------------------------------- decode configs

def time_decode(wl, steps, warmup, graph=True):
    """Times wl's step: K whole steps between two HIP events on the stream
    the library launches on; per-step spread; the decode calls alone back to
    back (the dominant kernel's time per call); and the step replayed as one
    submission."""
    import torch

    nb = len(wl.order)
    for _ in range(warmup):
        wl.step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(steps):
        wl.step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / steps
    # Per-step spread: K more steps, each between its own pair of events
    # (after the timed region, so that region is K steps and nothing else).
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for k in range(steps):
        wl.step()
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(steps)])
    spread = {f"p{q}": round(float(np.percentile(per_step, q)), 4) for q in (10, 50, 90)}
    # The decode calls alone, back to back over K rounds of every bank.
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for _ in range(steps):
        for i in range(nb):
            wl.call(i, decode_only=True)
    d1.record(stream)
    torch.cuda.synchronize()
    call_s = d0.elapsed_time(d1) / 1e3 / (steps * nb)
    res = {"ms_per_step": ms_per_step, "spread": spread, "call_s": call_s, "wall_s": wall}
    if graph:
        g = wl.step_graph()
        for _ in range(max(warmup, 1)):
            g.launch(stream)
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(steps):
            g.launch(stream)
        g1.record(stream)
        torch.cuda.synchronize()
        res["graph_ms"] = g0.elapsed_time(g1) / steps
        g.close()
    return res


def decode_summary(wl, t):
    """The step's figures: logical KV GB/s over the whole step, its share of
    HBM peak, tokens x planes per second, and the single-submission replay."""
    nb = len(wl.order)
    step_bytes = wl.kv_bytes_per_call * nb
    gbs = step_bytes / (t["ms_per_step"] / 1e3) / 1e9
    out = {"ms_per_step": round(t["ms_per_step"], 4),
           "ms_per_step_spread": t["spread"],
           "kv_GBps": round(gbs, 2),
           "hbm_frac_step": round(gbs / HBM_PEAK_GBS, 4),
           "tokens_planes_per_s": round(wl.batch * nb / (t["ms_per_step"] / 1e3), 1),
           "decode_call_us": round(t["call_s"] * 1e6, 2),
           "split": wl.split,
           "kv_bytes_per_call": wl.kv_bytes_per_call,
           "unique_kv_bytes_per_call": wl.unique_bytes_per_call}
    if "graph_ms" in t:
        g = t["graph_ms"]
        out["single_submission"] = {
            "ms_per_step": round(g, 4), "kv_GBps": round(step_bytes / (g / 1e3) / 1e9, 2),
            "tokens_planes_per_s": round(wl.batch * nb / (g / 1e3), 1),
            "how": "paged_decode_step_capture + graph launch per step"}
    return out


def run_ouro(args):
    """The headline: the Ouro-shaped 96-bank step."""
    wl = make_workload("ouro", args.partition, 0 if args.no_cpu_baseline else args.cpu_banks)
    wl.separate_write = args.separate_write
    t = time_decode(wl, args.steps, args.warmup)
    res = decode_summary(wl, t)
    achieved = wl.kv_bytes_per_call / t["call_s"] / 1e9
    res["roofline"] = roofline("ouro", wl.kernel_name, achieved, HBM_PEAK_GBS, "GB/s", "hbm",
                               wl.kv_bytes_per_call, t["call_s"],
                               bytes="logical K+V of every request's context per call")
    res["step"] = ("paged_kv_write + paged_decode_attn" if wl.separate_write
                   else "paged_decode_append_attn (store_kv of the newest token fused)")
    res["wall_s_timed"] = round(t["wall_s"], 3)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle): ouro ...")
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    return res


def run_huginn(args, steps=None):
    """The Huginn-shaped 132-bank step, 78% of prompt pages aliased: logical
    and unique bytes, and the early-exit variant of the same step."""
    import torch

    steps = steps or args.steps
    wl = make_workload("huginn", 0, 0 if args.no_cpu_baseline else args.cpu_banks)
    t = time_decode(wl, steps, args.warmup)
    res = decode_summary(wl, t)
    nb = len(wl.order)
    uniq = wl.unique_bytes_per_call * nb / (t["ms_per_step"] / 1e3) / 1e9
    res["kv_GBps_logical"] = res.pop("kv_GBps")
    res["hbm_frac_logical"] = res.pop("hbm_frac_step")
    res["kv_GBps_unique"] = round(uniq, 2)
    res["hbm_frac_unique"] = round(uniq / HBM_PEAK_GBS, 4)
    achieved = wl.unique_bytes_per_call / t["call_s"] / 1e9
    res["roofline"] = roofline(
        "huginn", wl.kernel_name, achieved, HBM_PEAK_GBS, "GB/s", "hbm",
        wl.unique_bytes_per_call, t["call_s"],
        bytes="unique K+V pages per call (each aliased prefix page once)",
        achieved_logical=round(wl.kv_bytes_per_call / t["call_s"] / 1e9, 2))
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle): huginn ...")
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget / 2)
    res["config"] = CONFIG_TEXT["huginn"]
    res["latest_bank"] = run_latest_bank(wl, steps=min(steps, 10))
    log(f"huginn: {res}")
    del wl
    torch.cuda.empty_cache()
    return res


def run_longctx(args, steps=None):
    """One long-context call (batch 256, 8k-32k tokens, GQA 8): the library's
    balanced split, then the stated split-K over fixed 512-token partitions."""
    import torch

    steps = steps or args.steps
    wl = make_workload("longctx", 0, 0, 0 if args.no_cpu_baseline else 32)
    t = time_decode(wl, steps, args.warmup, graph=False)
    res = {"balanced": decode_summary(wl, t)}
    achieved = wl.kv_bytes_per_call / t["call_s"] / 1e9
    res["balanced"]["roofline"] = roofline(
        "longctx", wl.kernel_name, achieved, HBM_PEAK_GBS, "GB/s", "hbm", wl.kv_bytes_per_call,
        t["call_s"], bytes="logical K+V of every request's context per call")
    fx = wl.time_fixed_partitions(512, steps, torch.cuda.current_stream())
    fx["roofline"] = roofline(
        "longctx_p512", fx["kernel"], fx["kv_GBps"], HBM_PEAK_GBS, "GB/s", "hbm",
        wl.kv_bytes_per_call, fx["us_per_call"] / 1e6,
        bytes="logical K+V of every request's context per call")
    res["fixed_partition_512"] = fx
    res["config"] = CONFIG_TEXT["longctx"]
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle): longctx ...")
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget / 2)
    log(f"longctx: {res}")
    del wl
    torch.cuda.empty_cache()
    return res


def run_probe(kind: str):
    """Plain copy / read of a buffer of known size, to calibrate the HBM byte
    counters (FETCH_SIZE, WRITE_SIZE) and to give the achievable bandwidth."""
    import torch

    nbytes = 1 << 30
    x = torch.empty(nbytes // 8, dtype=torch.int64, device="cuda").random_()
    y = torch.empty_like(x)
    fn = (lambda: y.copy_(x)) if kind == "copy" else (lambda: x.max())
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    moved = (2 if kind == "copy" else 1) * nbytes
    return {"probe": kind, "bytes_per_launch": nbytes, "read_bytes": nbytes,
            "write_bytes": nbytes if kind == "copy" else 0, "ms": round(ms, 4),
            "GBps": round(moved / ms / 1e6, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all", choices=["all", "ouro", "huginn", "longctx"],
                    help="all (default): the Ouro headline plus every other workload under "
                         "configs; otherwise one decode workload alone")
    ap.add_argument("--partition", type=int, default=0)
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill cases and the LOTUS loop")
    ap.add_argument("--no-supplementary", action="store_true",
                    help="skip the 8 x 2048-token prefill shape")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the chunked-prefill measurement (one JSON line of its cases)")
    ap.add_argument("--separate-write", action="store_true",
                    help="paged_kv_write + paged_decode_attn per bank instead of the fused call")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=8.0,
                    help="seconds of oracle time for the headline's CPU baseline (half that "
                         "for the Huginn and long-context ones)")
    ap.add_argument("--probe", choices=["copy", "read"], default=None,
                    help="time a plain copy/read of 1 GiB instead (counter calibration)")
    ap.add_argument("--cpu-banks", type=int, default=4,
                    help="bank calls snapshotted for the CPU baseline (upper bound)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path "
              f"has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)
    import torch

    import paged_kv_attention_kvcache_amd as pkv

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    pkv.lib()
    if args.probe:
        print(json.dumps(run_probe(args.probe)), flush=True)
        return
    if not args.no_cpu_baseline:
        cpu_threads()
    cpu = 0.0 if args.no_cpu_baseline else 1.0
    log(f"device: {torch.cuda.get_device_name(0)}; workload {args.workload}")
    if args.prefill_only:
        print(json.dumps({"prefill": run_prefill(supplementary=not args.no_supplementary,
                                                 cpu_budget=cpu),
                          "lotus": run_lotus()}), flush=True)
        return
    if args.workload in ("huginn", "longctx"):
        res = run_huginn(args) if args.workload == "huginn" else run_longctx(args)
        print(json.dumps({"metric": METRIC, "workload": CONFIG_TEXT[args.workload]["workload"],
                          "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "config": CONFIG_TEXT[args.workload], **res}), flush=True)
        return
    ouro = run_ouro(args)
    res = {
        "metric": METRIC,
        "value": ouro["kv_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ouro["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V/Q, random page permutation)",
        "config": dict(CONFIG_TEXT["ouro"], partition=args.partition),
        "roofline": ouro["roofline"],
    }
    if "cpu_baseline" in ouro:
        res["cpu_baseline"] = ouro["cpu_baseline"]
    configs = {"ouro_fixed_depth_decode": ouro}
    if args.workload == "all":
        torch.cuda.empty_cache()
        configs["tiny_decode"] = run_tiny(cpu_budget=cpu)
        configs["huginn_recurrent_depth_decode"] = run_huginn(args)
        configs["long_context_decode"] = run_longctx(args)
        if not args.no_prefill:
            pf = run_prefill(supplementary=not args.no_supplementary, cpu_budget=cpu)
            configs["cached_prefix_prefill"] = {k: pf[k] for k, *_ in PREFILL_CASES}
            configs["cached_prefix_prefill"]["config"] = dict(
                workload="cached_prefix_prefill", prompts=8, tokens=512, cached_tokens=496,
                heads=32, head_dim=128, page_size=16, banks_rotated=132)
            if SUPPLEMENTARY[0] in pf:
                configs["prefill_8x2048"] = pf[SUPPLEMENTARY[0]]
            res["lotus"] = run_lotus()
            torch.cuda.empty_cache()
            res["hbm_probe"] = {k: run_probe(k)["GBps"] for k in ("copy", "read")}
            res["hbm_probe"]["how"] = ("torch copy_ (read + write) and max (read) of 1 GiB: "
                                       "the bandwidth a library kernel reaches")
    res["configs"] = configs
    res["page_manager"] = run_page_mgr()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
