"""GPU-side helpers for the parity tests: device pools and transfers.

Nothing here computes attention; it moves the generator's arrays to and from
the device and wraps the library's pool."""
from __future__ import annotations

import math
import sys

import numpy as np

import paged_kv_attention_kvcache_amd as pkv
from paged_kv_attention_kvcache_amd import synth


def torch():
    import torch as _t

    return _t


def tdtype(dtype: str):
    t = torch()
    return t.bfloat16 if dtype == "bf16" else t.float32


def to_dev(a: np.ndarray, dtype: str):
    t = torch()
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return t.from_numpy(a.view(np.int16)).cuda().view(t.bfloat16)
    return t.from_numpy(a.astype(np.float32)).cuda()


def i32_dev(a) -> "torch.Tensor":
    return torch().from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).cuda()


def bits(t) -> np.ndarray:
    """Raw storage bits of a device tensor (uint16 for bf16, uint32 for fp32)."""
    T = torch()
    if t.dtype == T.bfloat16:
        return t.contiguous().view(T.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().view(T.int32).cpu().numpy().view(np.uint32)


def f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def gpu_pool(layout: synth.Layout, poison: bool = True) -> pkv.Pool:
    T = torch()
    bank_of, nb = pkv.bank_map(layout.num_planes, layout.num_layers, layout.rec_first,
                               layout.rec_count)
    dt = tdtype(layout.dtype)
    shape = (nb, layout.num_pages, layout.num_kv_heads, layout.page_size, layout.head_dim)
    fill = float("nan") if poison else 0.0
    k = T.full(shape, fill, dtype=dt, device="cuda")
    v = T.full(shape, fill, dtype=dt, device="cuda")
    return pkv.Pool(dt, layout.num_pages, layout.num_kv_heads, layout.head_dim, bank_of, nb,
                    page_size=layout.page_size, k=k, v=v)


def write(pool: pkv.Pool, plane, layer, k: np.ndarray, v: np.ndarray, slots: np.ndarray,
          dtype: str):
    if len(slots) == 0:
        return
    pkv.kv_write(pool, plane, layer, to_dev(k, dtype), to_dev(v, dtype), i32_dev(slots))


def gpu_decode_case(case: synth.DecodeCase, plane=0, layer=0, pool=None, partition=0,
                    scale=None):
    """Write the context and the new token through paged_kv_write, then decode."""
    dt = case.layout.dtype
    pool = pool if pool is not None else gpu_pool(case.layout)
    bd = case.banks[(plane, layer)]
    write(pool, plane, layer, bd.fill_k, bd.fill_v, bd.fill_slots, dt)
    write(pool, plane, layer, bd.new_k, bd.new_v, bd.new_slots, dt)
    q = to_dev(bd.q, dt)
    out, lse = pkv.decode(pool, plane, layer, q, i32_dev(case.page_table),
                          i32_dev(case.seq_lens), int(case.seq_lens.max()), scale=scale,
                          partition=partition)
    torch().cuda.synchronize()
    return out, lse, pool


def report(tag: str, got, ref_o, ref_l, got_l=None):
    """Max-abs error, LSE max-abs error and rel-RMS of an output vs the oracle."""
    g = f64(got) if not isinstance(got, np.ndarray) else got
    err = np.abs(g - ref_o)
    max_abs = float(err.max()) if err.size else 0.0
    rel_rms = float(np.sqrt(((g - ref_o) ** 2).sum() / max((ref_o ** 2).sum(), 1e-300)))
    lse_err = 0.0
    if got_l is not None:
        gl = f64(got_l)
        finite = np.isfinite(ref_l)
        assert np.array_equal(np.isfinite(gl), finite), f"{tag}: lse finiteness differs"
        if finite.any():
            lse_err = float(np.abs(gl[finite] - ref_l[finite]).max())
    print(f"[{tag}] max_abs={max_abs:.3e} lse_max_abs={lse_err:.3e} rel_rms={rel_rms:.3e}",
          file=sys.stderr, flush=True)
    return max_abs, lse_err, rel_rms


TOL = {"f32": dict(max_abs=1e-5, lse=1e-5, rel_rms=1e-5),
       "bf16": dict(max_abs=2e-2, lse=1e-4, rel_rms=5e-3)}


def check(tag: str, dtype: str, got, ref_o, ref_l, got_l=None):
    """The parity bar: max-abs <= 1e-5 (fp32) / 2e-2 (bf16) against the fp64
    oracle, plus LSE and rel-RMS diagnostics held to the bounds above."""
    max_abs, lse_err, rel = report(tag, got, ref_o, ref_l, got_l)
    tol = TOL[dtype]
    assert max_abs <= tol["max_abs"], f"{tag}: max_abs {max_abs}"
    assert lse_err <= tol["lse"], f"{tag}: lse {lse_err}"
    assert rel <= tol["rel_rms"] or np.abs(ref_o).max() == 0, f"{tag}: rel_rms {rel}"


def scale_of(D: int) -> float:
    return 1.0 / math.sqrt(D)


def sample_for_oracle(k_bank, v_bank, page_table: np.ndarray, seq_lens: np.ndarray, rows,
                      dtype: str):
    """Copy the pages of the sampled requests (one bank, as the generator left
    it) to the host and renumber them, for the oracle to attend over.

    Returns (oracle.Pool with one bank, page table of the sampled rows)."""
    import oracle

    T = torch()
    P = k_bank.shape[2]
    need = [page_table[r, :-(-int(seq_lens[r]) // P)] for r in rows]
    uniq = np.unique(np.concatenate(need)) if need else np.zeros(0, np.int32)
    remap = {int(p): i for i, p in enumerate(uniq)}
    idx = T.from_numpy(uniq.astype(np.int64)).cuda()
    hk = bits(k_bank.index_select(0, idx))[None]
    hv = bits(v_bank.index_select(0, idx))[None]
    if dtype == "f32":
        hk, hv = hk.view(np.float32), hv.view(np.float32)
    bank_of = np.zeros((1, 1), np.int32)
    pool = oracle.Pool(dtype, P, len(uniq), k_bank.shape[1], k_bank.shape[3], bank_of, 1,
                       hk, hv)
    stride = page_table.shape[1]
    table = np.zeros((len(rows), stride), np.int32)
    for i, r in enumerate(rows):
        for j, p in enumerate(need[i]):
            table[i, j] = remap[int(p)]
    return pool, table


def say(*a):
    """Names the case about to run (flushed, so a failing run shows it)."""
    print(*a, file=sys.stderr, flush=True)


def full_size_pool(f, seed=11):
    """The full workload's pool, page table, lengths and step inputs, generated
    on the device as the benchmark does."""
    import torch

    rng = np.random.default_rng(seed)
    if f["alias"] > 0:
        prompts = rng.integers(f["lo"], f["hi"] + 1, size=f["B"])
        seq = (prompts + 1).astype(np.int32)
        shared = synth.alias_pages(prompts, f["alias"], 16)
    else:
        seq = rng.integers(f["lo"], f["hi"] + 1, size=f["B"]).astype(np.int32)
        shared = None
    table, num_pages, _ = synth.allocate_pages(rng, seq, 16, shared_pages=shared)
    D = 128
    bank_of, nb = pkv.bank_map(1, 1)
    shape = (1, num_pages, f["hkv"], 16, D)
    k = synth.device_normal_(torch.empty(shape, dtype=torch.bfloat16, device="cuda"), 1)
    v = synth.device_normal_(torch.empty(shape, dtype=torch.bfloat16, device="cuda"), 2)
    pool = pkv.Pool(torch.bfloat16, num_pages, f["hkv"], D, bank_of, nb, k=k, v=v)
    q = synth.device_normal_(torch.empty((f["B"], f["hq"], D), dtype=torch.bfloat16,
                                         device="cuda"), 3)
    nk = synth.device_normal_(torch.empty((f["B"], f["hkv"], D), dtype=torch.bfloat16,
                                          device="cuda"), 4)
    nv = synth.device_normal_(torch.empty((f["B"], f["hkv"], D), dtype=torch.bfloat16,
                                          device="cuda"), 5)
    return pool, table, seq, q, nk, nv
