"""Seeded sweep of decode and prefill shapes against the oracle.

Each case draws its shape from a fixed seed: dtype (fp32 / bf16), head_dim
(64 / 128), GQA group (1, 2, 4, 8), kv heads, batch, a length range with
empty and one-token rows, a query scale (1 or the peaked 4), a split mode
(whole-context or balanced when partition is 0, else fixed partitions of a
multiple of 16 tokens) and, for decode, prompt pages aliased between
requests. Prefill cases draw ragged prompts, cached-prefix starts and chunk
sizes. Two more sweeps draw fixed-partition decode shapes (partitions of
16 to 512 tokens, so both fixed-partition kernels run) and short prefill
chunks (at most 16 / group rows per request). The bars are the same as in the
fixed parity cases."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import paged_kv_attention_kvcache_amd as pkv
from paged_kv_attention_kvcache_amd import synth

from cases import oracle_decode_case, oracle_pool
from gpu_util import check, f64, gpu_decode_case, gpu_pool, i32_dev, say, to_dev, write

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    pkv.lib()
    yield
    torch.cuda.synchronize()


def decode_shape(seed: int) -> dict:
    rng = np.random.default_rng(1000 + seed)
    dtype = ["f32", "bf16"][rng.integers(2)]
    D = [64, 128][rng.integers(2)]
    G = [1, 2, 4, 8][rng.integers(4)]
    hkv = [1, 2, 4, 8][rng.integers(4)]
    if seed % 6 == 5:  # enough (request, kv head) pairs for the whole-context mode
        batch, hkv = 64, 8
        hi = int(rng.integers(16, 1200))
    else:
        batch = int(rng.integers(1, 24))
        hi = int([16, 100, 700, 2500, 6000][rng.integers(5)])
    lens = rng.integers(0, hi + 1, size=batch)
    lens[rng.integers(batch)] = 1  # a one-token row in every case
    if batch > 2:
        lens[rng.integers(batch)] = 0  # and an empty one
    partition = int([0, 0, 16, 48, 256, 512][rng.integers(6)])
    q_scale = float([1.0, 4.0][rng.integers(2)])
    alias = float([0.0, 0.5][rng.integers(2)]) if batch > 1 else 0.0
    return dict(dtype=dtype, D=D, hq=G * hkv, hkv=hkv, lens=[int(x) for x in lens],
                partition=partition, q_scale=q_scale, alias=alias)


@pytest.mark.parametrize("seed", range(24))
def test_decode_sweep(seed):
    s = decode_shape(seed)
    say(f"decode sweep {seed}: {s['dtype']} D={s['D']} {s['hq']}/{s['hkv']} "
        f"B={len(s['lens'])} max_len={max(s['lens'])} partition={s['partition']} "
        f"q_scale={s['q_scale']} alias={s['alias']}")
    lens = s["lens"]
    kw = dict(seq_lens=lens, q_scale=s["q_scale"])
    if s["alias"] > 0:
        # that fraction of each request's full context pages come from one
        # shared chain (a nested common prefix)
        kw["shared"] = np.maximum(synth.alias_pages(np.asarray(lens) - 1, s["alias"], 16), 0)
    case = synth.make_decode_case(seed, s["dtype"], len(lens), (0, 0), s["hq"], s["hkv"],
                                  s["D"], **kw)
    ro, rl, _ = oracle_decode_case(case)
    out, lse, _ = gpu_decode_case(case, partition=s["partition"])
    check(f"sweep/decode/{seed}", s["dtype"], out, ro, rl, lse)
    zero = [i for i, n in enumerate(lens) if n == 0]
    if zero:
        assert np.all(f64(out)[zero] == 0) and np.all(f64(lse)[zero] == -np.inf)


def prefill_shape(seed: int) -> dict:
    rng = np.random.default_rng(2000 + seed)
    dtype = ["f32", "bf16", "bf16"][rng.integers(3)]
    D = [64, 128, 128][rng.integers(3)]
    G = [1, 2, 4, 8][rng.integers(4)]
    hkv = [1, 2, 4][rng.integers(3)]
    B = int(rng.integers(1, 7))
    lens = rng.integers(1, 1500, size=B)
    starts = np.array([int(rng.integers(0, n + 1)) if rng.random() < 0.6 else 0 for n in lens])
    starts = np.minimum(starts, lens - 1) if seed % 4 else starts  # some calls with a q_len of 0
    chunk = int([64, 200, 4096][rng.integers(3)])
    q_scale = float([1.0, 4.0][rng.integers(2)])
    return dict(dtype=dtype, D=D, hq=G * hkv, hkv=hkv, lens=[int(x) for x in lens],
                starts=[int(x) for x in starts], chunk=chunk, q_scale=q_scale)


@pytest.mark.parametrize("seed", range(16))
def test_prefill_sweep(seed):
    import torch

    s = prefill_shape(seed)
    say(f"prefill sweep {seed}: {s['dtype']} D={s['D']} {s['hq']}/{s['hkv']} lens={s['lens']} "
        f"starts={s['starts']} chunk={s['chunk']} q_scale={s['q_scale']}")
    case = synth.make_prefill_case(seed, s["dtype"], s["lens"], s["hq"], s["hkv"], s["D"],
                                   q_scale=s["q_scale"])
    gp, op = gpu_pool(case.layout), oracle_pool(case.layout)
    if any(s["starts"]):
        k, v, sl = synth.prefix_writes(case, s["starts"])
        write(gp, 0, 0, k, v, sl, s["dtype"])
        oracle.kv_write(op, 0, 0, k, v, sl)
    chunks = synth.chunk_schedule(case, s["chunk"], start=s["starts"])
    table = i32_dev(case.page_table)
    for i, ch in enumerate(chunks):
        write(gp, 0, 0, ch.k, ch.v, ch.slots, s["dtype"])
        ql = np.diff(ch.cu_q_lens)
        out, lse = pkv.prefill(gp, 0, 0, to_dev(ch.q, s["dtype"]), i32_dev(ch.cu_q_lens), table,
                               i32_dev(ch.seq_lens), int(ql.max()), int(ch.seq_lens.max()))
        torch.cuda.synchronize()
        oracle.kv_write(op, 0, 0, ch.k, ch.v, ch.slots)
        ro, rl = oracle.prefill(op, 0, 0, ch.q, ch.cu_q_lens, case.page_table, ch.seq_lens)
        check(f"sweep/prefill/{seed}/{i}", s["dtype"], out, ro, rl, lse)


def fixed_decode_shape(seed: int) -> dict:
    rng = np.random.default_rng(5000 + seed)
    dtype = ["bf16", "f32"][rng.integers(2)]
    D = [64, 128][rng.integers(2)]
    G = [1, 2, 4, 8][rng.integers(4)]
    hkv = [1, 2, 8][rng.integers(3)]
    B = int(rng.integers(1, 40))
    hi = int(rng.choice([40, 300, 3000]))
    lens = [int(x) for x in rng.integers(0, hi + 1, size=B)]
    partition = int(rng.choice([16, 32, 48, 64, 96, 128, 512]))
    q_scale = float(rng.choice([1.0, 4.0]))
    return dict(dtype=dtype, D=D, G=G, hkv=hkv, lens=lens, partition=partition, q_scale=q_scale)


@pytest.mark.parametrize("seed", range(16))
def test_decode_fixed_partition_sweep(seed):
    # fixed partitions of 16 to 512 tokens: partitions holding a whole number
    # of the fold's steps are streamed by a persistent grid, the others take
    # one workgroup each; up to 39 requests of up to 3000 tokens
    s = fixed_decode_shape(seed)
    say(f"fixed sweep {seed}: {s['dtype']} D={s['D']} G={s['G']} hkv={s['hkv']} "
        f"B={len(s['lens'])} max_len={max(s['lens'])} partition={s['partition']}")
    case = synth.make_decode_case(seed, s["dtype"], len(s["lens"]), (0, 0), s["G"] * s["hkv"],
                                  s["hkv"], s["D"], seq_lens=s["lens"], q_scale=s["q_scale"])
    ro, rl, _ = oracle_decode_case(case)
    out, lse, _ = gpu_decode_case(case, partition=s["partition"])
    check(f"sweep/fixed/{seed}", s["dtype"], out, ro, rl, lse)


@pytest.mark.parametrize("seed", range(16))
def test_prefill_short_chunk_sweep(seed):
    # chunks of at most 16 / group rows per request over cached prefixes
    # (the 16-column short-chunk kernel), requests with no rows, up to three
    # chunks in a row
    import torch

    rng = np.random.default_rng(7000 + seed)
    G = [1, 2, 4, 8][rng.integers(4)]
    hkv = [1, 2, 4][rng.integers(3)]
    rows = 16 // G
    B = int(rng.integers(1, 12))
    lens = [int(x) for x in rng.integers(1, 1200, size=B)]
    qls = [int(min(n, rng.integers(0, 3 * rows + 1))) for n in lens]
    qls[0] = max(qls[0], 1)
    starts = [n - q for n, q in zip(lens, qls)]
    say(f"short-chunk sweep {seed}: G={G} hkv={hkv} lens={lens} q_lens={qls}")
    case = synth.make_prefill_case(seed, "bf16", lens, G * hkv, hkv, 128, q_scale=2.0)
    gp, op = gpu_pool(case.layout), oracle_pool(case.layout)
    if any(starts):
        k, v, sl = synth.prefix_writes(case, starts)
        write(gp, 0, 0, k, v, sl, "bf16")
        oracle.kv_write(op, 0, 0, k, v, sl)
    table = i32_dev(case.page_table)
    for i, ch in enumerate(synth.chunk_schedule(case, rows, start=starts)):
        write(gp, 0, 0, ch.k, ch.v, ch.slots, "bf16")
        ql = np.diff(ch.cu_q_lens)
        assert ql.max() <= rows
        out, lse = pkv.prefill(gp, 0, 0, to_dev(ch.q, "bf16"), i32_dev(ch.cu_q_lens), table,
                               i32_dev(ch.seq_lens), int(ql.max()), int(ch.seq_lens.max()))
        torch.cuda.synchronize()
        oracle.kv_write(op, 0, 0, ch.k, ch.v, ch.slots)
        ro, rl = oracle.prefill(op, 0, 0, ch.q, ch.cu_q_lens, case.page_table, ch.seq_lens)
        check(f"sweep/short/{seed}/{i}", "bf16", out, ro, rl, lse)
