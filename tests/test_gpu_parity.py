"""GPU parity: the HIP path (through the C-ABI) against the fp64 oracle.

Bars: store_kv bit-exact over the whole pool; attention max-abs <= 1e-5
(fp32) / 2e-2 (bf16) with LSE and rel-RMS diagnostics (gpu_util.check);
page-placement and run-to-run invariants bitwise on the GPU.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest

import oracle
from cases import oracle_decode_case, oracle_pool
from gpu_util import (bits, check, f64, full_size_pool, gpu_decode_case, gpu_pool, i32_dev,
                      sample_for_oracle, tdtype, to_dev, write)
import paged_kv_attention_kvcache_amd as pkv
from paged_kv_attention_kvcache_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    pkv.lib()  # loud failure if the library is missing
    print(f"device: {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ store_kv

WRITE_CASES = {
    # tiny decode shape: fp32, 64-page pool, 2 KV heads, head_dim 64
    "tiny_f32": dict(dtype="f32", batch=4, seq_range=(17, 64), num_q_heads=4, num_kv_heads=2,
                     head_dim=64, num_pages=64),
    # Ouro shape (fewer requests): bf16, 8 KV heads, head_dim 128, 4 planes x 3 layers
    "ouro_bf16": dict(dtype="bf16", batch=8, seq_range=(512, 2048), num_q_heads=16,
                      num_kv_heads=8, head_dim=128, num_planes=4, num_layers=3,
                      planes_layers=[(0, 0), (1, 2), (3, 1)]),
    # Huginn shape: MHA 32 heads, packed planes, 78% aliased prompt pages
    "huginn_bf16": dict(dtype="bf16", batch=4, seq_range=(200, 2000), num_q_heads=32,
                        num_kv_heads=32, head_dim=128, num_planes=3, num_layers=8, rec_first=2,
                        rec_count=4, alias_frac=0.78, planes_layers=[(0, 0), (1, 3), (2, 5)]),
}


@pytest.mark.parametrize("name", sorted(WRITE_CASES))
def test_kv_write_bit_exact(name):
    kw = WRITE_CASES[name]
    say(f"kv_write case {name}")
    case = synth.make_decode_case(0, **kw)
    dt = case.layout.dtype
    gp = gpu_pool(case.layout)
    op = oracle_pool(case.layout)
    for pl, bd in case.banks.items():
        for k, v, s in ((bd.fill_k, bd.fill_v, bd.fill_slots), (bd.new_k, bd.new_v, bd.new_slots)):
            write(gp, *pl, k, v, s, dt)
            oracle.kv_write(op, *pl, k, v, s)
    import torch

    torch.cuda.synchronize()
    gk, gv = bits(gp.k), bits(gp.v)
    ok_ = op.k.view(gk.dtype), op.v.view(gv.dtype)
    assert np.array_equal(gk, ok_[0]) and np.array_equal(gv, ok_[1])


def test_kv_write_overwrite_and_padding():
    rng = np.random.default_rng(3)
    layout = synth.Layout("bf16", 16, 32, 8, 128, num_planes=2, num_layers=2)
    gp, op = gpu_pool(layout), oracle_pool(layout)
    slots = rng.permutation(32 * 16)[:100].astype(np.int32)
    slots[::7] = -1                          # padding rows are skipped
    for round_ in range(3):                  # the same slots again: in-place overwrite
        k = synth.draw(rng, (100, 8, 128), "bf16")
        v = synth.draw(rng, (100, 8, 128), "bf16")
        write(gp, 1, round_ % 2, k, v, slots, "bf16")
        oracle.kv_write(op, 1, round_ % 2, k, v, slots)
    import torch

    torch.cuda.synchronize()
    assert np.array_equal(bits(gp.k), op.k) and np.array_equal(bits(gp.v), op.v)


def test_kv_write_prefill_chunks_bit_exact():
    # cached-prefix prefill writes: 8 prompts x 512 tokens in chunks of 128, 32 heads, D 128
    case = synth.make_prefill_case(1, "bf16", [512] * 8, 32, 32, 128)
    gp, op = gpu_pool(case.layout), oracle_pool(case.layout)
    for ch in synth.chunk_schedule(case, 128):
        write(gp, 0, 0, ch.k, ch.v, ch.slots, "bf16")
        oracle.kv_write(op, 0, 0, ch.k, ch.v, ch.slots)
    import torch

    torch.cuda.synchronize()
    assert np.array_equal(bits(gp.k), op.k) and np.array_equal(bits(gp.v), op.v)


# ------------------------------------------------------------------ decode

DECODE_CASES = {
    # tiny decode, fp32
    "tiny_f32": dict(dtype="f32", batch=4, seq_range=(17, 64), num_q_heads=4,
                        num_kv_heads=2, head_dim=64, num_pages=64),
    # Ouro shape (16 of the 64 requests), G = 2
    "ouro": dict(dtype="bf16", batch=16, seq_range=(512, 2048), num_q_heads=16,
                    num_kv_heads=8, head_dim=128),
    # Huginn shape: MHA with 78% aliased prompt pages
    "huginn": dict(dtype="bf16", batch=16, seq_range=(200, 2000), num_q_heads=32,
                      num_kv_heads=32, head_dim=128, alias_frac=0.78),
    # long-context shape (4 of the 256 requests): GQA group 8, long context
    "longctx": dict(dtype="bf16", batch=4, seq_range=(8192, 32768), num_q_heads=64,
                       num_kv_heads=8, head_dim=128),
    # other kernel instances: bf16 head_dim 64 group 4; fp32 head_dim 128 group 1
    "bf16_d64_g4": dict(dtype="bf16", batch=6, seq_range=(1, 700), num_q_heads=8,
                        num_kv_heads=2, head_dim=64),
    "f32_d128_g1": dict(dtype="f32", batch=5, seq_range=(1, 600), num_q_heads=2,
                        num_kv_heads=2, head_dim=128),
    "f32_d64_g8": dict(dtype="f32", batch=3, seq_range=(30, 1100), num_q_heads=8,
                       num_kv_heads=1, head_dim=64),
    # matrix-core fold, group 4, ragged lengths incl. odd page counts
    "bf16_d128_g4": dict(dtype="bf16", batch=7, seq_range=(1, 1500), num_q_heads=16,
                         num_kv_heads=4, head_dim=128),
    # whole-context mode (64 x 8 (request, kv head) units) with persistent
    # workgroups that take several contexts each: group 2 (vector fold) and
    # group 8 (matrix-core fold)
    "whole_g2": dict(dtype="bf16", batch=64, seq_range=(1, 400), num_q_heads=16,
                     num_kv_heads=8, head_dim=128),
    "whole_g8": dict(dtype="bf16", batch=64, seq_range=(1, 400), num_q_heads=64,
                     num_kv_heads=8, head_dim=128),
}


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", sorted(DECODE_CASES))
def test_decode_parity(name, seed):
    kw = DECODE_CASES[name]
    for q_scale in (1.0, 4.0):  # 4.0: the peaked variant
        say(f"decode {name} seed={seed} q_scale={q_scale}")
        case = synth.make_decode_case(seed, q_scale=q_scale, **kw)
        ro, rl, _ = oracle_decode_case(case)
        for partition in (0, 64):
            out, lse, _ = gpu_decode_case(case, partition=partition)
            check(f"{name}/s{seed}/q{q_scale}/p{partition}", case.layout.dtype, out, ro, rl, lse)


APPEND_CASES = ["tiny_f32", "ouro", "huginn", "longctx", "bf16_d128_g4",
                "bf16_d64_g4", "whole_g2", "whole_g8"]


@pytest.mark.parametrize("partition", [0, 64])
@pytest.mark.parametrize("name", APPEND_CASES)
def test_decode_append_equals_write_then_attend(name, partition):
    """paged_decode_append_attn == paged_kv_write + paged_decode_attn, bitwise,
    outputs and pool bytes; and within tolerance of the oracle."""
    import torch

    kw = DECODE_CASES[name]
    case = synth.make_decode_case(8, **kw)
    dt = case.layout.dtype
    bd = case.banks[(0, 0)]
    out_a, lse_a, pool_a = gpu_decode_case(case, partition=partition)
    pool_b = gpu_pool(case.layout)
    write(pool_b, 0, 0, bd.fill_k, bd.fill_v, bd.fill_slots, dt)
    out_b, lse_b = pkv.decode(pool_b, 0, 0, to_dev(bd.q, dt), i32_dev(case.page_table),
                              i32_dev(case.seq_lens), int(case.seq_lens.max()),
                              partition=partition, k_new=to_dev(bd.new_k, dt),
                              v_new=to_dev(bd.new_v, dt))
    torch.cuda.synchronize()
    assert np.array_equal(bits(pool_a.k), bits(pool_b.k))
    assert np.array_equal(bits(pool_a.v), bits(pool_b.v))
    assert np.array_equal(bits(out_a), bits(out_b)) and np.array_equal(bits(lse_a), bits(lse_b))
    ro, rl, _ = oracle_decode_case(case)
    check(f"append/{name}/p{partition}", dt, out_b, ro, rl, lse_b)


@pytest.mark.parametrize("partition", [0, 16, 32, 512])
def test_decode_edge_lengths(partition):
    # seq_len 0 (empty row), 1, page and partition boundaries, a ragged tail
    lens = [0, 1, 15, 16, 17, 31, 32, 33, 511, 512, 513, 1000]
    case = synth.make_decode_case(5, "bf16", len(lens), (0, 0), 8, 4, 128,
                                  seq_lens=lens)
    ro, rl, _ = oracle_decode_case(case)
    out, lse, _ = gpu_decode_case(case, partition=partition)
    check(f"edge/p{partition}", "bf16", out, ro, rl, lse)
    assert np.all(f64(out)[0] == 0) and np.all(f64(lse)[0] == -np.inf)


@pytest.mark.parametrize("hq,hkv,partition", [(64, 8, 32), (64, 8, 48), (8, 8, 48), (16, 2, 512)])
def test_decode_fixed_partitions(hq, hkv, partition):
    # fixed partitions run on a persistent grid that streams them, one wave
    # per partition, when a partition holds a whole number of the fold's steps
    # (two pages for the matrix-core fold of groups 4 and 8), else one
    # workgroup per partition (48 tokens with group 8). 40 requests, so waves
    # cross request boundaries; lengths at, one below and one past partition
    # multiples, empty and one-token rows.
    rng = np.random.default_rng(17)
    P = partition
    lens = [int(x) for x in rng.integers(0, 3000, size=28)] + \
        [0, 1, P - 1, P, P + 1, 2 * P, 2 * P + 1, 3 * P - 1, 16, 17, 4095, 4096]
    say(f"decode fixed partitions {hq}/{hkv} partition={P}")
    case = synth.make_decode_case(7, "bf16", len(lens), (0, 0), hq, hkv, 128, seq_lens=lens)
    assert pkv.split_mode(gpu_pool(case.layout), len(lens), hq, max(lens), P) == "fixed"
    ro, rl, _ = oracle_decode_case(case)
    out, lse, _ = gpu_decode_case(case, partition=P)
    check(f"fixed/{hq}x{hkv}/p{P}", "bf16", out, ro, rl, lse)
    zero = [i for i, n in enumerate(lens) if n == 0]
    assert np.all(f64(out)[zero] == 0) and np.all(f64(lse)[zero] == -np.inf)


def test_decode_edge_lengths_whole():
    # the same edge lengths in whole-context mode (64 requests x 8 kv heads)
    lens = [0, 1, 15, 16, 17, 31, 32, 33, 511, 512, 513, 1000] * 5 + [0, 2, 4095, 4096]
    case = synth.make_decode_case(5, "bf16", len(lens), (0, 0), 16, 8, 128, seq_lens=lens)
    assert pkv.split_mode(gpu_pool(case.layout), len(lens), 16, max(lens)) == "whole"
    ro, rl, _ = oracle_decode_case(case)
    out, lse, _ = gpu_decode_case(case)
    check("edge/whole", "bf16", out, ro, rl, lse)
    assert np.all(f64(out)[0] == 0) and np.all(f64(lse)[0] == -np.inf)


def test_decode_reduce_on_oracle_partials():
    # the combine kernel alone, fed the oracle's own partials (base-2 units)
    case = synth.make_decode_case(6, "bf16", 6, (1, 900), 8, 2, 128)
    ro, rl, opool = oracle_decode_case(case)
    bd = case.banks[(0, 0)]
    part = 128
    mp = int(math.ceil(case.seq_lens.max() / part))
    pm, pl, pacc = oracle.decode_partials(opool, 0, 0, bd.q, case.page_table, case.seq_lens,
                                          part, mp)
    import torch

    m2 = np.where(np.isfinite(pm), pm * math.log2(math.e), -np.inf).astype(np.float32)
    out, lse = pkv.decode_reduce(
        torch.bfloat16, i32_dev(case.seq_lens), part,
        torch.from_numpy(m2).cuda(), torch.from_numpy(pl.astype(np.float32)).cuda(),
        torch.from_numpy(pacc.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    check("reduce", "bf16", out, ro, rl, lse)


# ------------------------------------------------------------------ prefill

def _prefill_gpu(case, chunks, pool):
    dt = case.layout.dtype
    res = {}
    for ch in chunks:
        write(pool, 0, 0, ch.k, ch.v, ch.slots, dt)
        ql = np.diff(ch.cu_q_lens)
        out, lse = pkv.prefill(pool, 0, 0, to_dev(ch.q, dt), i32_dev(ch.cu_q_lens),
                               i32_dev(case.page_table), i32_dev(ch.seq_lens), int(ql.max()),
                               int(ch.seq_lens.max()))
        res[id(ch)] = (out, lse)
    import torch

    torch.cuda.synchronize()
    return res


def _prefill_oracle(case, chunks, pool):
    res = {}
    for ch in chunks:
        oracle.kv_write(pool, 0, 0, ch.k, ch.v, ch.slots)
        res[id(ch)] = oracle.prefill(pool, 0, 0, ch.q, ch.cu_q_lens, case.page_table,
                                     ch.seq_lens)
    return res


def _prefill_compare(tag, case, chunks, gp, op):
    g = _prefill_gpu(case, chunks, gp)
    o = _prefill_oracle(case, chunks, op)
    for i, ch in enumerate(chunks):
        check(f"{tag}/chunk{i}", case.layout.dtype, g[id(ch)][0], o[id(ch)][0], o[id(ch)][1],
              g[id(ch)][1])


@pytest.mark.parametrize("mode", ["suffix", "chunk128", "chunk2048"])
def test_prefill_cached_prefix_workload(mode):
    # 8 prompts of 512 tokens, 32 MHA heads, head_dim 128, bf16; the first 496
    # tokens of each prompt are cached pages (suffix mode) or prompts are cold.
    say(f"prefill cached-prefix workload {mode}")
    case = synth.make_prefill_case(0, "bf16", [512] * 8, 32, 32, 128)
    gp, op = gpu_pool(case.layout), oracle_pool(case.layout)
    if mode == "suffix":
        k, v, s = synth.prefix_writes(case, [496] * 8)
        write(gp, 0, 0, k, v, s, "bf16")
        oracle.kv_write(op, 0, 0, k, v, s)
        chunks = synth.chunk_schedule(case, 4096, start=[496] * 8)
    else:
        chunks = synth.chunk_schedule(case, 128 if mode == "chunk128" else 2048)
    _prefill_compare(f"cached_prefix/{mode}", case, chunks, gp, op)


def test_prefill_shared_prefix_suffix():
    # all 8 prompts alias one 496-token prefix; the suffix is prefilled
    case = synth.make_prefill_case(2, "bf16", [512] * 8, 32, 32, 128,
                                   shared_prefix_tokens=496)
    gp, op = gpu_pool(case.layout), oracle_pool(case.layout)
    k, v, s = synth.prefix_writes(case, [496] * 8)
    write(gp, 0, 0, k, v, s, "bf16")
    oracle.kv_write(op, 0, 0, k, v, s)
    _prefill_compare("shared_suffix", case, synth.chunk_schedule(case, 4096, start=[496] * 8),
                     gp, op)


@pytest.mark.parametrize("hq,hkv", [(32, 32), (16, 8), (16, 4), (16, 2)])
def test_prefill_short_chunks(hq, hkv):
    # chunks of at most 16 / group rows per request (bf16, head_dim 128) fold
    # each (request, kv head) as one 16-column pass: ragged prompts of 1, 16,
    # 17 tokens and page tails, cached prefixes, a request with no rows, and
    # several chunks in a row
    rows = 16 // (hq // hkv)
    say(f"prefill short chunks {hq}/{hkv}: {rows} rows per request")
    prompts = [512, 37, 1, 200, 16, 1000, 17, 300]
    q_lens = [3 * rows, 2 * rows - 1, 1, rows + 1, 0, rows, 1, 2 * rows]
    starts = [n - min(ql, n) for n, ql in zip(prompts, q_lens)]
    case = synth.make_prefill_case(13, "bf16", prompts, hq, hkv, 128, q_scale=2.0)
    gp, op = gpu_pool(case.layout), oracle_pool(case.layout)
    k, v, sl = synth.prefix_writes(case, starts)
    write(gp, 0, 0, k, v, sl, "bf16")
    oracle.kv_write(op, 0, 0, k, v, sl)
    chunks = synth.chunk_schedule(case, rows, start=starts)
    assert len(chunks) == 3 and all(np.diff(c.cu_q_lens).max() <= rows for c in chunks)
    _prefill_compare(f"short/{hq}x{hkv}", case, chunks, gp, op)


@pytest.mark.parametrize("hq,hkv,chunk", [(32, 32, 64), (16, 4, 64), (16, 2, 64), (16, 2, 65)])
def test_prefill_64_row_tiles(hq, hkv, chunk):
    # calls with at most 64 rows per request run on 64-row tiles (one block of
    # 16 query rows per wave), 65 on 128-row tiles: ragged q_lens of 1 to 130
    # over cached prefixes, a request with no rows, a page-tail prompt, and
    # several chunks in a row
    say(f"prefill 64-row tiles {hq}/{hkv} chunk {chunk}")
    prompts = [600, 64, 1, 300, 130, 1000, 17, 47]
    q_lens = [130, 64, 1, 63, 0, 33, 17, 47]
    starts = [n - min(ql, n) for n, ql in zip(prompts, q_lens)]
    case = synth.make_prefill_case(17, "bf16", prompts, hq, hkv, 128, q_scale=2.0)
    gp, op = gpu_pool(case.layout), oracle_pool(case.layout)
    k, v, sl = synth.prefix_writes(case, starts)
    write(gp, 0, 0, k, v, sl, "bf16")
    oracle.kv_write(op, 0, 0, k, v, sl)
    chunks = synth.chunk_schedule(case, chunk, start=starts)
    assert int(np.diff(chunks[0].cu_q_lens).max()) == chunk
    _prefill_compare(f"tiles64/{hq}x{hkv}/{chunk}", case, chunks, gp, op)


@pytest.mark.parametrize("dtype,hq,hkv,D", [("f32", 8, 2, 64), ("bf16", 8, 1, 128),
                                            ("f32", 2, 2, 128), ("bf16", 4, 2, 64)])
def test_prefill_ragged(dtype, hq, hkv, D):
    # ragged prompts, chunk 48 (not a page multiple), a q_len-0 request mid-batch
    case = synth.make_prefill_case(3, dtype, [37, 100, 16, 1, 200], hq, hkv, D, q_scale=2.0)
    chunks = synth.chunk_schedule(case, 48)
    gp, op = gpu_pool(case.layout), oracle_pool(case.layout)
    _prefill_compare(f"ragged/{dtype}/{hq}x{hkv}x{D}", case, chunks, gp, op)


@pytest.mark.parametrize("hq,hkv", [(16, 16), (16, 2)])
def test_prefill_tile_pairs(hq, hkv):
    # the matrix-core prefill pairs each request's query tiles (T-1-p, p):
    # ragged requests of 1, 2, 3, 5, 7 and 8 tiles of 128 rows in one call
    # (odd counts leave a middle tile alone), q_lens that are not tile
    # multiples, over cached prefixes, plus a request with nothing to do
    say(f"prefill tile pairs {hq}/{hkv}")
    prompts = [900, 200, 700, 600, 64, 1000, 100]
    starts = [0, 0, 400, 20, 64, 150, 0]  # q_len 900, 200, 300, 580, 0, 850, 100: 8, 2, 3, 5, 0, 7, 1 tiles
    case = synth.make_prefill_case(9, "bf16", prompts, hq, hkv, 128)
    gp, op = gpu_pool(case.layout), oracle_pool(case.layout)
    k, v, sl = synth.prefix_writes(case, starts)
    write(gp, 0, 0, k, v, sl, "bf16")
    oracle.kv_write(op, 0, 0, k, v, sl)
    _prefill_compare(f"pairs/{hq}x{hkv}", case, synth.chunk_schedule(case, 4096, start=starts),
                     gp, op)


def test_prefill_full_size_every_prompt():
    """The 8 x 2048 cold prefill in the launch the benchmark prices (one
    2048-token chunk of 8 prompts, 32 MHA heads, head_dim 128, written then
    attended); the oracle checks every row of every prompt on heads 0, 9, 17
    and 31, and every output of the launch is finite."""
    import torch

    say("prefill full-size 8 x 2048")
    case = synth.make_prefill_case(12, "bf16", [2048] * 8, 32, 32, 128)
    chunks = synth.chunk_schedule(case, 2048)
    assert len(chunks) == 1
    out, lse = _prefill_gpu(case, chunks, gpu_pool(case.layout))[id(chunks[0])]
    prompts, heads = list(range(8)), [0, 9, 17, 31]
    sub = synth.PrefillCase(
        synth.Layout("bf16", 16, case.layout.num_pages, len(heads), 128), len(heads),
        case.prompt_lens[prompts], case.page_table[prompts],
        [np.ascontiguousarray(case.k[r][:, heads]) for r in prompts],
        [np.ascontiguousarray(case.v[r][:, heads]) for r in prompts],
        [np.ascontiguousarray(case.q[r][:, heads]) for r in prompts], case.shared[prompts])
    sc = synth.chunk_schedule(sub, 2048)
    ro, rl = _prefill_oracle(sub, sc, oracle_pool(sub.layout))[id(sc[0])]
    rows = torch.from_numpy(np.concatenate([np.arange(r * 2048, (r + 1) * 2048)
                                            for r in prompts])).cuda()
    hd = torch.tensor(heads, device="cuda")
    check("full/8x2048", "bf16", out[rows][:, hd], ro, rl, lse[rows][:, hd])
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(lse).all())


@pytest.mark.parametrize("lens,start", [([36000, 1000], [35800, 900]),
                                        ([70000], [69900])])
def test_prefill_long_context(lens, start):
    # suffixes over long cached prefixes: contexts past 32k tokens take the
    # four-stage matrix-core kernel, past 64k tokens the three-stage one
    say(f"prefill long context {lens}")
    case = synth.make_prefill_case(6, "bf16", lens, 4, 2, 128)
    gp, op = gpu_pool(case.layout), oracle_pool(case.layout)
    k, v, s = synth.prefix_writes(case, start)
    write(gp, 0, 0, k, v, s, "bf16")
    oracle.kv_write(op, 0, 0, k, v, s)
    _prefill_compare(f"long/{lens}", case, synth.chunk_schedule(case, 1 << 20, start=start),
                     gp, op)


# ------------------------------------------------------------------ bitwise invariants

def test_decode_bitwise_invariants():
    kw = DECODE_CASES["huginn"]
    case = synth.make_decode_case(4, **kw)
    a, la, pool = gpu_decode_case(case)
    # run to run
    for _ in range(2):
        b, lb, _ = gpu_decode_case(case, pool=pool)
        assert np.array_equal(bits(a), bits(b)) and np.array_equal(bits(la), bits(lb))
    # a different physical placement of the same logical context, no aliasing
    rng = np.random.default_rng(77)
    table, num_pages, _ = synth.allocate_pages(rng, case.seq_lens, 16)
    layout = synth.Layout("bf16", 16, num_pages, 32, 128)
    gp = gpu_pool(layout)
    bd = case.banks[(0, 0)]
    for r in range(case.batch):
        n = int(case.seq_lens[r])
        write(gp, 0, 0, bd.logical_k[r], bd.logical_v[r],
              synth.slots_of(table, r, np.arange(n), 16), "bf16")
    c, lc = pkv.decode(gp, 0, 0, to_dev(bd.q, "bf16"), i32_dev(table), i32_dev(case.seq_lens),
                       int(case.seq_lens.max()))
    import torch

    torch.cuda.synchronize()
    assert np.array_equal(bits(a), bits(c)) and np.array_equal(bits(la), bits(lc))


def test_prefill_bitwise_shared_vs_private():
    shared = synth.make_prefill_case(2, "bf16", [512] * 4, 32, 32, 128, shared_prefix_tokens=496)
    private = synth.make_prefill_case(2, "bf16", [512] * 4, 32, 32, 128, shared_prefix_tokens=496)
    rng = np.random.default_rng(5)
    private.page_table, n, _ = synth.allocate_pages(rng, private.prompt_lens, 16)
    private.layout.num_pages = n
    private.shared[:] = 0
    outs = []
    for case in (shared, private):
        gp = gpu_pool(case.layout)
        k, v, s = synth.prefix_writes(case, [496] * 4)
        write(gp, 0, 0, k, v, s, "bf16")
        chunks = synth.chunk_schedule(case, 4096, start=[496] * 4)
        res = _prefill_gpu(case, chunks, gp)
        outs.append([(bits(res[id(c)][0]), bits(res[id(c)][1])) for c in chunks])
    for (a, la), (b, lb) in zip(*outs):
        assert np.array_equal(a, b) and np.array_equal(la, lb)


# ------------------------------------------------------------------ full-size, every row

FULL = {
    # one bank call at the full Ouro shape: every request, every head
    "ouro_full": dict(B=64, lo=512, hi=2048, hq=16, hkv=8, alias=0.0, kv_heads=None),
    # Huginn, 78% aliased prompts: every request, every head
    "huginn_full": dict(B=16, lo=200, hi=2000, hq=32, hkv=32, alias=0.78, kv_heads=None),
    # long context: 256 requests, 8k-32k context, GQA 8; the library's balanced
    # split and the stated split-K over fixed 512-token partitions. Every
    # request on kv heads 0 and 5 (q heads 0-7 and 40-47): the host copy of
    # all eight heads would be 43 GB.
    "longctx_full": dict(B=256, lo=8192, hi=32768, hq=64, hkv=8, alias=0.0, kv_heads=[0, 5]),
    "longctx_full_p512": dict(B=256, lo=8192, hi=32768, hq=64, hkv=8, alias=0.0,
                              kv_heads=[0, 5], partition=512),
}


@pytest.mark.parametrize("name", sorted(FULL))
def test_full_size_every_row(name):
    """The full workload in the launch configuration the benchmark times; the
    oracle checks every request (on every kv head, or on two for the long
    context), element by element."""
    import torch

    f = FULL[name]
    say(f"full-size {name}")
    pool, table, seq, q, nk, nv = full_size_pool(f)
    k, v = pool.k, pool.v
    G = f["hq"] // f["hkv"]
    heads = list(range(f["hkv"])) if f["kv_heads"] is None else f["kv_heads"]
    qheads = [h * G + g for h in heads for g in range(G)]
    rows = np.arange(f["B"])
    hidx = torch.tensor(heads, device="cuda")
    # the oracle's copy of the sampled kv heads, taken before any kernel runs
    opool, otable = sample_for_oracle(k[0].index_select(1, hidx), v[0].index_select(1, hidx),
                                      table, seq, rows, "bf16")
    oracle.kv_write(opool, 0, 0, bits(nk)[:, heads], bits(nv)[:, heads],
                    synth.slots_of_last(otable, seq, 16))
    ro, rl = oracle.decode(opool, 0, 0, np.ascontiguousarray(bits(q)[:, qheads]), otable, seq)
    del opool
    # the GPU path: write the new token, then decode, as the benchmark does
    slots = synth.slots_of_last(table, seq, 16)
    pkv.kv_write(pool, 0, 0, nk, nv, i32_dev(slots))
    out, lse = pkv.decode(pool, 0, 0, q, i32_dev(table), i32_dev(seq), int(seq.max()),
                          partition=f.get("partition", 0))
    torch.cuda.synchronize()
    qh = torch.tensor(qheads, device="cuda")
    check(name, "bf16", out.index_select(1, qh), ro, rl, lse.index_select(1, qh))
    # the rows of heads outside the sample are finite (no stray read of
    # poison or of another request's partials)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
