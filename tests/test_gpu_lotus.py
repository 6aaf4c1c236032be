"""The LOTUS in-place loop on the GPU ("Faster fuzzy minds", section
"LOTUS"): paged_extend_attn passes over a fixed block of slots.

Per pass: the block's pool bytes are exactly that pass's K/V (bit-exact
overwrite) and the prompt's bytes are untouched; the pass's attention matches
the oracle's LOTUS loop within tolerance (so it sees only that pass's block);
and paged_extend_attn equals paged_kv_write followed by paged_prefill_attn,
bit for bit."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import paged_kv_attention_kvcache_amd as pkv
from paged_kv_attention_kvcache_amd import synth

from cases import oracle_pool
from gpu_util import bits, check, gpu_pool, i32_dev, say, to_dev, write

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    pkv.lib()
    yield
    torch.cuda.synchronize()


def gather_dev(pool: pkv.Pool, slots: np.ndarray):
    import torch

    s = torch.from_numpy(slots.astype(np.int64)).cuda()
    P = pool.page_size
    return pool.k[0, s // P, :, s % P, :], pool.v[0, s // P, :, s % P, :]


@pytest.mark.parametrize("dtype,hq,hkv,D,prompts,block", [
    ("bf16", 32, 32, 128, [512, 512, 300, 17], 64),   # matrix-core prefill
    ("bf16", 64, 8, 128, [1000, 33], 40),             # GQA 8, ragged block
    ("f32", 4, 2, 64, [37, 70, 5], 23),               # vector prefill
])
def test_lotus_passes(dtype, hq, hkv, D, prompts, block):
    import torch

    say(f"lotus {dtype} {hq}/{hkv} D={D} prompts={prompts} block={block}")
    case = synth.make_lotus_case(7, dtype, prompts, block, 3, hq, hkv, D)
    B = len(prompts)
    cu = np.arange(B + 1, dtype=np.int32) * block
    seq = np.asarray(prompts, np.int32) + block
    op = oracle_pool(case.layout)
    pk, pv = np.concatenate(case.prompt_k), np.concatenate(case.prompt_v)
    oracle.kv_write(op, 0, 0, pk, pv, case.prompt_slots)
    ref = oracle.lotus_loop(op, 0, 0, case.passes, case.block_slots, cu, case.page_table, seq)

    gp = gpu_pool(case.layout)            # the LOTUS driver, one extend call per pass
    gq = gpu_pool(case.layout)            # store_kv + prefill as two calls
    for pool in (gp, gq):
        write(pool, 0, 0, pk, pv, case.prompt_slots, dtype)
    table = i32_dev(case.page_table)
    lb = pkv.LotusBlock(gp, 0, 0, table, prompts, block)
    for i, (k, v, q) in enumerate(case.passes):
        kd, vd, qd = to_dev(k, dtype), to_dev(v, dtype), to_dev(q, dtype)
        out, lse = lb.pass_(kd, vd, qd)
        pkv.kv_write(gq, 0, 0, kd, vd, lb.slots)
        out2, lse2 = pkv.prefill(gq, 0, 0, qd, lb.cu, table, lb.seq, block, lb.max_seq)
        torch.cuda.synchronize()
        bk, bv = gather_dev(gp, case.block_slots)
        assert np.array_equal(bits(bk), bits(kd)) and np.array_equal(bits(bv), bits(vd)), i
        ak, av = gather_dev(gp, case.prompt_slots)
        assert np.array_equal(bits(ak), bits(to_dev(pk, dtype))), i
        assert np.array_equal(bits(av), bits(to_dev(pv, dtype))), i
        assert np.array_equal(bits(out), bits(out2)) and np.array_equal(bits(lse), bits(lse2))
        assert np.array_equal(bits(gp.k), bits(gq.k)) and np.array_equal(bits(gp.v), bits(gq.v))
        check(f"lotus/pass{i}", dtype, out, ref[i][0], ref[i][1], lse)


@pytest.mark.parametrize("chunk,start", [(2048, 0), (128, 0), (200, 37)])
def test_extend_equals_write_then_prefill(chunk, start):
    """paged_extend_attn over a chunk schedule equals paged_kv_write +
    paged_prefill_attn bit for bit, pool included, and the oracle within
    tolerance. Chunks of 2048 (four query tiles, paired), 128 (one tile over
    earlier chunks) and 200 from position 37 (chunks that start and end
    inside a page)."""
    import torch

    say(f"extend chunk={chunk} start={start}")
    case = synth.make_prefill_case(5, "bf16", [512, 300, 450, 129], 16, 8, 128)
    B = len(case.prompt_lens)
    starts = [start] * B
    chunks = synth.chunk_schedule(case, chunk, start=starts)
    op = oracle_pool(case.layout)
    ga, gb = gpu_pool(case.layout), gpu_pool(case.layout)
    if start:
        k, v, sl = synth.prefix_writes(case, starts)
        oracle.kv_write(op, 0, 0, k, v, sl)
        for g in (ga, gb):
            write(g, 0, 0, k, v, sl, "bf16")
    table = i32_dev(case.page_table)
    for ci, ch in enumerate(chunks):
        kd, vd, qd = to_dev(ch.k, "bf16"), to_dev(ch.v, "bf16"), to_dev(ch.q, "bf16")
        sd, cu, seq = i32_dev(ch.slots), i32_dev(ch.cu_q_lens), i32_dev(ch.seq_lens)
        mq, ms = int(np.diff(ch.cu_q_lens).max()), int(ch.seq_lens.max())
        out_a, lse_a = pkv.extend(ga, 0, 0, kd, vd, sd, qd, cu, table, seq, mq, ms)
        pkv.kv_write(gb, 0, 0, kd, vd, sd)
        out_b, lse_b = pkv.prefill(gb, 0, 0, qd, cu, table, seq, mq, ms)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out_a), bits(out_b)) and np.array_equal(bits(lse_a), bits(lse_b))
        assert np.array_equal(bits(ga.k), bits(gb.k)) and np.array_equal(bits(ga.v), bits(gb.v))
        oracle.kv_write(op, 0, 0, ch.k, ch.v, ch.slots)
        ro, rl = oracle.prefill(op, 0, 0, ch.q, ch.cu_q_lens, case.page_table, ch.seq_lens)
        check(f"extend/c{chunk}/s{start}/{ci}", "bf16", out_a, ro, rl, lse_a)
