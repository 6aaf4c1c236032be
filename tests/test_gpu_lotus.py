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
