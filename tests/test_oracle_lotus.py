"""Pins for the oracle's LOTUS loop ("Faster fuzzy minds", section "LOTUS"):
the block's slots are handed to store_kv on every pass, so each pass
overwrites the previous one in place, and each pass is one extend-prefill of
the whole block.

Checked without trusting the oracle: the pool bytes at the block's slots
after pass i are pass i's K/V (gathered by plain slot arithmetic); the prompt
bytes are untouched; pass i's attention equals brute-force dense attention
over the prompt's logical K/V followed by pass i's block K/V, and differs
from the same with pass i-1's block (so a loop that did not overwrite would
fail)."""
from __future__ import annotations

import numpy as np
import pytest

import brute
import oracle
from cases import oracle_pool
from paged_kv_attention_kvcache_amd import synth


def gather(pool: oracle.Pool, bank: int, slots: np.ndarray):
    P = pool.page_size
    return pool.k[bank, slots // P, :, slots % P, :], pool.v[bank, slots // P, :, slots % P, :]


@pytest.mark.parametrize("dtype,hq,hkv,D,block", [("bf16", 4, 2, 64, 16), ("f32", 2, 2, 64, 5),
                                                  ("bf16", 8, 1, 128, 40)])
def test_lotus_loop_overwrites_and_attends_its_own_pass(dtype, hq, hkv, D, block):
    prompts = [37, 16, 70]
    case = synth.make_lotus_case(4, dtype, prompts, block, 3, hq, hkv, D)
    pool = oracle_pool(case.layout)
    bank = int(pool.bank_of[0, 0])
    pk = np.concatenate(case.prompt_k)
    pv = np.concatenate(case.prompt_v)
    oracle.kv_write(pool, 0, 0, pk, pv, case.prompt_slots)
    B = len(prompts)
    cu = np.arange(B + 1, dtype=np.int32) * block
    seq = np.asarray(prompts, np.int32) + block
    scale = 1.0 / np.sqrt(D)
    seen = []

    def after(i):
        k, v = gather(pool, bank, case.block_slots)
        assert np.array_equal(k, case.passes[i][0]) and np.array_equal(v, case.passes[i][1])
        k, v = gather(pool, bank, case.prompt_slots)
        assert np.array_equal(k, pk) and np.array_equal(v, pv)
        seen.append(i)

    res = oracle.lotus_loop(pool, 0, 0, case.passes, case.block_slots, cu, case.page_table, seq,
                            scale, after_pass=after)
    assert seen == [0, 1, 2]
    for i, (out, lse) in enumerate(res):
        k, v, q = case.passes[i]
        for r, n in enumerate(prompts):
            rows = slice(r * block, (r + 1) * block)
            lk = np.concatenate([case.prompt_k[r], k[rows]])
            lv = np.concatenate([case.prompt_v[r], v[rows]])
            bo, bl = brute.attention(q[rows], lk, lv, n + np.arange(block), scale)
            assert np.max(np.abs(out[rows] - bo)) < 1e-12
            assert np.max(np.abs(lse[rows] - bl)) < 1e-12
            if i > 0:  # the previous pass's block would give another answer
                pk_, pv_ = case.passes[i - 1][0], case.passes[i - 1][1]
                so, _ = brute.attention(q[rows], np.concatenate([case.prompt_k[r], pk_[rows]]),
                                        np.concatenate([case.prompt_v[r], pv_[rows]]),
                                        n + np.arange(block), scale)
                assert np.max(np.abs(out[rows] - so)) > 1e-3
