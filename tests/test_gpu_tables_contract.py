"""Device-resident tables outside their contract stay inside the buffers.

The header promises that values outside the contract of page_table,
slot_mapping, seq_lens and cu_q_lens give unspecified results but no access
outside the buffers it describes: the kernels clamp every index they derive
from those tables. Here each entry point runs on tables holding negative,
oversized and unordered values. Every call must complete; calls that write
nothing by contract (decode without append, prefill) must leave the pool
bytes unchanged, and a write whose slots are all out of range writes nothing."""
from __future__ import annotations

import numpy as np
import pytest

import paged_kv_attention_kvcache_amd as pkv
from paged_kv_attention_kvcache_amd import synth

from gpu_util import bits, gpu_pool, i32_dev, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    pkv.lib()
    yield
    torch.cuda.synchronize()


def _bad_table(rng, batch, stride, num_pages):
    t = rng.integers(0, num_pages, size=(batch, stride)).astype(np.int64)
    t[:, ::3] = -rng.integers(1, 1 << 30, size=t[:, ::3].shape)
    t[:, 1::5] = num_pages + rng.integers(0, 1 << 30, size=t[:, 1::5].shape)
    return t.astype(np.int32)


@pytest.mark.parametrize("mode,hq", [("whole", 16), ("balanced", 16), ("fixed", 16),
                                     ("fixed", 64), ("fixed48", 64)])
def test_decode_tables_out_of_contract(mode, hq):
    # fixed with group 2 (vector fold) and group 8 (matrix-core fold) take the
    # streamed fixed partitions; 48-token partitions with group 8 take one
    # workgroup per partition
    import torch

    rng = np.random.default_rng(41)
    layout = synth.Layout("bf16", 16, 96, 8, 128)
    pool = gpu_pool(layout, poison=False)
    before = (bits(pool.k), bits(pool.v))
    batch = 64 if mode == "whole" else 6
    max_seq, stride = 512, 32
    seq = rng.integers(-(1 << 30), 1 << 30, size=batch).astype(np.int32)
    seq[::4] = rng.integers(0, max_seq + 1, size=seq[::4].shape)
    table = _bad_table(rng, batch, stride, layout.num_pages)
    q = to_dev(synth.draw(rng, (batch, hq, 128), "bf16"), "bf16")
    partition = {"fixed": 64, "fixed48": 48}.get(mode, 0)
    say(f"decode out-of-contract tables, {mode} hq={hq}: "
        f"{pkv.split_mode(pool, batch, hq, max_seq, partition)}")
    out, lse = pkv.decode(pool, 0, 0, q, i32_dev(table), i32_dev(seq), max_seq,
                          partition=partition)
    torch.cuda.synchronize()
    assert np.array_equal(bits(pool.k), before[0]) and np.array_equal(bits(pool.v), before[1])
    assert out.shape == (batch, hq, 128) and lse.shape == (batch, hq)


@pytest.mark.parametrize("dtype,D,max_q", [("bf16", 128, 256), ("f32", 64, 256),
                                           ("bf16", 128, 8)])
def test_prefill_tables_out_of_contract(dtype, D, max_q):
    # max_q 8 with a group of 2: the 16-column short-chunk kernel
    import torch

    rng = np.random.default_rng(43)
    layout = synth.Layout(dtype, 16, 64, 4, D)
    pool = gpu_pool(layout, poison=False)
    before = (bits(pool.k), bits(pool.v))
    batch, total_q, max_seq, stride = 5, 200, 400, 25
    cu = np.array([0, 150, 40, -7, 1 << 30, total_q + 60], np.int32)
    seq = np.array([300, -5, 1 << 30, 17, 400], np.int32)
    table = _bad_table(rng, batch, stride, layout.num_pages)
    q = to_dev(synth.draw(rng, (total_q, 8, D), dtype), dtype)
    say(f"prefill out-of-contract tables, {dtype} D={D} max_q_len={max_q}")
    out, lse = pkv.prefill(pool, 0, 0, q, i32_dev(cu), i32_dev(table), i32_dev(seq), max_q,
                           max_seq)
    torch.cuda.synchronize()
    assert np.array_equal(bits(pool.k), before[0]) and np.array_equal(bits(pool.v), before[1])
    assert out.shape == (total_q, 8, D)


def test_kv_write_slots_out_of_range_write_nothing():
    import torch

    rng = np.random.default_rng(47)
    layout = synth.Layout("bf16", 16, 32, 8, 128)
    pool = gpu_pool(layout, poison=False)
    before = (bits(pool.k), bits(pool.v))
    n = 300
    slots = np.where(rng.random(n) < 0.5, -rng.integers(1, 1 << 30, size=n),
                     32 * 16 + rng.integers(0, 1 << 30, size=n)).astype(np.int32)
    k = to_dev(synth.draw(rng, (n, 8, 128), "bf16"), "bf16")
    v = to_dev(synth.draw(rng, (n, 8, 128), "bf16"), "bf16")
    say("kv_write with every slot out of range")
    pkv.kv_write(pool, 0, 0, k, v, i32_dev(slots))
    torch.cuda.synchronize()
    assert np.array_equal(bits(pool.k), before[0]) and np.array_equal(bits(pool.v), before[1])
