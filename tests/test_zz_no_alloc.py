"""The allocation-free decode entry point (paged_decode_attn_noalloc) through
the C-ABI, against paged_decode_attn with a workspace of its own.

Two calls in a row per split mode, the second smaller than the first: each
must give the same bits (out and lse) as the workspace path on the same
inputs, which is the parity bar and more, and both stay within the fp64
oracle's bar. The modes covered are the ones that keep split-K partials
(balanced split, fixed partitions on the streamed grid and on the
per-partition grid with its reduction)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from cases import oracle_decode_case
from gpu_util import bits, check, gpu_pool, i32_dev, to_dev, write
import paged_kv_attention_kvcache_amd as pkv
from paged_kv_attention_kvcache_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    pkv.lib()
    yield
    torch.cuda.synchronize()


# (tag, generator arguments of the first call, of the second call, partition, split mode)
CASES = [
    ("balanced_gqa8", dict(dtype="bf16", batch=6, seq_range=(2000, 9000), num_q_heads=64,
                           num_kv_heads=8, head_dim=128),
     dict(dtype="bf16", batch=3, seq_range=(300, 1500), num_q_heads=64, num_kv_heads=8,
          head_dim=128), 0, "balanced"),
    ("balanced_mha", dict(dtype="bf16", batch=5, seq_range=(400, 3000), num_q_heads=32,
                          num_kv_heads=32, head_dim=128, alias_frac=0.78),
     dict(dtype="bf16", batch=2, seq_range=(260, 700), num_q_heads=32, num_kv_heads=32,
          head_dim=128), 0, "balanced"),
    ("fixed512_gqa8", dict(dtype="bf16", batch=7, seq_range=(1000, 5000), num_q_heads=64,
                           num_kv_heads=8, head_dim=128),
     dict(dtype="bf16", batch=3, seq_range=(100, 1200), num_q_heads=64, num_kv_heads=8,
          head_dim=128), 512, "fixed"),
    ("fixed48_f32", dict(dtype="f32", batch=5, seq_range=(100, 900), num_q_heads=4,
                         num_kv_heads=2, head_dim=64),
     dict(dtype="f32", batch=2, seq_range=(17, 200), num_q_heads=4, num_kv_heads=2,
          head_dim=64), 48, "fixed"),
]


def run_pair(case, partition):
    """The same inputs through both entry points; returns both results."""
    import torch

    dt = case.layout.dtype
    pool = gpu_pool(case.layout)
    bd = case.banks[(0, 0)]
    write(pool, 0, 0, bd.fill_k, bd.fill_v, bd.fill_slots, dt)
    write(pool, 0, 0, bd.new_k, bd.new_v, bd.new_slots, dt)
    q = to_dev(bd.q, dt)
    table, seq = i32_dev(case.page_table), i32_dev(case.seq_lens)
    mx = int(case.seq_lens.max())
    B, Hq, D = q.shape
    out_n = torch.empty_like(q)
    lse_n = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    pkv.decode_noalloc(pool, 0, 0, q, table, seq, mx, out_n, lse_n, partition=partition)
    out_w, lse_w = pkv.decode(pool, 0, 0, q, table, seq, mx, partition=partition)
    torch.cuda.synchronize()
    return pool, (out_n, lse_n), (out_w, lse_w)


@pytest.mark.parametrize("tag,first,second,partition,mode", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_path(tag, first, second, partition, mode):
    for i, kw in enumerate((first, second)):
        case = synth.make_decode_case(10 + i, **kw)
        print(f"[{tag}] call {i}: batch {kw['batch']}, seq_lens {case.seq_lens.tolist()}, "
              f"partition {partition}", file=sys.stderr, flush=True)
        pool, (on, ln), (ow, lw) = run_pair(case, partition)
        assert pkv.split_mode(pool, kw["batch"], kw["num_q_heads"], int(case.seq_lens.max()),
                              partition) == mode
        assert pkv.workspace_bytes(pool, kw["batch"], kw["num_q_heads"],
                                   int(case.seq_lens.max()), partition) <= pkv.SCRATCH_BYTES
        assert np.array_equal(bits(on), bits(ow)), f"{tag} call {i}: out differs"
        assert np.array_equal(bits(ln), bits(lw)), f"{tag} call {i}: lse differs"
        ro, rl, _ = oracle_decode_case(case)
        check(f"{tag} call {i}", kw["dtype"], on, ro, rl, ln)
