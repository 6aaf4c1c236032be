"""One decode step over several (plane, layer) banks: paged_decode_step in one
host call, and the same step captured once as a graph and replayed.

Both must equal the per-call path bit for bit (outputs, lse and the pool
bytes the fused append writes), and the per-call path must match the oracle.
Graph replays are checked one by one, with eager work and synchronisations
between them, and after the inputs' contents change."""
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
    pkv.lib()  # loud failure if the library is missing
    yield
    torch.cuda.synchronize()

# a packed recurrent-depth step: plane 0 runs layers 0..3, planes 1 and 2
# only the recurrent layers 1..2, in model order
ORDER = [(0, 0)] + [(t, l) for t in range(3) for l in (1, 2)] + [(0, 3)]


def _case(seed, batch, seq_range, hq, hkv):
    return synth.make_decode_case(seed, "bf16", batch, seq_range, hq, hkv, 128, num_planes=3,
                                  num_layers=4, rec_first=1, rec_count=2, planes_layers=ORDER)


def _fresh(case):
    import torch

    gp = gpu_pool(case.layout)
    for pl in ORDER:
        bd = case.banks[pl]
        write(gp, pl[0], pl[1], bd.fill_k, bd.fill_v, bd.fill_slots, "bf16")
    torch.cuda.synchronize()
    return gp


def _inputs(case):
    import torch

    q = torch.stack([to_dev(case.banks[pl].q, "bf16") for pl in ORDER])
    nk = torch.stack([to_dev(case.banks[pl].new_k, "bf16") for pl in ORDER])
    nv = torch.stack([to_dev(case.banks[pl].new_v, "bf16") for pl in ORDER])
    return q, nk, nv


def _buffers(case):
    import torch

    n, B, Hq = len(ORDER), case.batch, case.num_q_heads
    out = torch.zeros((n, B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((n, B, Hq), dtype=torch.float32, device="cuda")
    return out, lse


@pytest.mark.parametrize("shape", [(64, (1, 400), 16, 8), (16, (200, 900), 32, 32),
                                   (8, (300, 5000), 64, 8)])
def test_step_and_graph_equal_per_call(shape):
    import torch

    batch, rng_, hq, hkv = shape
    case = _case(3, batch, rng_, hq, hkv)
    q, nk, nv = _inputs(case)
    table, seq = i32_dev(case.page_table), i32_dev(case.seq_lens)
    mx = int(case.seq_lens.max())
    say(f"step shape={shape} mode={pkv.split_mode(gpu_pool(case.layout), batch, hq, mx)}")

    # per call
    gp_a = _fresh(case)
    out_a, lse_a = _buffers(case)
    for i, (p, l) in enumerate(ORDER):
        pkv.decode(gp_a, p, l, q[i], table, seq, mx, out=out_a[i], lse=lse_a[i], k_new=nk[i],
                   v_new=nv[i])
    torch.cuda.synchronize()
    # the oracle, call by call, on its own pool
    op = oracle_pool(case.layout)
    for i, pl in enumerate(ORDER):
        bd = case.banks[pl]
        oracle.kv_write(op, pl[0], pl[1], bd.fill_k, bd.fill_v, bd.fill_slots)
        oracle.kv_write(op, pl[0], pl[1], bd.new_k, bd.new_v, bd.new_slots)
        ro, rl = oracle.decode(op, pl[0], pl[1], bd.q, case.page_table, case.seq_lens)
        check(f"step/{pl}", "bf16", out_a[i], ro, rl, lse_a[i])

    # one host call
    gp_b = _fresh(case)
    out_b, lse_b = _buffers(case)
    pkv.decode_step(gp_b, ORDER, q, table, seq, mx, out_b, lse_b, k_new=nk, v_new=nv)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_a), bits(out_b)) and np.array_equal(bits(lse_a), bits(lse_b))
    assert np.array_equal(bits(gp_a.k), bits(gp_b.k)) and np.array_equal(bits(gp_a.v), bits(gp_b.v))

    # captured once, replayed; nothing runs at capture
    gp_c = _fresh(case)
    out_c, lse_c = _buffers(case)
    g = pkv.StepGraph(gp_c, ORDER, q, table, seq, mx, out_c, lse_c, k_new=nk, v_new=nv)
    torch.cuda.synchronize()
    assert not bits(out_c).any()
    scratch = torch.empty(1 << 20, device="cuda")
    for rep in range(3):
        out_c.zero_()
        lse_c.zero_()
        scratch.normal_()  # eager work between replays
        float(scratch.sum())
        g.launch()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out_a), bits(out_c)), rep
        assert np.array_equal(bits(lse_a), bits(lse_c)), rep
        assert np.array_equal(bits(gp_a.k), bits(gp_c.k)) and np.array_equal(bits(gp_a.v),
                                                                               bits(gp_c.v))
    # replays read the buffers' contents at replay time
    q2 = q.clone()
    q.mul_(-1.0)
    g.launch()
    torch.cuda.synchronize()
    for i, (p, l) in enumerate(ORDER):
        pkv.decode(gp_a, p, l, q[i], table, seq, mx, out=out_a[i], lse=lse_a[i], k_new=nk[i],
                   v_new=nv[i])
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_a), bits(out_c)) and np.array_equal(bits(lse_a), bits(lse_c))
    assert not np.array_equal(bits(q), bits(q2))
    g.close()
