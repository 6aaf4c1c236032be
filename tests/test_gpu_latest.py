"""Early-exit ("latest bank") decode on the GPU against the oracle ("Faster
fuzzy minds", section "Can we actually stop early?"): position pos is read
from plane min(query plane, exit depth of pos) of the same layer.

Covered: every plane of a packed recurrent layer, groups 1, 2 (vector
folds), 4 and 8 (matrix-core fold; fp32 and head_dim 64 take the vector
fold), bf16 and fp32, the whole-context, balanced, fixed-partition and
per-partition-block splits; bitwise equalities with the ordinary decode when
no token exits before the query's plane (including depth bytes past the
plane or negative, which read the query's plane), and of the fused append
with a write followed by the early-exit decode."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import paged_kv_attention_kvcache_amd as pkv
from paged_kv_attention_kvcache_amd import synth

from cases import oracle_pool
from gpu_util import bits, check, gpu_pool, i32_dev, say, to_dev, write

pytestmark = pytest.mark.gpu

PLANES = 5


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    pkv.lib()
    yield
    torch.cuda.synchronize()


def setup(seed, dtype, batch, seq_range, hq, hkv, D):
    """Layer 1 of a packed 3-layer map (plane 0 holds 0..2, deeper planes 1..2)
    filled on every plane, on the oracle and on the GPU."""
    import torch

    order = [(p, 1) for p in range(PLANES)]
    case = synth.make_decode_case(seed, dtype, batch, seq_range, hq, hkv, D, num_planes=PLANES,
                                  num_layers=3, rec_first=1, rec_count=2, planes_layers=order)
    op = oracle_pool(case.layout)
    gp = gpu_pool(case.layout)
    for pl in order:
        bd = case.banks[pl]
        for pool, wr in ((op, oracle.kv_write), (gp, None)):
            if wr:
                wr(pool, *pl, bd.fill_k, bd.fill_v, bd.fill_slots)
                wr(pool, *pl, bd.new_k, bd.new_v, bd.new_slots)
            else:
                write(pool, *pl, bd.fill_k, bd.fill_v, bd.fill_slots, dtype)
                write(pool, *pl, bd.new_k, bd.new_v, bd.new_slots, dtype)
    torch.cuda.synchronize()
    stride = (int(case.seq_lens.max()) + 15) // 16 * 16 + 16
    return case, op, gp, stride


def depth_dev(depth: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(depth, dtype=np.int8)).cuda()


CASES = {
    "g1_whole": ("bf16", 16, (1, 600), 32, 32, 128, 0),     # 512 units: whole contexts
    "g2_whole": ("bf16", 64, (1, 300), 16, 8, 128, 0),      # persistent whole contexts
    "g1_balanced": ("bf16", 3, (100, 3000), 4, 4, 128, 0),  # balanced split + combine
    "g2_fixed": ("bf16", 5, (1, 700), 4, 2, 128, 64),       # fixed partitions of 64
    "f32_g2": ("f32", 4, (17, 64), 4, 2, 64, 0),            # tiny fp32 decode shape
    "g4_whole": ("bf16", 16, (1, 600), 16, 4, 128, 0),      # matrix-core fold, whole
    "g8_balanced": ("bf16", 3, (100, 3000), 16, 2, 128, 0),  # matrix-core fold, balanced
    "g8_fixed": ("bf16", 5, (1, 700), 16, 2, 128, 64),      # fixed partitions of 64
    "g4_block48": ("bf16", 5, (1, 700), 8, 2, 128, 48),     # 3-page partitions: block kernel
    "f32_g4": ("f32", 4, (17, 300), 8, 2, 64, 0),           # vector fold of group 4
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_latest_matches_oracle(name):
    dtype, batch, rng_, hq, hkv, D, partition = CASES[name]
    case, op, gp, stride = setup(1, dtype, batch, rng_, hq, hkv, D)
    table, seq = i32_dev(case.page_table), i32_dev(case.seq_lens)
    mx = int(case.seq_lens.max())
    depth = np.random.default_rng(2).integers(0, PLANES, size=(batch, stride)).astype(np.int8)
    ed = depth_dev(depth)
    for p in range(PLANES):
        say(f"latest {name} plane={p} mode={pkv.split_mode(gp, batch, hq, mx, partition)}")
        q = case.banks[(p, 1)].q
        ro, rl = oracle.decode_latest(op, p, 1, depth, q, case.page_table, case.seq_lens)
        out, lse = pkv.decode_latest(gp, p, 1, ed, to_dev(q, dtype), table, seq, mx,
                                     partition=partition)
        check(f"latest/{name}/plane{p}", dtype, out, ro, rl, lse)


@pytest.mark.parametrize("hq,hkv", [(16, 4), (16, 2)])
def test_latest_bitwise_no_exit_groups(hq, hkv):
    # matrix-core fold: with no token exiting before the query's plane the
    # early-exit decode is the ordinary decode, bit for bit
    import torch

    case, op, gp, stride = setup(5, "bf16", 8, (1, 700), hq, hkv, 128)
    table, seq = i32_dev(case.page_table), i32_dev(case.seq_lens)
    mx = int(case.seq_lens.max())
    rng = np.random.default_rng(6)
    for p in (0, PLANES - 1):
        q = to_dev(case.banks[(p, 1)].q, "bf16")
        deep = rng.integers(p, 128, size=(case.batch, stride)).astype(np.int8)
        deep[:, ::5] = -3
        for partition in (0, 64):
            say(f"latest no-exit hq={hq} hkv={hkv} plane={p} partition={partition}")
            a, la = pkv.decode_latest(gp, p, 1, depth_dev(deep), q, table, seq, mx,
                                      partition=partition)
            b, lb = pkv.decode(gp, p, 1, q, table, seq, mx, partition=partition)
            torch.cuda.synchronize()
            assert np.array_equal(bits(a), bits(b)) and np.array_equal(bits(la), bits(lb))


def test_latest_bitwise_equalities():
    import torch

    case, op, gp, stride = setup(3, "bf16", 16, (1, 500), 32, 32, 128)
    table, seq = i32_dev(case.page_table), i32_dev(case.seq_lens)
    mx = int(case.seq_lens.max())
    B = case.batch
    rng = np.random.default_rng(4)
    for p in range(PLANES):
        q = to_dev(case.banks[(p, 1)].q, "bf16")
        # nobody exits before plane p: bytes p..127 and negative ones all read plane p
        deep = rng.integers(p, 128, size=(B, stride)).astype(np.int8)
        deep[:, ::7] = -1
        a, la = pkv.decode_latest(gp, p, 1, depth_dev(deep), q, table, seq, mx)
        b, lb = pkv.decode(gp, p, 1, q, table, seq, mx)
        torch.cuda.synchronize()
        assert np.array_equal(bits(a), bits(b)) and np.array_equal(bits(la), bits(lb)), p
    # fused append == write of the newest token + early-exit decode (the
    # newest token is computed at the query's plane, so its depth reaches it)
    depth = rng.integers(0, PLANES, size=(B, stride)).astype(np.int8)
    p = PLANES - 1
    depth[np.arange(B), case.seq_lens - 1] = p
    ed = depth_dev(depth)
    bd = case.banks[(p, 1)]
    nk, nv = rng.standard_normal(bd.new_k.shape), rng.standard_normal(bd.new_v.shape)
    nk = to_dev(synth.bf16_bits(nk.astype(np.float32)), "bf16")
    nv = to_dev(synth.bf16_bits(nv.astype(np.float32)), "bf16")
    q = to_dev(bd.q, "bf16")
    k0, v0 = gp.k.clone(), gp.v.clone()
    a, la = pkv.decode_latest(gp, p, 1, ed, q, table, seq, mx, k_new=nk, v_new=nv)
    ka, va = gp.k.clone(), gp.v.clone()
    gp.k.copy_(k0)
    gp.v.copy_(v0)
    pkv.kv_write(gp, p, 1, nk, nv, i32_dev(bd.new_slots))
    b, lb = pkv.decode_latest(gp, p, 1, ed, q, table, seq, mx)
    torch.cuda.synchronize()
    assert np.array_equal(bits(ka), bits(gp.k)) and np.array_equal(bits(va), bits(gp.v))
    assert np.array_equal(bits(a), bits(b)) and np.array_equal(bits(la), bits(lb))
