"""Pins for the oracle's early-exit decode ("Faster fuzzy minds", section "Can
we actually stop early?": a token that halted at depth e keeps its KV of
depth e, and a later token attending at depth p reads it from the latest
bank it has, min(p, e)).

* brute force: per-plane logical K/V are drawn for each request; the context
  a plane-p query sees is built here by picking, position by position, the
  rows of plane min(p, e[pos]) -- before any paging -- and dense attention
  over it must equal the oracle within 1e-12;
* special cases: exit depths at or past the query's plane reduce to the
  ordinary decode of that plane, and all-zero depths to decode on plane 0
  (both exactly);
* errors: a depth outside the pool's planes, and a source plane that does
  not hold the layer, are rejected.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import brute
import oracle
from cases import oracle_pool
from paged_kv_attention_kvcache_amd import synth


def latest_case(seed, dtype, batch, seq_range, hq, hkv, D, planes, layer_rec=(1, 2)):
    """A packed pool: plane 0 holds layers 0..2, planes >= 1 layers 1..2; all
    planes of layer 1 are filled; returns the case and per-plane bank data."""
    order = [(p, 1) for p in range(planes)]
    case = synth.make_decode_case(seed, dtype, batch, seq_range, hq, hkv, D, num_planes=planes,
                                  num_layers=3, rec_first=layer_rec[0], rec_count=layer_rec[1],
                                  planes_layers=order)
    pool = oracle_pool(case.layout)
    for pl in order:
        bd = case.banks[pl]
        oracle.kv_write(pool, *pl, bd.fill_k, bd.fill_v, bd.fill_slots)
        oracle.kv_write(pool, *pl, bd.new_k, bd.new_v, bd.new_slots)
    return case, pool


@pytest.mark.parametrize("dtype,hq,hkv,D", [("bf16", 4, 4, 64), ("f32", 8, 2, 32),
                                            ("bf16", 2, 1, 128)])
def test_latest_matches_brute_force(dtype, hq, hkv, D):
    planes = 5
    case, pool = latest_case(2, dtype, 4, (1, 80), hq, hkv, D, planes)
    rng = np.random.default_rng(9)
    stride = int(case.seq_lens.max()) + 3
    depth = rng.integers(0, planes, size=(case.batch, stride)).astype(np.int8)
    scale = 1 / math.sqrt(D)
    for p in range(planes):
        q = case.banks[(p, 1)].q
        o, l = oracle.decode_latest(pool, p, 1, depth, q, case.page_table, case.seq_lens)
        for r in range(case.batch):
            n = int(case.seq_lens[r])
            src = np.minimum(depth[r, :n], p)
            lk = np.stack([case.banks[(int(src[t]), 1)].logical_k[r][t] for t in range(n)])
            lv = np.stack([case.banks[(int(src[t]), 1)].logical_v[r][t] for t in range(n)])
            bo, bl = brute.attention(q[r:r + 1], lk, lv, np.array([n - 1]), scale)
            assert np.max(np.abs(o[r] - bo[0])) < 1e-12
            assert np.max(np.abs(l[r] - bl[0])) < 1e-12


def test_latest_special_cases():
    planes = 4
    case, pool = latest_case(3, "bf16", 3, (1, 60), 4, 2, 64, planes)
    stride = int(case.seq_lens.max())
    for p in range(planes):
        q = case.banks[(p, 1)].q
        deep = np.full((case.batch, stride), planes - 1, np.int8)
        o, l = oracle.decode_latest(pool, p, 1, deep, q, case.page_table, case.seq_lens)
        ro, rl = oracle.decode(pool, p, 1, q, case.page_table, case.seq_lens)
        assert np.array_equal(o, ro) and np.array_equal(l, rl)
        zero = np.zeros((case.batch, stride), np.int8)
        o, l = oracle.decode_latest(pool, p, 1, zero, q, case.page_table, case.seq_lens)
        ro, rl = oracle.decode(pool, 0, 1, q, case.page_table, case.seq_lens)
        assert np.array_equal(o, ro) and np.array_equal(l, rl)


def test_latest_rejects():
    planes = 3
    case, pool = latest_case(4, "f32", 2, (5, 20), 2, 2, 16, planes)
    stride = int(case.seq_lens.max())
    q = case.banks[(2, 1)].q
    bad = np.full((case.batch, stride), planes, np.int8)
    with pytest.raises(oracle.OracleError) as e:
        oracle.decode_latest(pool, 2, 1, bad, q, case.page_table, case.seq_lens)
    assert e.value.code == oracle.ORC_EINVAL
    # a map where plane 1 does not hold layer 1 but plane 2 does
    bank_of = pool.bank_of.copy()
    bank_of[1, 1] = -1
    pool2 = oracle.Pool(pool.dtype, pool.page_size, pool.num_pages, pool.num_kv_heads,
                        pool.head_dim, bank_of, pool.num_banks, pool.k, pool.v)
    one = np.ones((case.batch, stride), np.int8)
    with pytest.raises(oracle.OracleError) as e:
        oracle.decode_latest(pool2, 2, 1, one, q, case.page_table, case.seq_lens)
    assert e.value.code == oracle.ORC_ENOTHELD
