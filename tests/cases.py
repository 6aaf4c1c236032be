"""Small helpers shared by the tests: build oracle pools from synthetic cases."""
from __future__ import annotations

import numpy as np

import oracle
from paged_kv_attention_kvcache_amd import synth


def oracle_pool(layout: synth.Layout) -> "oracle.Pool":
    bank_of, nb = oracle.bank_map(layout.num_planes, layout.num_layers,
                                  layout.rec_first, layout.rec_count)
    return oracle.Pool(layout.dtype, layout.page_size, layout.num_pages,
                       layout.num_kv_heads, layout.head_dim, bank_of, nb,
                       fill=synth.poison_value(layout.dtype))


def oracle_decode_case(case: synth.DecodeCase, plane=0, layer=0, pool=None, scale=None):
    """Write context + new token through the oracle's store_kv, then decode."""
    pool = pool if pool is not None else oracle_pool(case.layout)
    bd = case.banks[(plane, layer)]
    oracle.kv_write(pool, plane, layer, bd.fill_k, bd.fill_v, bd.fill_slots)
    oracle.kv_write(pool, plane, layer, bd.new_k, bd.new_v, bd.new_slots)
    out, lse = oracle.decode(pool, plane, layer, bd.q, case.page_table, case.seq_lens, scale)
    return out, lse, pool


def oracle_prefill_chunks(case: synth.PrefillCase, chunks, pool=None, plane=0, layer=0,
                          scale=None):
    """Run a chunk schedule (write then attend per chunk) on the oracle.

    Returns per-request outputs [n_r rows attended, Hq, D] and lse, keyed by
    position, assembled from the chunks."""
    pool = pool if pool is not None else oracle_pool(case.layout)
    B = len(case.prompt_lens)
    Hq, D = case.num_q_heads, case.layout.head_dim
    outs = [dict() for _ in range(B)]
    for ch in chunks:
        oracle.kv_write(pool, plane, layer, ch.k, ch.v, ch.slots)
        o, l = oracle.prefill(pool, plane, layer, ch.q, ch.cu_q_lens, case.page_table,
                              ch.seq_lens, scale)
        for i, (r, lo) in enumerate(ch.rows):
            for j in range(ch.cu_q_lens[i + 1] - ch.cu_q_lens[i]):
                row = ch.cu_q_lens[i] + j
                outs[r][lo + j] = (o[row], l[row])
    return outs, pool


def stack_rows(outs_r: dict, positions):
    o = np.stack([outs_r[p][0] for p in positions])
    l = np.stack([outs_r[p][1] for p in positions])
    return o, l
