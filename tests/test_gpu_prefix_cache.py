"""A prefix-cache hit end to end on the GPU: the host page manager
(pkv_mgr_*) feeding the kernels.

The flow follows vllm-rlt pull 152, section "Summary" (a request's pages are
published as a reusable prefix only once every layer that each plane in use
holds has written them; with Huginn's packed map plane 0 holds all 8 layers
and deeper planes the 4 recurrent ones) and "Faster fuzzy minds", section
"When scheduler does the work" (a request that hits the cache inherits the
prefix's KV and only its suffix is prefilled):

1. request A allocates its pages and store_kv writes its prompt into every
   held (plane, layer), noted in the manager; publication is checked to wait
   for the last held layer of the deepest plane;
2. request B aliases A's published pages (retain), allocates pages for its
   own suffix, writes the suffix and prefills only it, then runs one decode
   step on several planes -- all through B's page table, compared element by
   element with the fp64 oracle on the same writes;
3. releasing B frees exactly its own pages and leaves A's pages held once.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from gpu_util import check, gpu_pool, i32_dev, to_dev, write
import paged_kv_attention_kvcache_amd as pkv
from paged_kv_attention_kvcache_amd import synth

pytestmark = pytest.mark.gpu

P = 16
PLANES, LAYERS, REC_FIRST, REC_COUNT = 3, 8, 2, 4  # Huginn's packed map, three planes
HKV, D = 8, 128  # MHA


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    pkv.lib()
    yield
    torch.cuda.synchronize()


def held(bank_of):
    return [(p, l) for p in range(PLANES) for l in range(LAYERS) if bank_of[p, l] >= 0]


@pytest.mark.parametrize("prompt_a,suffix_b", [(200, 40), (517, 131)])
def test_prefix_cache_hit(prompt_a, suffix_b):
    import torch

    rng = np.random.default_rng(prompt_a)
    layout = synth.Layout(dtype="bf16", page_size=P, num_pages=64, num_kv_heads=HKV, head_dim=D,
                          num_planes=PLANES, num_layers=LAYERS, rec_first=REC_FIRST,
                          rec_count=REC_COUNT)
    bank_of, nb = pkv.bank_map(PLANES, LAYERS, REC_FIRST, REC_COUNT)
    gp = gpu_pool(layout)
    op = oracle.Pool("bf16", P, 64, HKV, D, bank_of, nb, fill=synth.poison_value("bf16"))
    mgr = pkv.PageManager(64, bank_of)
    free0 = mgr.free_count()
    print(f"prefix cache: prompt {prompt_a}, suffix {suffix_b}", file=sys.stderr, flush=True)

    # 1. Request A: pages, prompt written in every held (plane, layer).
    pages_a = mgr.alloc(-(-prompt_a // P))
    table_a = pages_a[None, :]
    slots_a = synth.slots_of(table_a, 0, np.arange(prompt_a), P)
    order = held(bank_of)
    for i, (p, l) in enumerate(order):
        k = synth.draw(rng, (prompt_a, HKV, D), "bf16")
        v = synth.draw(rng, (prompt_a, HKV, D), "bf16")
        write(gp, p, l, k, v, slots_a, "bf16")
        oracle.kv_write(op, p, l, k, v, slots_a)
        mgr.note_write(p, l, slots_a)
        if i == len(order) - 2:  # the deepest plane's last held layer is still missing
            assert mgr.published_prefix(PLANES, pages_a) == 0
            assert mgr.published_prefix(PLANES - 1, pages_a) == prompt_a // P
    published = mgr.published_prefix(PLANES, pages_a)
    assert published == prompt_a // P  # every full page; the partial last page never
    shared = pages_a[:published]

    # 2. Request B: the published prefix aliased, its own suffix allocated.
    mgr.retain(shared)
    prefix = published * P
    n_b = prefix + suffix_b
    own = mgr.alloc(-(-(n_b + 1) // P) - published)  # + room for one decode token
    table_b = np.concatenate([shared, own])[None, :].astype(np.int32)
    assert all(mgr.refcount(int(p)) == 2 for p in shared)
    slots_b = synth.slots_of(table_b, 0, np.arange(prefix, n_b), P)
    cu = np.array([0, suffix_b], np.int32)
    seq = np.array([n_b], np.int32)
    checked = [(0, 0), (0, 3), (1, 2), (2, 5), (0, 7)]
    for p, l in order:
        k = synth.draw(rng, (suffix_b, HKV, D), "bf16")
        v = synth.draw(rng, (suffix_b, HKV, D), "bf16")
        write(gp, p, l, k, v, slots_b, "bf16")
        oracle.kv_write(op, p, l, k, v, slots_b)
        mgr.note_write(p, l, slots_b)
        if (p, l) not in checked:
            continue
        q = synth.draw(rng, (suffix_b, HKV, D), "bf16")
        out, lse = pkv.prefill(gp, p, l, to_dev(q, "bf16"), i32_dev(cu), i32_dev(table_b),
                               i32_dev(seq), suffix_b, n_b)
        ro, rl = oracle.prefill(op, p, l, q, cu, table_b, seq)
        torch.cuda.synchronize()
        check(f"suffix prefill plane {p} layer {l}", "bf16", out, ro, rl, lse)

    # One decode step of B on every checked bank: the newest token appended
    # (fused store_kv) and attended over the aliased prefix and the suffix.
    seq_d = np.array([n_b + 1], np.int32)
    new_slot = synth.slots_of(table_b, 0, np.array([n_b]), P)
    for p, l in checked:
        k = synth.draw(rng, (1, HKV, D), "bf16")
        v = synth.draw(rng, (1, HKV, D), "bf16")
        q = synth.draw(rng, (1, HKV, D), "bf16")
        out, lse = pkv.decode(gp, p, l, to_dev(q, "bf16"), i32_dev(table_b), i32_dev(seq_d),
                              n_b + 1, k_new=to_dev(k, "bf16"), v_new=to_dev(v, "bf16"))
        oracle.kv_write(op, p, l, k, v, new_slot)
        ro, rl = oracle.decode(op, p, l, q, table_b, seq_d)
        torch.cuda.synchronize()
        check(f"decode plane {p} layer {l}", "bf16", out, ro, rl, lse)
        mgr.note_write(p, l, new_slot)

    # The GPU pool holds exactly the oracle's bytes after all of it.
    ib = torch.int16
    assert np.array_equal(gp.k.view(ib).cpu().numpy().view(np.uint16), op.k)
    assert np.array_equal(gp.v.view(ib).cpu().numpy().view(np.uint16), op.v)

    # 3. Release B: its own pages are free again, A's are held once.
    before = mgr.free_count()
    mgr.release(table_b[0])
    assert mgr.free_count() == before + len(own)
    assert all(mgr.refcount(int(p)) == 1 for p in pages_a)
    assert all(mgr.refcount(int(p)) == 0 for p in own)
    mgr.release(pages_a)
    assert mgr.free_count() == free0
    mgr.close()
