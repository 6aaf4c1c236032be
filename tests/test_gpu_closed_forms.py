"""Closed forms of attention on the GPU, at the workloads' full shapes.

Attention reaches softmax over the visible keys, so three inputs have answers
that need no oracle:
* V = 1 everywhere: the weights sum to one, so every output is exactly 1
  (in bf16, whatever the rounding of the probabilities on the way);
* K = 0 everywhere: every score is 0, the weights are uniform, the output is
  the mean of the visible V rows and lse = ln(number of visible keys);
* one visible key: the output is that key's V row, bit for bit, and lse is
  its score.
The expected values are computed here from the host copies of the inputs
(before any library kernel runs), in float64. Bounds: bf16 outputs within
half a bf16 ulp of the fp64 mean plus 5e-5 for the fp32 accumulation; lse
within 1e-5 of ln n. The decode shapes run in the launch configurations the
benchmark times (whole contexts for the Ouro and Huginn shapes, the balanced
split and fixed 512-token partitions for the long-context shape), the
prefill shapes as one cold chunk (8 x 512 and 8 x 2048 tokens, 32 heads).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest

from gpu_util import bits, full_size_pool, i32_dev, to_dev, write, gpu_pool
import paged_kv_attention_kvcache_amd as pkv
from paged_kv_attention_kvcache_amd import synth

pytestmark = pytest.mark.gpu

ONE_BF16 = 0x3F80
DECODE = {
    "ouro": dict(B=64, lo=512, hi=2048, hq=16, hkv=8, alias=0.0, kv_heads=None),
    "huginn": dict(B=16, lo=200, hi=2000, hq=32, hkv=32, alias=0.78, kv_heads=None),
    "longctx": dict(B=256, lo=8192, hi=32768, hq=64, hkv=8, alias=0.0, kv_heads=[0, 5]),
    "longctx_p512": dict(B=256, lo=8192, hi=32768, hq=64, hkv=8, alias=0.0, kv_heads=[0, 5],
                         partition=512),
}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    pkv.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_mean(tag, got_bits, want, got_lse=None, want_lse=None):
    got = bf16_f64(got_bits)
    err = np.abs(got - want)
    bound = np.abs(want) * 2.0 ** -8 + 5e-5
    worst = float((err - bound).max())
    say(f"[{tag}] max_abs={float(err.max()):.3e} worst excess over bound={worst:.3e}")
    assert (err <= bound).all(), f"{tag}: {int((err > bound).sum())} outputs off the mean"
    if got_lse is not None:
        lerr = float(np.abs(got_lse.astype(np.float64) - want_lse).max())
        say(f"[{tag}] lse max_abs={lerr:.3e}")
        assert lerr <= 1e-5, f"{tag}: lse {lerr}"


@pytest.mark.parametrize("name", sorted(DECODE))
def test_decode_closed_forms(name):
    import torch

    f = DECODE[name]
    say(f"closed forms, decode {name}")
    pool, table, seq, q, nk, nv = full_size_pool(f)
    G = f["hq"] // f["hkv"]
    heads = list(range(f["hkv"])) if f["kv_heads"] is None else f["kv_heads"]
    part = f.get("partition", 0)
    mx = int(seq.max())
    slots = i32_dev(synth.slots_of_last(table, seq, 16))
    tab, sq = i32_dev(table), i32_dev(seq)

    # K = 0: host copy of V on the sampled heads (new token included) first.
    hidx = torch.tensor(heads, device="cuda")
    vh = bits(pool.v[0].index_select(1, hidx))  # [pages, heads, 16, D]
    nvh = bits(nv)[:, heads]
    pool.k.zero_()
    nk.zero_()
    pkv.kv_write(pool, 0, 0, nk, nv, slots)
    out, lse = pkv.decode(pool, 0, 0, q, tab, sq, mx, partition=part)
    torch.cuda.synchronize()
    ob, lb = bits(out), lse.cpu().numpy()
    want = np.empty((f["B"], len(heads), 128))
    for r in range(f["B"]):
        n = int(seq[r])
        pages = table[r, :-(-n // 16)]
        ctx = vh[pages].transpose(1, 0, 2, 3).reshape(len(heads), -1, 128)[:, :n - 1]
        ctx = (ctx.astype(np.uint32) << 16).view(np.float32)
        want[r] = (ctx.sum(axis=1, dtype=np.float64) + bf16_f64(nvh[r])) / n
    del vh
    for i, h in enumerate(heads):
        for g in range(G):
            qh = h * G + g
            check_mean(f"{name} K=0 kv head {h} q head {qh}", ob[:, qh], want[:, i],
                       lb[:, qh], np.log(seq.astype(np.float64)))

    # V = 1: every output is exactly one.
    pool.v.fill_(1.0)
    nv.fill_(1.0)
    synth.device_normal_(pool.k, 7)
    synth.device_normal_(nk, 8)
    pkv.kv_write(pool, 0, 0, nk, nv, slots)
    out, lse = pkv.decode(pool, 0, 0, q, tab, sq, mx, partition=part)
    torch.cuda.synchronize()
    ob = bits(out)
    say(f"[{name} V=1] outputs not exactly 1: {int((ob != ONE_BF16).sum())}")
    assert (ob == ONE_BF16).all()
    assert torch.isfinite(lse).all()

    # One visible key: out = that key's V row bit for bit, lse = its score.
    # Each request's only page is its newest page, which no other request
    # shares.
    one = np.ones(f["B"], np.int32)
    table1 = table.copy()
    table1[:, 0] = table[np.arange(f["B"]), (seq - 1) // 16]
    synth.device_normal_(nv, 9)
    slot0 = i32_dev(synth.slots_of_last(table1, one, 16))
    pkv.kv_write(pool, 0, 0, nk, nv, slot0)
    out, lse = pkv.decode(pool, 0, 0, q, i32_dev(table1), i32_dev(one), 1, partition=part)
    torch.cuda.synchronize()
    ob, nvb = bits(out), bits(nv)
    qf, kf = bf16_f64(bits(q)), bf16_f64(bits(nk))
    for h in range(f["hkv"]):
        for g in range(G):
            assert np.array_equal(ob[:, h * G + g], nvb[:, h]), (name, h, g)
    s = np.einsum("bhgd,bhd->bhg", qf.reshape(f["B"], f["hkv"], G, 128), kf) / math.sqrt(128)
    lerr = float(np.abs(lse.cpu().numpy().reshape(f["B"], f["hkv"], G) - s).max())
    say(f"[{name} one key] lse max_abs={lerr:.3e}")
    assert lerr <= 1e-4 * max(1.0, float(np.abs(s).max()))


@pytest.mark.parametrize("n", [512, 2048])
def test_prefill_closed_forms(n):
    import torch

    say(f"closed forms, prefill 8 x {n}")
    case = synth.make_prefill_case(21, "bf16", [n] * 8, 32, 32, 128)
    (ch,) = synth.chunk_schedule(case, 2048 if n <= 2048 else n)
    tab = i32_dev(case.page_table)
    cu, sl = i32_dev(ch.cu_q_lens), i32_dev(ch.seq_lens)
    q = to_dev(ch.q, "bf16")

    # K = 0: row j of a prompt attends positions 0..j; out = their mean V.
    gp = gpu_pool(case.layout)
    write(gp, 0, 0, np.zeros_like(ch.k), ch.v, ch.slots, "bf16")
    out, lse = pkv.prefill(gp, 0, 0, q, cu, tab, sl, n, n)
    torch.cuda.synchronize()
    ob, lb = bits(out).reshape(8, n, 32, 128), lse.cpu().numpy().reshape(8, n, 32)
    pos = np.arange(1, n + 1, dtype=np.float64)
    for r in range(8):
        v = bf16_f64(ch.v[r * n:(r + 1) * n])          # [n, 32, D], the prompt's V
        want = np.cumsum(v, axis=0) / pos[:, None, None]
        check_mean(f"prefill {n} K=0 prompt {r}", ob[r], want, lb[r],
                   np.broadcast_to(np.log(pos)[:, None], (n, 32)))
        assert np.array_equal(ob[r, 0], ch.v[r * n])   # one visible key: v0 exactly
    del gp

    # V = 1: every output is exactly one.
    gp = gpu_pool(case.layout)
    ones = np.full_like(ch.v, ONE_BF16)
    write(gp, 0, 0, ch.k, ones, ch.slots, "bf16")
    out, lse = pkv.prefill(gp, 0, 0, q, cu, tab, sl, n, n)
    torch.cuda.synchronize()
    ob = bits(out)
    say(f"[prefill {n} V=1] outputs not exactly 1: {int((ob != ONE_BF16).sum())}")
    assert (ob == ONE_BF16).all()
    assert torch.isfinite(lse).all()
