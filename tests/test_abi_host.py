"""CPU-side checks of the C-ABI library: it loads, exports every entry point the
header declares, and its host logic (bank map, workspace size, argument
validation) behaves as documented. No kernel is launched here: every call
below fails validation before anything is enqueued."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import paged_kv_attention_kvcache_amd as pkv
from paged_kv_attention_kvcache_amd import build as pkv_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(pkv.LIB_PATH):
        pkv_build.build()
    return pkv.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[a-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_exports_every_declared_symbol(L):
    declared = header_functions()
    assert set(declared) == set(pkv.EXPORTS), declared
    out = subprocess.run(["nm", "-D", "--defined-only", pkv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in declared:
        assert name in exported, name
        assert hasattr(L, name)


def test_library_is_gfx950_only(L):
    # The offload bundle entries of the library this repository built name
    # their target; every one must be gfx950.
    blob = open(pkv.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx\w+)", blob))
    assert targets == {b"gfx950"}, targets


def test_bank_map_matches_golden(L):
    from test_oracle_pins import read_golden

    for name, g in read_golden().items():
        p = g["params"]
        bank_of, nb = pkv.bank_map(p["planes"], p["layers"], p["rec_first"], p["rec_count"])
        assert nb == g["num_banks"], name
        for (pl, la), b in g["entries"].items():
            assert bank_of[pl, la] == b, (name, pl, la)


def test_bank_map_rejects(L):
    with pytest.raises(pkv.PagedKVError):
        pkv.bank_map(2, 4, 3, 2)
    # a recurrent range whose end overflows int32 is rejected, not wrapped
    out = np.zeros(8, np.int32)
    assert L.pkv_bank_map(2, 4, 3, 2**31 - 2, out.ctypes.data) == pkv.PKV_EINVAL
    assert L.pkv_bank_map(2, 4, 1, -1, out.ctypes.data) == pkv.PKV_EINVAL


def test_workspace_bytes(L):
    # fixed partitions: rows * parts floats for m and l, rows * parts * D for
    # acc, each 256-aligned; or, if larger, the streamed kernel's segment
    # partials: two (m, l, acc) slots per wave and head of the group, for a
    # grid of at most the call's 3 * 2 * 4 = 24 partitions (24 waves)
    st, keep = _pool(kv=2)
    rows, parts, D, G = 3 * 8, 4, 128, 4
    need = L.paged_decode_workspace_bytes(ctypes.byref(st), 3, 8, 2048, 512)
    al = lambda x: (x + 255) // 256 * 256
    slots = 24 * 2 * G
    assert need == max(2 * al(rows * parts * 4) + al(rows * parts * D * 4),
                       al(slots * 2 * 4) + al(slots * D * 4))
    # balanced split: two (m, l, acc) slots per wave and head of the group
    assert L.paged_decode_workspace_bytes(ctypes.byref(st), 3, 8, 2048, 0) > 0
    assert L.paged_decode_workspace_bytes(ctypes.byref(st), 0, 8, 2048, 512) == 0
    assert L.paged_decode_workspace_bytes(ctypes.byref(st), 3, 7, 2048, 512) == 0


def test_split_mode_keeps_prefix_sums_in_32_bits(L):
    # the balanced split sums the call's pages in 32 bits: a call with more
    # than 2^31 - 1 (request, kv head, page) entries takes fixed partitions
    st, keep = _pool(kv=8)
    mode = lambda b, s, p=0: L.paged_decode_split_mode(ctypes.byref(st), b, 64, s, p)
    assert mode(256, 32768) == 1                    # balanced
    assert mode(4096, (1 << 20) - 16) == 1          # 4096 * 8 * 65535 pages fit
    assert mode(4096, 1 << 20) == 2                 # 4096 * 8 * 65536 = 2^31 do not
    assert mode(4097, 32768) == 2                   # more rows than the split keeps
    assert mode(64, 2048) == 0                      # whole contexts


def _pool(dtype=1, page_size=16, head_dim=128, planes=2, layers=3, rec=(0, 3), kv=2,
          pages=8, ptr=1 << 20):
    bank_of, nb = pkv.bank_map(planes, layers, *rec)
    st = pkv._Pool(dtype, page_size, pages, kv, head_dim, planes, layers, nb,
                   bank_of.ctypes.data, ptr, ptr)
    return st, bank_of


FAKE = 1 << 20  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), pkv.PKV_EUNSUPPORTED),
    (dict(page_size=8), pkv.PKV_EUNSUPPORTED),
    (dict(head_dim=96), pkv.PKV_EUNSUPPORTED),
    (dict(ptr=0), pkv.PKV_EINVAL),
    (dict(ptr=FAKE + 4), pkv.PKV_EINVAL),
])
def test_pool_validation(L, kw, code):
    st, keep = _pool(**kw)
    rc = L.paged_kv_write(ctypes.byref(st), 0, 0, FAKE, FAKE, FAKE, 4, None)
    assert rc == code
    assert pkv.last_error()


def test_not_held(L):
    st, keep = _pool(planes=3, layers=4, rec=(1, 2))
    assert L.paged_kv_write(ctypes.byref(st), 2, 0, FAKE, FAKE, FAKE, 1, None) == pkv.PKV_ENOTHELD
    assert L.paged_decode_attn(ctypes.byref(st), 1, 3, FAKE, 4, FAKE, 4, FAKE, 1, 64, 1.0, 0,
                               FAKE, None, None, 0, None) == pkv.PKV_ENOTHELD
    assert L.paged_prefill_attn(ctypes.byref(st), 2, 3, FAKE, 4, FAKE, 8, FAKE, 4, FAKE, 1, 8,
                                64, 1.0, FAKE, None, None) == pkv.PKV_ENOTHELD
    assert L.paged_kv_write(ctypes.byref(st), 3, 0, FAKE, FAKE, FAKE, 1, None) == pkv.PKV_EINVAL


def test_decode_validation(L):
    st, keep = _pool(kv=2)
    call = lambda **o: L.paged_decode_attn(
        ctypes.byref(st), 0, 0, FAKE, o.get("hq", 4), FAKE, o.get("stride", 4), FAKE,
        o.get("batch", 2), o.get("max_seq", 64), 1.0, o.get("part", 0), FAKE, None,
        o.get("ws", None), o.get("ws_bytes", 0), None)
    assert call(hq=3) == pkv.PKV_EINVAL           # not a multiple of Hkv
    assert call(hq=6) == pkv.PKV_EUNSUPPORTED     # group 3
    assert call(batch=0) == pkv.PKV_EINVAL
    assert call(max_seq=65) == pkv.PKV_EINVAL     # beyond stride * page_size
    assert call(part=24) == pkv.PKV_EINVAL        # not a multiple of 16
    assert call(max_seq=64, part=16) == pkv.PKV_EWORKSPACE
    assert call(max_seq=64, part=16, ws=FAKE, ws_bytes=16) == pkv.PKV_EWORKSPACE
    assert call(max_seq=64, part=0, ws=FAKE, ws_bytes=16) == pkv.PKV_EWORKSPACE
    assert "workspace" in pkv.last_error()


def test_prefill_validation(L):
    st, keep = _pool(kv=2)
    call = lambda **o: L.paged_prefill_attn(
        ctypes.byref(st), 0, 0, FAKE, o.get("hq", 2), FAKE, o.get("total", 8), FAKE,
        o.get("stride", 4), FAKE, o.get("batch", 1), o.get("max_q", 8), o.get("max_seq", 64),
        1.0, FAKE, None, None)
    assert call(hq=5) == pkv.PKV_EINVAL
    assert call(batch=0) == pkv.PKV_EINVAL
    assert call(total=-1) == pkv.PKV_EINVAL
    assert call(max_seq=80) == pkv.PKV_EINVAL
    assert call(max_q=70) == pkv.PKV_EINVAL
    assert call(total=0) == pkv.PKV_OK            # nothing to do, nothing enqueued


def test_reduce_validation(L):
    assert L.paged_decode_reduce(3, 1, 1, 128, FAKE, 512, 1, FAKE, FAKE, FAKE, FAKE, None,
                                 None) == pkv.PKV_EUNSUPPORTED
    assert L.paged_decode_reduce(1, 1, 1, 128, FAKE, 0, 1, FAKE, FAKE, FAKE, FAKE, None,
                                 None) == pkv.PKV_EINVAL


def test_write_zero_tokens_is_noop(L):
    st, keep = _pool()
    assert L.paged_kv_write(ctypes.byref(st), 0, 0, None, None, None, 0, None) == pkv.PKV_OK


def test_decode_step_validation(L):
    # every call is validated before any is enqueued: a bad second call
    # rejects the whole step, and the message names the call
    st, keep = _pool(planes=3, layers=4, rec=(1, 2))
    P = ctypes.c_void_p

    def step(planes, layers, n=None, q_null=False, kv="both"):
        n = len(planes) if n is None else n
        pl = (ctypes.c_int32 * len(planes))(*planes)
        ly = (ctypes.c_int32 * len(layers))(*layers)
        ptrs = (P * len(planes))(*([None if q_null else FAKE] * len(planes)))
        kn = ptrs if kv in ("both", "k") else None
        vn = ptrs if kv == "both" else None
        return L.paged_decode_step(ctypes.byref(st), n, pl, ly, kn, vn, ptrs, 4, FAKE, 4, FAKE,
                                   2, 64, 1.0, 0, ptrs, None, FAKE, 1 << 30, None)

    assert step([0, 2], [1, 0]) == pkv.PKV_ENOTHELD      # plane 2 does not hold layer 0
    assert "call 1" in pkv.last_error()
    assert step([0, 3], [1, 1]) == pkv.PKV_EINVAL        # plane 3 outside the pool
    assert step([0], [0], q_null=True) == pkv.PKV_EINVAL
    assert step([0], [0], kv="k") == pkv.PKV_EINVAL      # k_new without v_new
    assert step([0], [0], n=-1) == pkv.PKV_EINVAL
    assert step([], [], n=0) == pkv.PKV_OK               # nothing to do
    # a misaligned q or out in call 1 rejects the step before call 0 is
    # enqueued (with no GPU here, enqueueing call 0 would report a launch
    # failure instead)
    for which in ("q", "out"):
        pl = (ctypes.c_int32 * 2)(0, 0)
        ly = (ctypes.c_int32 * 2)(0, 1)
        good = (P * 2)(FAKE, FAKE)
        bad = (P * 2)(FAKE, FAKE + 8)
        qp, op = (bad, good) if which == "q" else (good, bad)
        rc = L.paged_decode_step(ctypes.byref(st), 2, pl, ly, good, good, qp, 4, FAKE, 4, FAKE,
                                 2, 64, 1.0, 0, op, None, FAKE, 1 << 30, None)
        assert rc == pkv.PKV_EINVAL, which
        assert "call 1" in pkv.last_error() and "aligned" in pkv.last_error()
    handle = ctypes.c_void_p()
    pl = (ctypes.c_int32 * 1)(0)
    ptrs = (P * 1)(FAKE)
    # capture needs a real (non-null) stream; nothing is recorded on failure
    assert L.paged_decode_step_capture(ctypes.byref(st), 1, pl, pl, None, None, ptrs, 4, FAKE, 4,
                                       FAKE, 2, 64, 1.0, 0, ptrs, None, FAKE, 1 << 30, None,
                                       ctypes.byref(handle)) == pkv.PKV_EINVAL
    assert not handle.value
    assert L.paged_decode_step_graph_launch(None, None) == pkv.PKV_EINVAL
    L.paged_decode_step_graph_destroy(None)  # a no-op


def test_decode_latest_validation(L):
    st, keep = _pool(planes=4, layers=3, rec=(1, 2), kv=2)
    call = lambda plane=2, layer=1, ed=FAKE, stride=64, hq=2, **o: L.paged_decode_latest_attn(
        ctypes.byref(st), plane, layer, ed, stride, None, None, FAKE, hq, FAKE, 4, FAKE, 2,
        o.get("max_seq", 64), 1.0, 0, FAKE, None, FAKE, 1 << 30, None)
    assert call(ed=None) == pkv.PKV_EINVAL
    assert call(ed=FAKE + 8) == pkv.PKV_EINVAL          # not 16-byte aligned
    assert call(stride=40) == pkv.PKV_EINVAL            # not a multiple of 16
    assert call(stride=48) == pkv.PKV_EINVAL            # shorter than max_seq_len
    assert call(hq=6) == pkv.PKV_EUNSUPPORTED           # group 3
    assert call(layer=0, plane=1) == pkv.PKV_ENOTHELD   # plane 1 does not hold layer 0
    assert call(layer=0, plane=0, max_seq=65) == pkv.PKV_EINVAL  # beyond stride * page_size


def test_span_slots(L):
    # pkv_span_slots against the slot definition written out position by
    # position: page id of the position's page times 16, plus its offset
    rng = np.random.default_rng(3)
    B, stride, pages = 5, 9, 64
    table = rng.permutation(pages)[:B * stride].reshape(B, stride).astype(np.int32)
    starts = np.array([0, 5, 16, 31, 80], np.int32)
    span = 64
    out = np.full((B, span), -9, np.int32)
    args = lambda st, sp, o: (table.ctypes.data, stride, 16, pages, st.ctypes.data, B, sp,
                              o.ctypes.data)
    assert L.pkv_span_slots(*args(starts, span, out)) == pkv.PKV_OK
    for r in range(B):
        for j in range(span):
            pos = int(starts[r]) + j
            assert out[r, j] == table[r, pos // 16] * 16 + pos % 16
    # errors write nothing
    for bad_starts, bad_span in ((np.array([0, 5, 16, 31, 81], np.int32), span),
                                 (np.array([-1, 0, 0, 0, 0], np.int32), 4)):
        o = np.full((B, bad_span), -9, np.int32)
        assert L.pkv_span_slots(*args(bad_starts, bad_span, o)) == pkv.PKV_EINVAL
        assert (o == -9).all()
    t2 = table.copy()
    t2[4, 8] = pages  # a page id outside the pool, inside the span of request 4
    o = np.full((B, span), -9, np.int32)
    assert L.pkv_span_slots(t2.ctypes.data, stride, 16, pages, starts.ctypes.data, B, span,
                            o.ctypes.data) == pkv.PKV_EINVAL
    assert (o == -9).all()
    # the binding's LotusBlock takes its slots from the library
    assert "pkv_span_slots" in open(os.path.join(ROOT, "paged_kv_attention_kvcache_amd",
                                                 "__init__.py")).read()


def test_noalloc_rejects_sizes_beyond_its_scratch(L):
    # the header's PKV_SCRATCH_BYTES is the binding's constant
    text = open(HEADER).read()
    m = re.search(r"#define PKV_SCRATCH_BYTES \((\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == pkv.SCRATCH_BYTES
    # 256 long contexts on fixed 512-token partitions need far more than the
    # scratch array: rejected, with nothing enqueued
    st, keep = _pool(kv=8, pages=1 << 16)
    call = lambda part, batch=256, max_seq=32768: L.paged_decode_attn_noalloc(
        ctypes.byref(st), 0, 0, FAKE, 64, FAKE, 2048, FAKE, batch, max_seq, 1.0, part, FAKE,
        None, None)
    need = L.paged_decode_workspace_bytes(ctypes.byref(st), 256, 64, 32768, 512)
    assert need > pkv.SCRATCH_BYTES
    assert call(512) == pkv.PKV_EWORKSPACE
    assert "scratch" in pkv.last_error()
    # invalid sizes report paged_decode_attn's own errors
    assert call(24) == pkv.PKV_EINVAL                   # partition not a multiple of 16
    assert call(0, batch=0) == pkv.PKV_EINVAL
