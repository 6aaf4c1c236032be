"""fp64 CPU oracle for paged-KV attention over a multi-plane page pool.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package. It wraps the plain C
library in ``oracle.c`` (its own C-ABI, host pointers, fp64 arithmetic) with
ctypes and numpy; it shares no code with the GPU library.

What it computes (the pages it follows are cited in ``oracle.h``):

* ``bank_map``   -- per-plane layer map: depth 0 holds every layer, deeper
  planes only the recurrent ones ("Faster fuzzy minds", section "Recurrent
  depth"; vllm-rlt PR 152, section "Summary").
* ``kv_write``   -- store_kv slot scatter ("Faster fuzzy minds", section
  "LOTUS").
* ``decode`` / ``prefill`` -- softmax attention over the context gathered
  through the page table ("Faster fuzzy minds", section "When scheduler does
  the work": page_table[request, position] -> slot).
* ``decode_partials`` / ``combine`` -- the split-K partials and their combine
  (a rewriting of the same softmax, used to pin the reduction step).
* ``decode_latest`` -- decode with early exit: each position is read from the
  deepest plane it holds, up to the query's plane ("Faster fuzzy minds",
  section "Can we actually stop early?").
* ``lotus_loop`` -- the in-place latent loop: every pass hands the block's
  fixed slots to store_kv again (an overwrite) and runs one extend-prefill
  over all block positions ("Faster fuzzy minds", section "LOTUS").

Arrays: bf16 data travels as ``np.uint16`` raw bits, fp32 as ``np.float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liborc.so")
_lock = threading.Lock()
_lib = None

ORC_OK = 0
ORC_EINVAL = -1
ORC_ENOTHELD = -3
ORC_ESLOT = -10
ORC_EDUP = -11
ORC_EPAGE = -12
ORC_ELEN = -13

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared"]


def build(src: str = _SRC, out: str = _LIB_PATH, extra: list[str] | None = None) -> str:
    """Compile the oracle with gcc (plain C11 + OpenMP)."""
    cmd = ["gcc", *CFLAGS, *(extra or []), "-I", _HERE, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what} returned {code}")
        self.code = code


class _Pool(ctypes.Structure):
    _fields_ = [
        ("elem_bytes", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_planes", ctypes.c_int32),
        ("num_layers", ctypes.c_int32),
        ("num_banks", ctypes.c_int32),
        ("bank_of", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
    ]


def _bind(lib):
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.orc_bank_map.argtypes = [i32, i32, i32, i32, P]
    lib.orc_kv_write.argtypes = [P, i32, i32, P, P, P, i32]
    lib.orc_attend.argtypes = [P, i32, i32, P, i32, P, P, i32, P, i32, ctypes.c_double, P, P]
    lib.orc_decode_partials.argtypes = [P, i32, i32, P, i32, P, i32, P, i32,
                                        ctypes.c_double, i32, i32, P, P, P]
    lib.orc_combine.argtypes = [i32, i32, i32, P, P, P, P, P, P]
    lib.orc_decode_latest.argtypes = [P, i32, i32, P, i32, P, i32, P, i32, P, i32,
                                      ctypes.c_double, P, P]
    for f in (lib.orc_bank_map, lib.orc_kv_write, lib.orc_attend,
              lib.orc_decode_partials, lib.orc_combine, lib.orc_decode_latest):
        f.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or (
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
                build()
            _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags.c_contiguous, "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def bank_map(num_planes: int, num_layers: int, rec_first: int = 0,
             rec_count: int | None = None, lib=None) -> tuple[np.ndarray, int]:
    """Returns (bank_of[num_planes, num_layers], num_banks)."""
    lib = lib or load()
    if rec_count is None:
        rec_count = num_layers - rec_first
    out = np.full((num_planes, num_layers), -7, dtype=np.int32)
    n = lib.orc_bank_map(num_planes, num_layers, rec_first, rec_count, _ptr(out))
    if n < 0:
        raise OracleError(n, "bank_map")
    return out, n


class Pool:
    """Host pool: k, v are [num_banks, num_pages, Hkv, P, D] (uint16 for bf16)."""

    def __init__(self, dtype: str, page_size: int, num_pages: int, num_kv_heads: int,
                 head_dim: int, bank_of: np.ndarray, num_banks: int,
                 k: np.ndarray | None = None, v: np.ndarray | None = None, fill=None):
        assert dtype in ("f32", "bf16")
        self.dtype = dtype
        self.np_dtype = np.float32 if dtype == "f32" else np.uint16
        self.page_size, self.num_pages = page_size, num_pages
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        self.bank_of = _i32(bank_of).reshape(bank_of.shape)
        self.num_planes, self.num_layers = self.bank_of.shape
        self.num_banks = num_banks
        shape = (num_banks, num_pages, num_kv_heads, page_size, head_dim)
        if k is None:
            k = np.zeros(shape, self.np_dtype)
            v = np.zeros(shape, self.np_dtype)
            if fill is not None:
                k[...] = fill
                v[...] = fill
        assert k.shape == shape and v.shape == shape
        assert k.dtype == self.np_dtype and v.dtype == self.np_dtype
        self.k = np.ascontiguousarray(k)
        self.v = np.ascontiguousarray(v)

    def _struct(self) -> _Pool:
        return _Pool(4 if self.dtype == "f32" else 2, self.page_size, self.num_pages,
                     self.num_kv_heads, self.head_dim, self.num_planes, self.num_layers,
                     self.num_banks, _ptr(self.bank_of), _ptr(self.k), _ptr(self.v))

    def copy(self) -> "Pool":
        return Pool(self.dtype, self.page_size, self.num_pages, self.num_kv_heads,
                    self.head_dim, self.bank_of.copy(), self.num_banks,
                    self.k.copy(), self.v.copy())


def _check(rc: int, what: str):
    if rc != ORC_OK:
        raise OracleError(rc, what)


def kv_write(pool: Pool, plane: int, layer: int, k: np.ndarray, v: np.ndarray,
             slots, lib=None) -> None:
    lib = lib or load()
    k = np.ascontiguousarray(k, dtype=pool.np_dtype)
    v = np.ascontiguousarray(v, dtype=pool.np_dtype)
    slots = _i32(slots)
    T = slots.shape[0]
    assert k.shape == (T, pool.num_kv_heads, pool.head_dim) and v.shape == k.shape
    st = pool._struct()
    _check(lib.orc_kv_write(ctypes.byref(st), plane, layer, _ptr(k), _ptr(v),
                            _ptr(slots), T), "kv_write")


def _attend(pool: Pool, plane, layer, q, cu_q_lens, page_table, seq_lens, scale, lib):
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=pool.np_dtype)
    rows, Hq, D = q.shape
    assert D == pool.head_dim
    page_table = _i32(page_table)
    seq_lens = _i32(seq_lens)
    B = seq_lens.shape[0]
    stride = page_table.shape[1] if page_table.ndim == 2 else 0
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((rows, Hq, D), np.float64)
    lse = np.zeros((rows, Hq), np.float64)
    cu = None if cu_q_lens is None else _i32(cu_q_lens)
    st = pool._struct()
    _check(lib.orc_attend(ctypes.byref(st), plane, layer, _ptr(q), Hq, _ptr(cu),
                          _ptr(page_table), stride, _ptr(seq_lens), B, float(scale),
                          _ptr(out), _ptr(lse)), "attend")
    return out, lse


def decode(pool: Pool, plane: int, layer: int, q: np.ndarray, page_table, seq_lens,
           scale: float | None = None, lib=None):
    """q [B, Hq, D] -> (out [B, Hq, D] fp64, lse [B, Hq] fp64)."""
    assert q.shape[0] == len(seq_lens)
    return _attend(pool, plane, layer, q, None, page_table, seq_lens, scale, lib)


def prefill(pool: Pool, plane: int, layer: int, q: np.ndarray, cu_q_lens, page_table,
            seq_lens, scale: float | None = None, lib=None):
    """Packed q [sum q_len, Hq, D] -> (out, lse) in fp64."""
    return _attend(pool, plane, layer, q, cu_q_lens, page_table, seq_lens, scale, lib)


def decode_latest(pool: Pool, plane: int, layer: int, exit_depth, q: np.ndarray, page_table,
                  seq_lens, scale: float | None = None, lib=None):
    """Early-exit decode ("Faster fuzzy minds", section "Can we actually stop
    early?"): position pos of request r is read from plane
    min(plane, exit_depth[r, pos]) of the same layer. exit_depth int8
    [B, stride >= max seq_len]. Returns (out, lse) in fp64."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=pool.np_dtype)
    B, Hq, D = q.shape
    page_table = _i32(page_table)
    seq_lens = _i32(seq_lens)
    ed = np.ascontiguousarray(exit_depth, dtype=np.int8)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, Hq, D), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    st = pool._struct()
    _check(lib.orc_decode_latest(ctypes.byref(st), plane, layer, _ptr(ed), ed.shape[1], _ptr(q),
                                 Hq, _ptr(page_table), page_table.shape[1], _ptr(seq_lens), B,
                                 float(scale), _ptr(out), _ptr(lse)), "decode_latest")
    return out, lse


def decode_partials(pool: Pool, plane: int, layer: int, q: np.ndarray, page_table,
                    seq_lens, partition: int, max_parts: int,
                    scale: float | None = None, lib=None):
    """Split-K partials: (m [B,Hq,P], l [B,Hq,P], acc [B,Hq,P,D]) in fp64."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=pool.np_dtype)
    B, Hq, D = q.shape
    page_table = _i32(page_table)
    seq_lens = _i32(seq_lens)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    pm = np.zeros((B, Hq, max_parts), np.float64)
    pl = np.zeros((B, Hq, max_parts), np.float64)
    pacc = np.zeros((B, Hq, max_parts, D), np.float64)
    st = pool._struct()
    _check(lib.orc_decode_partials(ctypes.byref(st), plane, layer, _ptr(q), Hq,
                                   _ptr(page_table), page_table.shape[1], _ptr(seq_lens),
                                   B, float(scale), partition, max_parts,
                                   _ptr(pm), _ptr(pl), _ptr(pacc)), "decode_partials")
    return pm, pl, pacc


def combine(n_parts, pm: np.ndarray, pl: np.ndarray, pacc: np.ndarray, lib=None):
    """Combine partials row by row -> (out [rows, D], lse [rows]) in fp64."""
    lib = lib or load()
    max_parts = pm.shape[-1]
    D = pacc.shape[-1]
    pm = np.ascontiguousarray(pm, np.float64).reshape(-1, max_parts)
    rows = pm.shape[0]
    pl = np.ascontiguousarray(pl, np.float64).reshape(rows, max_parts)
    pacc = np.ascontiguousarray(pacc, np.float64).reshape(rows, max_parts, D)
    n_parts = _i32(n_parts).reshape(rows)
    out = np.zeros((rows, D), np.float64)
    lse = np.zeros((rows,), np.float64)
    _check(lib.orc_combine(rows, max_parts, D, _ptr(n_parts), _ptr(pm), _ptr(pl),
                           _ptr(pacc), _ptr(out), _ptr(lse)), "combine")
    return out, lse


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 raw bits (for tests)."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def lotus_loop(pool: Pool, plane: int, layer: int, passes, block_slots, cu_q_lens, page_table,
               seq_lens, scale: float | None = None, lib=None, after_pass=None):
    """LOTUS ("Faster fuzzy minds", section "LOTUS"): the block's slots are
    chosen once; each pass (k, v, q) writes its K/V to those same slots,
    overwriting the previous pass, then runs one extend-prefill of all block
    rows (query row j of request r at position seq_lens[r] - q_len + j) over
    the prefix and the block. Returns [(out, lse)] per pass. after_pass(i) is
    called after pass i's write and attention (for inspection)."""
    res = []
    for i, (k, v, q) in enumerate(passes):
        kv_write(pool, plane, layer, k, v, block_slots, lib)
        res.append(prefill(pool, plane, layer, q, cu_q_lens, page_table, seq_lens, scale, lib))
        if after_pass is not None:
            after_pass(i)
    return res
