"""Paged-KV attention over a multi-plane page pool, for MI355X (gfx950).

A thin ctypes binding over the C-ABI in include/pagedkv.h (libpagedkv.so,
built in-tree by ``build.py``). Every step of the path runs in the library's
HIP kernels; this module only marshals torch tensors (device memory) and the
current HIP stream into the C calls, and allocates outputs and the split-K
workspace through torch when the caller does not pass them.

If the library is missing, importing the binding functions raises: there is
no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpagedkv.so")

PKV_F32, PKV_BF16 = 0, 1
PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_ENOTHELD, PKV_EWORKSPACE, PKV_ELAUNCH = 0, -1, -2, -3, -4, -5
PKV_ENOSPACE = -6
DEFAULT_PARTITION = 512
SCRATCH_BYTES = 32 << 20  # PKV_SCRATCH_BYTES: paged_decode_attn_noalloc's per-GPU array

_lib = None


class PagedKVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class _Pool(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_planes", ctypes.c_int32),
        ("num_layers", ctypes.c_int32),
        ("num_banks", ctypes.c_int32),
        ("bank_of", ctypes.c_void_p),
        ("k_base", ctypes.c_void_p),
        ("v_base", ctypes.c_void_p),
    ]


EXPORTS = ("pkv_bank_map", "pkv_pool_bytes", "paged_kv_write", "paged_decode_workspace_bytes",
           "paged_decode_attn", "paged_decode_attn_noalloc", "paged_decode_append_attn",
           "paged_decode_latest_attn",
           "paged_decode_split_mode",
           "paged_decode_step", "paged_decode_step_capture", "paged_decode_step_graph_launch",
           "paged_decode_step_graph_destroy", "paged_decode_reduce", "paged_prefill_attn",
           "paged_extend_attn", "pkv_mgr_create", "pkv_mgr_destroy", "pkv_mgr_free_count",
           "pkv_mgr_alloc", "pkv_mgr_retain", "pkv_mgr_release", "pkv_mgr_refcount",
           "pkv_mgr_note_write", "pkv_mgr_published_prefix", "pkv_span_slots",
           "pkv_last_error")


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run paged_kv_attention_kvcache_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.pkv_bank_map.argtypes = [i32, i32, i32, i32, P]
        L.pkv_bank_map.restype = ctypes.c_int
        L.pkv_pool_bytes.argtypes = [P]
        L.pkv_pool_bytes.restype = sz
        L.paged_kv_write.argtypes = [P, i32, i32, P, P, P, i32, P]
        L.paged_kv_write.restype = ctypes.c_int
        L.paged_decode_workspace_bytes.argtypes = [P, i32, i32, i32, i32]
        L.paged_decode_workspace_bytes.restype = sz
        L.paged_decode_attn.argtypes = [P, i32, i32, P, i32, P, i32, P, i32, i32, ctypes.c_float,
                                        i32, P, P, P, sz, P]
        L.paged_decode_attn.restype = ctypes.c_int
        L.paged_decode_attn_noalloc.argtypes = [P, i32, i32, P, i32, P, i32, P, i32, i32,
                                                ctypes.c_float, i32, P, P, P]
        L.paged_decode_attn_noalloc.restype = ctypes.c_int
        L.paged_decode_append_attn.argtypes = [P, i32, i32, P, P, P, i32, P, i32, P, i32, i32,
                                               ctypes.c_float, i32, P, P, P, sz, P]
        L.paged_decode_append_attn.restype = ctypes.c_int
        L.paged_decode_latest_attn.argtypes = [P, i32, i32, P, i32, P, P, P, i32, P, i32, P, i32,
                                               i32, ctypes.c_float, i32, P, P, P, sz, P]
        L.paged_decode_latest_attn.restype = ctypes.c_int
        L.paged_decode_split_mode.argtypes = [P, i32, i32, i32, i32]
        L.paged_decode_split_mode.restype = ctypes.c_int
        step = [P, i32, P, P, P, P, P, i32, P, i32, P, i32, i32, ctypes.c_float, i32, P, P, P,
                sz, P]
        L.paged_decode_step.argtypes = step
        L.paged_decode_step.restype = ctypes.c_int
        L.paged_decode_step_capture.argtypes = step + [ctypes.POINTER(P)]
        L.paged_decode_step_capture.restype = ctypes.c_int
        L.paged_decode_step_graph_launch.argtypes = [P, P]
        L.paged_decode_step_graph_launch.restype = ctypes.c_int
        L.paged_decode_step_graph_destroy.argtypes = [P]
        L.paged_decode_step_graph_destroy.restype = None
        L.paged_decode_reduce.argtypes = [i32, i32, i32, i32, P, i32, i32, P, P, P, P, P, P]
        L.paged_decode_reduce.restype = ctypes.c_int
        L.paged_prefill_attn.argtypes = [P, i32, i32, P, i32, P, i32, P, i32, P, i32, i32, i32,
                                         ctypes.c_float, P, P, P]
        L.paged_prefill_attn.restype = ctypes.c_int
        L.paged_extend_attn.argtypes = [P, i32, i32, P, P, P, P, i32, P, i32, P, i32, P, i32,
                                        i32, i32, ctypes.c_float, P, P, P]
        L.paged_extend_attn.restype = ctypes.c_int
        L.pkv_mgr_create.argtypes = [i32, i32, i32, i32, P]
        L.pkv_mgr_create.restype = P
        L.pkv_mgr_destroy.argtypes = [P]
        L.pkv_mgr_destroy.restype = None
        L.pkv_mgr_free_count.argtypes = [P]
        L.pkv_mgr_free_count.restype = i32
        for name in ("pkv_mgr_alloc", "pkv_mgr_retain", "pkv_mgr_release"):
            getattr(L, name).argtypes = [P, i32, P]
            getattr(L, name).restype = ctypes.c_int
        L.pkv_mgr_refcount.argtypes = [P, i32]
        L.pkv_mgr_refcount.restype = i32
        L.pkv_mgr_note_write.argtypes = [P, i32, i32, i32, P]
        L.pkv_mgr_note_write.restype = ctypes.c_int
        L.pkv_mgr_published_prefix.argtypes = [P, i32, P, i32]
        L.pkv_mgr_published_prefix.restype = i32
        L.pkv_span_slots.argtypes = [P, i32, i32, i32, P, i32, i32, P]
        L.pkv_span_slots.restype = ctypes.c_int
        L.pkv_last_error.argtypes = []
        L.pkv_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().pkv_last_error().decode()


def _check(rc: int):
    if rc < 0:
        raise PagedKVError(rc, last_error())
    return rc


def bank_map(num_planes: int, num_layers: int, rec_first: int = 0,
             rec_count: int | None = None) -> tuple[np.ndarray, int]:
    """Per-plane layer map -> (bank_of [planes, layers] int32, num_banks)."""
    if rec_count is None:
        rec_count = num_layers - rec_first
    out = np.full((num_planes, num_layers), -7, np.int32)
    n = _check(lib().pkv_bank_map(num_planes, num_layers, rec_first, rec_count,
                                  out.ctypes.data))
    return out, n


def _torch():
    import torch

    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dptr(t) -> int | None:
    return None if t is None else t.data_ptr()


class Pool:
    """A multi-plane page pool in device memory.

    k, v: torch tensors [num_banks, num_pages, num_kv_heads, 16, head_dim] of
    dtype float32 or bfloat16 on the GPU (allocated here if not given).
    bank_of: [num_planes, num_layers] int32 (from ``bank_map``).
    """

    def __init__(self, dtype, num_pages: int, num_kv_heads: int, head_dim: int,
                 bank_of: np.ndarray, num_banks: int, page_size: int = 16,
                 k=None, v=None, device="cuda"):
        torch = _torch()
        self.torch_dtype = dtype
        self.dtype = PKV_BF16 if dtype == torch.bfloat16 else PKV_F32
        self.page_size, self.num_pages = page_size, num_pages
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        self.bank_of = np.ascontiguousarray(bank_of, dtype=np.int32)
        self.num_planes, self.num_layers = self.bank_of.shape
        self.num_banks = num_banks
        shape = (num_banks, num_pages, num_kv_heads, page_size, head_dim)
        if k is None:
            k = torch.empty(shape, dtype=dtype, device=device)
            v = torch.empty(shape, dtype=dtype, device=device)
        assert tuple(k.shape) == shape and tuple(v.shape) == shape
        assert k.dtype == dtype and v.dtype == dtype and k.is_contiguous() and v.is_contiguous()
        self.k, self.v = k, v
        self._st = _Pool(self.dtype, page_size, num_pages, num_kv_heads, head_dim,
                         self.num_planes, self.num_layers, num_banks,
                         self.bank_of.ctypes.data, k.data_ptr(), v.data_ptr())

    @property
    def ref(self):
        return ctypes.byref(self._st)


def kv_write(pool: Pool, plane: int, layer: int, k, v, slot_mapping, stream=None) -> None:
    """store_kv: k, v [T, Hkv, D] (pool dtype, device), slot_mapping [T] int32."""
    T = int(slot_mapping.shape[0])
    _check(lib().paged_kv_write(pool.ref, plane, layer, _dptr(k), _dptr(v),
                                _dptr(slot_mapping), T, _stream(stream)))


def workspace_bytes(pool: "Pool", batch: int, num_q_heads: int, max_seq_len: int,
                    partition: int = 0) -> int:
    return int(lib().paged_decode_workspace_bytes(pool.ref, batch, num_q_heads, max_seq_len,
                                                  partition))


SPLIT_MODES = {0: "whole", 1: "balanced", 2: "fixed"}


def split_mode(pool: "Pool", batch: int, num_q_heads: int, max_seq_len: int,
               partition: int = 0) -> str:
    """The work split paged_decode_attn takes for these sizes."""
    return SPLIT_MODES[_check(lib().paged_decode_split_mode(pool.ref, batch, num_q_heads,
                                                           max_seq_len, partition))]


def decode(pool: Pool, plane: int, layer: int, q, page_table, seq_lens, max_seq_len: int,
           scale: float | None = None, partition: int = 0, out=None, lse=None,
           workspace=None, with_lse: bool = True, stream=None, k_new=None, v_new=None):
    """Decode attention. q [B, Hq, D]; page_table [B, stride] int32; seq_lens [B] int32.
    With k_new, v_new [B, Hkv, D]: the decode step that first appends each
    request's newest token at position seq_len - 1 (one kernel).

    Returns (out [B, Hq, D], lse [B, Hq] fp32 or None)."""
    torch = _torch()
    B, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = workspace_bytes(pool, B, Hq, max_seq_len, partition)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    if k_new is not None:
        _check(lib().paged_decode_append_attn(
            pool.ref, plane, layer, _dptr(k_new), _dptr(v_new), _dptr(q), Hq,
            _dptr(page_table), int(page_table.shape[1]), _dptr(seq_lens), B, max_seq_len,
            float(scale), partition, _dptr(out), _dptr(lse), _dptr(workspace), ws_bytes,
            _stream(stream)))
        return out, lse
    _check(lib().paged_decode_attn(pool.ref, plane, layer, _dptr(q), Hq, _dptr(page_table),
                                   int(page_table.shape[1]), _dptr(seq_lens), B, max_seq_len,
                                   float(scale), partition, _dptr(out), _dptr(lse),
                                   _dptr(workspace), ws_bytes, _stream(stream)))
    return out, lse


def decode_noalloc(pool: Pool, plane: int, layer: int, q, page_table, seq_lens,
                   max_seq_len: int, out, lse=None, scale: float | None = None,
                   partition: int = 0, stream=None):
    """paged_decode_attn_noalloc: decode attention whose split-K partials go
    to the library's fixed per-GPU scratch array, so nothing is allocated
    here or in the library. out [B, Hq, D] and lse [B, Hq] (or None) are the
    caller's. Returns (out, lse)."""
    B, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check(lib().paged_decode_attn_noalloc(pool.ref, plane, layer, _dptr(q), Hq,
                                           _dptr(page_table), int(page_table.shape[1]),
                                           _dptr(seq_lens), B, max_seq_len, float(scale),
                                           partition, _dptr(out), _dptr(lse), _stream(stream)))
    return out, lse


def decode_latest(pool: Pool, plane: int, layer: int, exit_depth, q, page_table, seq_lens,
                  max_seq_len: int, scale: float | None = None, partition: int = 0, out=None,
                  lse=None, workspace=None, with_lse: bool = True, stream=None, k_new=None,
                  v_new=None):
    """Early-exit decode (paged_decode_latest_attn): exit_depth int8 [B, stride]
    (stride a multiple of 16, >= max_seq_len) gives each position's deepest
    plane; position pos is read from plane min(plane, exit_depth[r, pos])."""
    torch = _torch()
    B, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = workspace_bytes(pool, B, Hq, max_seq_len, partition)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().paged_decode_latest_attn(
        pool.ref, plane, layer, _dptr(exit_depth), int(exit_depth.shape[1]), _dptr(k_new),
        _dptr(v_new), _dptr(q), Hq, _dptr(page_table), int(page_table.shape[1]),
        _dptr(seq_lens), B, max_seq_len, float(scale), partition, _dptr(out), _dptr(lse),
        _dptr(workspace), ws_bytes, _stream(stream)))
    return out, lse


def _ptr_array(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _step_args(pool: Pool, calls, q, page_table, seq_lens, max_seq_len, scale, partition, out,
               lse, workspace, k_new, v_new):
    """Marshals a decode step: calls [(plane, layer)], per-call tensors q[i],
    out[i], lse[i], k_new[i], v_new[i] (sequences or stacked tensors)."""
    n = len(calls)
    B, Hq, D = q[0].shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    planes = np.ascontiguousarray([c[0] for c in calls], dtype=np.int32)
    layers = np.ascontiguousarray([c[1] for c in calls], dtype=np.int32)
    keep = [planes, layers]
    arrs = {}
    for name, ts in (("q", q), ("out", out), ("lse", lse), ("k_new", k_new), ("v_new", v_new)):
        if ts is None:
            arrs[name] = None
            continue
        assert len(ts) == n, name
        a = _ptr_array([ts[i] for i in range(n)])
        keep.append(a)
        arrs[name] = a
    need = workspace_bytes(pool, B, Hq, max_seq_len, partition)
    ws_bytes = workspace.numel() * workspace.element_size()
    args = [pool.ref, n, planes.ctypes.data, layers.ctypes.data, arrs["k_new"], arrs["v_new"],
            arrs["q"], Hq, _dptr(page_table), int(page_table.shape[1]), _dptr(seq_lens), B,
            max_seq_len, float(scale), partition, arrs["out"], arrs["lse"], _dptr(workspace),
            ws_bytes]
    return args, keep, need


def decode_step(pool: Pool, calls, q, page_table, seq_lens, max_seq_len: int, out, lse=None,
                workspace=None, k_new=None, v_new=None, scale: float | None = None,
                partition: int = 0, stream=None) -> None:
    """One decode step over several (plane, layer) banks in one C call
    (paged_decode_step). q[i], out[i] [B, Hq, D]; lse[i] [B, Hq] or lse None;
    k_new[i], v_new[i] [B, Hkv, D] or both None (no append)."""
    if workspace is None:
        torch = _torch()
        B, Hq, _ = q[0].shape
        workspace = torch.empty(max(workspace_bytes(pool, B, Hq, max_seq_len, partition), 1),
                                dtype=torch.uint8, device=q[0].device)
    args, keep, _ = _step_args(pool, calls, q, page_table, seq_lens, max_seq_len, scale,
                               partition, out, lse, workspace, k_new, v_new)
    _check(lib().paged_decode_step(*args, _stream(stream)))


class StepGraph:
    """A decode step captured once (paged_decode_step_capture) and replayed as
    one submission. The tensors passed here are the step's fixed buffers:
    replays read their contents at replay time."""

    def __init__(self, pool: Pool, calls, q, page_table, seq_lens, max_seq_len: int, out,
                 lse=None, workspace=None, k_new=None, v_new=None, scale: float | None = None,
                 partition: int = 0):
        torch = _torch()
        if workspace is None:
            B, Hq, _ = q[0].shape
            workspace = torch.empty(max(workspace_bytes(pool, B, Hq, max_seq_len, partition), 1),
                                    dtype=torch.uint8, device=q[0].device)
        # keep every buffer the graph points at alive with the graph
        self._bufs = (pool, q, page_table, seq_lens, out, lse, workspace, k_new, v_new)
        args, self._keep, _ = _step_args(pool, calls, q, page_table, seq_lens, max_seq_len, scale,
                                         partition, out, lse, workspace, k_new, v_new)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        torch.cuda.current_stream().synchronize()
        handle = ctypes.c_void_p()
        _check(lib().paged_decode_step_capture(*args, side.cuda_stream, ctypes.byref(handle)))
        self._h = handle

    def launch(self, stream=None) -> None:
        _check(lib().paged_decode_step_graph_launch(self._h, _stream(stream)))

    def close(self) -> None:
        if self._h is not None and self._h.value:
            lib().paged_decode_step_graph_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def decode_reduce(dtype, seq_lens, partition: int, part_m, part_l, part_acc, out=None,
                  lse=None, stream=None):
    """Split-K combine. part_m/part_l [B, Hq, max_parts] fp32 (base-2 units),
    part_acc [B, Hq, max_parts, D]."""
    torch = _torch()
    B, Hq, max_parts = part_m.shape
    D = part_acc.shape[-1]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=dtype, device=part_m.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=part_m.device)
    code = PKV_BF16 if dtype == torch.bfloat16 else PKV_F32
    _check(lib().paged_decode_reduce(code, B, Hq, D, _dptr(seq_lens), partition, max_parts,
                                     _dptr(part_m), _dptr(part_l), _dptr(part_acc), _dptr(out),
                                     _dptr(lse), _stream(stream)))
    return out, lse


def prefill(pool: Pool, plane: int, layer: int, q, cu_q_lens, page_table, seq_lens,
            max_q_len: int, max_seq_len: int, scale: float | None = None, out=None, lse=None,
            with_lse: bool = True, stream=None):
    """Chunked causal prefill. q [total_q, Hq, D] packed; cu_q_lens [B+1] int32."""
    torch = _torch()
    total_q, Hq, D = q.shape
    B = int(seq_lens.shape[0])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    _check(lib().paged_prefill_attn(pool.ref, plane, layer, _dptr(q), Hq, _dptr(cu_q_lens),
                                    total_q, _dptr(page_table), int(page_table.shape[1]),
                                    _dptr(seq_lens), B, max_q_len, max_seq_len, float(scale),
                                    _dptr(out), _dptr(lse), _stream(stream)))
    return out, lse


def extend(pool: Pool, plane: int, layer: int, k, v, slot_mapping, q, cu_q_lens, page_table,
           seq_lens, max_q_len: int, max_seq_len: int, scale: float | None = None, out=None,
           lse=None, with_lse: bool = True, stream=None):
    """One extend pass (paged_extend_attn): store_kv of the span's k, v
    [total_q, Hkv, D] to slot_mapping [total_q], then causal prefill of q
    [total_q, Hq, D] over the context, in one call."""
    torch = _torch()
    total_q, Hq, D = q.shape
    B = int(seq_lens.shape[0])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    _check(lib().paged_extend_attn(pool.ref, plane, layer, _dptr(k), _dptr(v),
                                   _dptr(slot_mapping), _dptr(q), Hq, _dptr(cu_q_lens), total_q,
                                   _dptr(page_table), int(page_table.shape[1]), _dptr(seq_lens),
                                   B, max_q_len, max_seq_len, float(scale), _dptr(out),
                                   _dptr(lse), _stream(stream)))
    return out, lse


class LotusBlock:
    """The in-place latent loop of one batch of requests on one bank: each
    request's block of positions [start_r, start_r + block) is handed the
    same slots on every pass, so pass k overwrites pass k-1's K/V and attends
    the prefix plus its own block ("Faster fuzzy minds", section "LOTUS").
    The slots are computed once by the library (pkv_span_slots), from the
    page table, when the loop starts.

    pass_(k, v, q) runs one pass: k, v [B * block, Hkv, D] and q
    [B * block, Hq, D], request-major."""

    def __init__(self, pool: Pool, plane: int, layer: int, page_table, starts, block: int,
                 page_size: int = 16):
        torch = _torch()
        starts = np.ascontiguousarray(starts, dtype=np.int32)
        table = page_table.cpu().numpy() if hasattr(page_table, "cpu") else np.asarray(page_table)
        table = np.ascontiguousarray(table, dtype=np.int32)
        B = len(starts)
        slots = np.empty((B, block), np.int32)
        _check(lib().pkv_span_slots(table.ctypes.data, table.shape[1], page_size,
                                    pool.num_pages, starts.ctypes.data, B, block,
                                    slots.ctypes.data))
        dev = pool.k.device
        self.pool, self.plane, self.layer, self.block = pool, plane, layer, block
        self.page_table = page_table if hasattr(page_table, "data_ptr") else \
            torch.from_numpy(table).to(dev)
        self.slots = torch.from_numpy(slots.reshape(-1)).to(dev)
        self.cu = torch.from_numpy((np.arange(B + 1) * block).astype(np.int32)).to(dev)
        ends = (starts + block).astype(np.int32)
        self.seq = torch.from_numpy(ends).to(dev)
        self.max_seq = int(ends.max())

    def pass_(self, k, v, q, out=None, lse=None, with_lse: bool = True, scale=None, stream=None):
        return extend(self.pool, self.plane, self.layer, k, v, self.slots, q, self.cu,
                      self.page_table, self.seq, self.block, self.max_seq, scale=scale, out=out,
                      lse=lse, with_lse=with_lse, stream=stream)


class PageManager:
    """Host page manager of a multi-plane pool (pkv_mgr_*): reference-counted
    pages, a constant-time free count, and per-plane prefix publication."""

    def __init__(self, num_pages: int, bank_of: np.ndarray, page_size: int = 16):
        self.bank_of = np.ascontiguousarray(bank_of, dtype=np.int32)
        planes, layers = self.bank_of.shape
        self._h = lib().pkv_mgr_create(num_pages, page_size, planes, layers,
                                       self.bank_of.ctypes.data)
        if not self._h:
            raise PagedKVError(PKV_EINVAL, "pkv_mgr_create: invalid arguments")

    @staticmethod
    def _ids(ids) -> np.ndarray:
        return np.ascontiguousarray(np.asarray(ids, dtype=np.int32).reshape(-1))

    def free_count(self) -> int:
        return int(_check(lib().pkv_mgr_free_count(self._h)))

    def alloc(self, n: int) -> np.ndarray:
        out = np.empty(n, np.int32)
        _check(lib().pkv_mgr_alloc(self._h, n, out.ctypes.data))
        return out

    def retain(self, ids) -> None:
        a = self._ids(ids)
        _check(lib().pkv_mgr_retain(self._h, len(a), a.ctypes.data))

    def release(self, ids) -> None:
        a = self._ids(ids)
        _check(lib().pkv_mgr_release(self._h, len(a), a.ctypes.data))

    def refcount(self, page: int) -> int:
        return int(_check(lib().pkv_mgr_refcount(self._h, page)))

    def note_write(self, plane: int, layer: int, slots) -> None:
        a = self._ids(slots)
        _check(lib().pkv_mgr_note_write(self._h, plane, layer, len(a), a.ctypes.data))

    def published_prefix(self, planes_used: int, page_ids) -> int:
        a = self._ids(page_ids)
        return int(_check(lib().pkv_mgr_published_prefix(self._h, planes_used, a.ctypes.data,
                                                         len(a))))

    def close(self) -> None:
        if self._h:
            lib().pkv_mgr_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
