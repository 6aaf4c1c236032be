"""Seeded synthetic inputs for paged-KV attention.

This module is the only code shared by the GPU library's tests/benchmark and
the oracle. It holds none of the method's arithmetic: it draws random values,
picks physical pages for each request (the scheduler's job: allocate KV pages
and hand out the slots to write, "Faster fuzzy minds", section "When scheduler
does the work") and lists which tokens go to which slot. Attention, the
gather through the page table and the slot scatter itself live on each side
separately.

Recipe (the shapes and distributions of the workloads the pages describe):

* values: Q, K, V ~ N(0, 1) drawn in fp32 (numpy ``default_rng(seed)``), then
  rounded to the storage dtype (bf16 by round-to-nearest-even); an optional
  ``q_scale`` multiplies Q before rounding (the "peaked" variant);
* pages: a seeded permutation of the pool's page ids, handed out in request
  order, position order; pool size defaults to 1.125 x the pages in use;
* aliasing: the first ``k_r`` full pages of request ``r`` point into one
  shared chain of pages (a nested common prefix), ``k_r = min(floor(f *
  ceil(prompt/16)), floor(prompt/16))``; the page holding the newest token is
  always private;
* poison: every slot not written holds NaN, so a stray read poisons the output.
"""
from __future__ import annotations

import dataclasses
from typing import Sequence

import numpy as np

NAN_BF16 = np.uint16(0x7FC0)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 -> bf16 (round-to-nearest-even) and return the raw bits."""
    import torch  # local: torch only for its bf16 rounding

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 raw bits to fp32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def draw(rng: np.random.Generator, shape, dtype: str, scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) in the storage representation (float32 or bf16 bits)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x = (x * np.float32(scale)).astype(np.float32)
    return x if dtype == "f32" else bf16_bits(x)


def poison_value(dtype: str):
    return np.float32(np.nan) if dtype == "f32" else NAN_BF16


def storage_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


@dataclasses.dataclass
class Layout:
    """Static description of a multi-plane pool."""

    dtype: str            # "f32" | "bf16"
    page_size: int
    num_pages: int
    num_kv_heads: int
    head_dim: int
    num_planes: int = 1
    num_layers: int = 1
    rec_first: int = 0    # planes >= 1 hold layers [rec_first, rec_first+rec_count)
    rec_count: int | None = None  # default: every layer from rec_first on

    def __post_init__(self):
        if self.rec_count is None:
            self.rec_count = self.num_layers - self.rec_first

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def page_bytes(self) -> int:
        """Bytes of one page of one bank, K and V together."""
        return 2 * self.num_kv_heads * self.page_size * self.head_dim * self.elem_bytes


def allocate_pages(rng: np.random.Generator, seq_lens: Sequence[int], page_size: int,
                   num_pages: int | None = None, shared_pages: Sequence[int] | None = None,
                   stride: int | None = None, spare: float = 1.125):
    """Hand out physical pages.

    Request r needs ceil(n_r / P) pages; its first shared_pages[r] of them come
    from one shared chain, the rest are its own. Physical ids are a seeded
    permutation of [0, num_pages) taken in order: the chain first, then each
    request's private pages in position order. Unused table entries are 0
    (never read: a kernel only reads the first ceil(n_r / P) entries).

    Returns (page_table [B, stride] int32, num_pages, chain ids).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = len(seq_lens)
    need = -(-seq_lens // page_size)
    shared = np.zeros(B, np.int64) if shared_pages is None else np.asarray(shared_pages, np.int64)
    assert np.all(shared <= need)
    chain_len = int(shared.max()) if B else 0
    used = chain_len + int((need - shared).sum())
    if num_pages is None:
        num_pages = max(1, int(np.ceil(used * spare)))
    assert used <= num_pages, f"pool of {num_pages} pages cannot hold {used}"
    if stride is None:
        stride = max(1, int(need.max()) if B else 1)
    perm = rng.permutation(num_pages).astype(np.int32)
    chain = perm[:chain_len]
    cursor = chain_len
    table = np.zeros((B, stride), np.int32)
    for r in range(B):
        k = int(shared[r])
        table[r, :k] = chain[:k]
        own = int(need[r] - k)
        table[r, k:k + own] = perm[cursor:cursor + own]
        cursor += own
    return table, num_pages, chain


def slots_of(page_table: np.ndarray, r: int, positions: np.ndarray, page_size: int) -> np.ndarray:
    """The slots the scheduler hands store_kv for positions of request r."""
    positions = np.asarray(positions, dtype=np.int64)
    return (page_table[r, positions // page_size].astype(np.int64) * page_size
            + positions % page_size).astype(np.int32)


def slots_of_last(page_table: np.ndarray, seq_lens: Sequence[int], page_size: int) -> np.ndarray:
    """Slot of each request's newest token (position n - 1); -1 for n = 0."""
    out = np.full(len(seq_lens), -1, np.int32)
    for r, n in enumerate(seq_lens):
        if n > 0:
            out[r] = slots_of(page_table, r, np.array([int(n) - 1]), page_size)[0]
    return out


def alias_pages(prompt_lens: Sequence[int], frac: float, page_size: int) -> np.ndarray:
    """Shared full pages per request for an aliased-prefix workload."""
    p = np.asarray(prompt_lens, np.int64)
    k = np.minimum(np.floor(frac * (-(-p // page_size))).astype(np.int64), p // page_size)
    return k


@dataclasses.dataclass
class BankData:
    """What one (plane, layer) bank receives in one decode step."""

    fill_k: np.ndarray     # [T, Hkv, D] context tokens (positions < n - 1)
    fill_v: np.ndarray
    fill_slots: np.ndarray  # [T]
    new_k: np.ndarray      # [B, Hkv, D] the token at position n - 1
    new_v: np.ndarray
    new_slots: np.ndarray  # [B]
    q: np.ndarray          # [B, Hq, D]
    logical_k: list | None  # per request [n_r, Hkv, D] (whole context, new token included)
    logical_v: list | None


@dataclasses.dataclass
class DecodeCase:
    layout: Layout
    num_q_heads: int
    seq_lens: np.ndarray   # [B] int32, counts the new token
    page_table: np.ndarray  # [B, stride] int32
    shared: np.ndarray     # [B] shared pages per request
    banks: dict            # (plane, layer) -> BankData

    @property
    def batch(self) -> int:
        return len(self.seq_lens)


def make_decode_case(seed: int, dtype: str, batch: int, seq_range: tuple[int, int],
                     num_q_heads: int, num_kv_heads: int, head_dim: int,
                     page_size: int = 16, num_pages: int | None = None,
                     num_planes: int = 1, num_layers: int = 1, rec_first: int = 0,
                     rec_count: int | None = None, alias_frac: float = 0.0,
                     planes_layers: Sequence[tuple[int, int]] = ((0, 0),),
                     q_scale: float = 1.0, keep_logical: bool = True,
                     seq_lens: Sequence[int] | None = None,
                     page_table: np.ndarray | None = None,
                     shared: Sequence[int] | None = None) -> DecodeCase:
    """Decode workload: every request holds n_r - 1 context tokens and gets one
    new token at position n_r - 1 (written through its slot, then attended).

    seq_range bounds the *prompt* when alias_frac > 0 (n = prompt + 1), else
    the sequence length itself (uniform integers, inclusive).
    """
    rng = np.random.default_rng(seed)
    if rec_count is None:
        rec_count = num_layers - rec_first
    if seq_lens is None:
        lo, hi = seq_range
        if alias_frac > 0:
            prompts = rng.integers(lo, hi + 1, size=batch)
            seq_lens = prompts + 1
        else:
            seq_lens = rng.integers(lo, hi + 1, size=batch)
    seq_lens = np.asarray(seq_lens, np.int32)
    if shared is None:
        shared = alias_pages(seq_lens - 1, alias_frac, page_size) if alias_frac > 0 else \
            np.zeros(batch, np.int64)
    shared = np.asarray(shared, np.int64)
    if page_table is None:
        page_table, num_pages, _ = allocate_pages(rng, seq_lens, page_size, num_pages, shared)
    assert num_pages is not None
    layout = Layout(dtype, page_size, num_pages, num_kv_heads, head_dim, num_planes,
                    num_layers, rec_first, rec_count)
    banks = {}
    for (plane, layer) in planes_layers:
        banks[(plane, layer)] = _bank_data(rng, layout, num_q_heads, seq_lens, page_table,
                                           shared, q_scale, keep_logical)
    return DecodeCase(layout, num_q_heads, seq_lens, page_table, shared, banks)


def _bank_data(rng, layout: Layout, Hq: int, seq_lens, page_table, shared, q_scale,
               keep_logical) -> BankData:
    P, Hkv, D, dt = layout.page_size, layout.num_kv_heads, layout.head_dim, layout.dtype
    B = len(seq_lens)
    chain_tokens = int(shared.max()) * P if B else 0
    chain_k = draw(rng, (chain_tokens, Hkv, D), dt)
    chain_v = draw(rng, (chain_tokens, Hkv, D), dt)
    fk, fv, fs, lk, lv = [], [], [], [], []
    # The shared chain is written once, by the first request that holds all of it.
    if chain_tokens:
        owner = int(np.argmax(shared))
        fk.append(chain_k)
        fv.append(chain_v)
        fs.append(slots_of(page_table, owner, np.arange(chain_tokens), P))
    new_k = np.empty((B, Hkv, D), storage_dtype(dt))
    new_v = np.empty_like(new_k)
    new_slots = np.empty(B, np.int32)
    for r in range(B):
        n = int(seq_lens[r])
        s0 = int(shared[r]) * P
        own_k = draw(rng, (n - s0, Hkv, D), dt)
        own_v = draw(rng, (n - s0, Hkv, D), dt)
        if n - 1 > s0:
            fk.append(own_k[:n - 1 - s0])
            fv.append(own_v[:n - 1 - s0])
            fs.append(slots_of(page_table, r, np.arange(s0, n - 1), P))
        if n >= 1:
            new_k[r] = own_k[n - 1 - s0]
            new_v[r] = own_v[n - 1 - s0]
            new_slots[r] = slots_of(page_table, r, np.array([n - 1]), P)[0]
        else:
            new_k[r] = 0
            new_v[r] = 0
            new_slots[r] = -1
        if keep_logical:
            lk.append(np.concatenate([chain_k[:s0], own_k]))
            lv.append(np.concatenate([chain_v[:s0], own_v]))
    q = draw(rng, (B, Hq, D), dt, q_scale)
    sd = storage_dtype(dt)

    def cat(parts):
        return np.concatenate(parts) if parts else np.zeros((0, Hkv, D), sd)

    return BankData(cat(fk), cat(fv),
                    np.concatenate(fs).astype(np.int32) if fs else np.zeros(0, np.int32),
                    new_k, new_v, new_slots, q,
                    lk if keep_logical else None, lv if keep_logical else None)


@dataclasses.dataclass
class PrefillCase:
    """Prompts whose K/V and Q are known; the chunk schedule is chosen later."""

    layout: Layout
    num_q_heads: int
    prompt_lens: np.ndarray  # [B]
    page_table: np.ndarray   # [B, stride]
    k: list                  # per prompt [n, Hkv, D] logical K (storage dtype)
    v: list
    q: list                  # per prompt [n, Hq, D]
    shared: np.ndarray       # [B] shared pages


def make_prefill_case(seed: int, dtype: str, prompt_lens: Sequence[int], num_q_heads: int,
                      num_kv_heads: int, head_dim: int, page_size: int = 16,
                      num_pages: int | None = None, shared_prefix_tokens: int = 0,
                      q_scale: float = 1.0) -> PrefillCase:
    """Prompts with N(0,1) K/V/Q. If shared_prefix_tokens > 0 (a multiple of the
    page size), every prompt's first tokens are one common prefix whose pages
    all prompts alias (the shared-prefix variant); else every page is private."""
    rng = np.random.default_rng(seed)
    prompt_lens = np.asarray(prompt_lens, np.int32)
    B = len(prompt_lens)
    assert shared_prefix_tokens % page_size == 0
    shared = np.full(B, shared_prefix_tokens // page_size, np.int64)
    page_table, num_pages, _ = allocate_pages(rng, prompt_lens, page_size, num_pages, shared)
    layout = Layout(dtype, page_size, num_pages, num_kv_heads, head_dim)
    pk = draw(rng, (shared_prefix_tokens, num_kv_heads, head_dim), dtype)
    pv = draw(rng, (shared_prefix_tokens, num_kv_heads, head_dim), dtype)
    ks, vs, qs = [], [], []
    for r in range(B):
        n = int(prompt_lens[r])
        k = draw(rng, (n, num_kv_heads, head_dim), dtype)
        v = draw(rng, (n, num_kv_heads, head_dim), dtype)
        k[:shared_prefix_tokens] = pk[:n]
        v[:shared_prefix_tokens] = pv[:n]
        ks.append(k)
        vs.append(v)
        qs.append(draw(rng, (n, num_q_heads, head_dim), dtype, q_scale))
    return PrefillCase(layout, num_q_heads, prompt_lens, page_table, ks, vs, qs, shared)


@dataclasses.dataclass
class Chunk:
    """One varlen call: write these tokens, then attend with these query rows."""

    k: np.ndarray          # [T, Hkv, D] tokens written by this chunk
    v: np.ndarray
    slots: np.ndarray      # [T]
    q: np.ndarray          # [T, Hq, D] packed query rows (same tokens)
    cu_q_lens: np.ndarray  # [B + 1]
    seq_lens: np.ndarray   # [B] = tokens of the prompt held after this chunk
    rows: list             # (request, first position) per request


def chunk_schedule(case: PrefillCase, chunk: int, start: Sequence[int] | None = None,
                   skip_shared_writes: bool = True) -> list[Chunk]:
    """Split prompts into chunks of at most `chunk` tokens per request, from
    position start[r] (default 0) on. Chunk c of every request goes into one
    varlen call. Tokens in shared pages are written by request 0 only."""
    B = len(case.prompt_lens)
    P = case.layout.page_size
    start = np.zeros(B, np.int64) if start is None else np.asarray(start, np.int64)
    out = []
    pos = start.copy()
    while np.any(pos < case.prompt_lens):
        ks, vs, ss, qs, cu, sl, rows = [], [], [], [], [0], [], []
        for r in range(B):
            n = int(case.prompt_lens[r])
            lo = int(pos[r])
            hi = min(lo + chunk, n)
            positions = np.arange(lo, hi)
            qs.append(case.q[r][lo:hi])
            writes = positions
            if skip_shared_writes and r > 0:
                writes = positions[positions >= case.shared[r] * P]
            ks.append(case.k[r][writes])
            vs.append(case.v[r][writes])
            ss.append(slots_of(case.page_table, r, writes, P))
            cu.append(cu[-1] + (hi - lo))
            sl.append(hi)
            rows.append((r, lo))
            pos[r] = hi
        out.append(Chunk(np.concatenate(ks), np.concatenate(vs),
                         np.concatenate(ss).astype(np.int32), np.concatenate(qs),
                         np.asarray(cu, np.int32), np.asarray(sl, np.int32), rows))
    return out


def prefix_writes(case: PrefillCase, upto: Sequence[int]):
    """Tokens [0, upto[r]) of every prompt as one write (shared pages once)."""
    P = case.layout.page_size
    ks, vs, ss = [], [], []
    for r in range(len(case.prompt_lens)):
        positions = np.arange(int(upto[r]))
        if r > 0:
            positions = positions[positions >= case.shared[r] * P]
        ks.append(case.k[r][positions])
        vs.append(case.v[r][positions])
        ss.append(slots_of(case.page_table, r, positions, case.layout.page_size))
    return np.concatenate(ks), np.concatenate(vs), np.concatenate(ss).astype(np.int32)


@dataclasses.dataclass
class LotusCase:
    """A latent block of `block` positions after each request's prompt, run
    for several passes: the prompt's K/V are written once; every pass brings
    new K/V and Q for the block's rows (request-major, packed)."""

    layout: Layout
    num_q_heads: int
    prompt_lens: np.ndarray  # [B]
    block: int
    page_table: np.ndarray   # [B, stride], room for prompt + block
    prompt_k: list           # per request [prompt, Hkv, D]
    prompt_v: list
    prompt_slots: np.ndarray  # [sum prompt] slots of the prompt tokens, request-major
    block_slots: np.ndarray  # [B * block] slots of the block positions (fixed)
    passes: list             # per pass (k [B*block, Hkv, D], v, q [B*block, Hq, D])


def make_lotus_case(seed: int, dtype: str, prompt_lens: Sequence[int], block: int,
                    num_passes: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    page_size: int = 16, q_scale: float = 1.0) -> LotusCase:
    rng = np.random.default_rng(seed)
    prompt_lens = np.asarray(prompt_lens, np.int32)
    B = len(prompt_lens)
    total = prompt_lens + block
    page_table, num_pages, _ = allocate_pages(rng, total, page_size)
    layout = Layout(dtype, page_size, num_pages, num_kv_heads, head_dim)
    pk, pv, ps, bs = [], [], [], []
    for r in range(B):
        n = int(prompt_lens[r])
        pk.append(draw(rng, (n, num_kv_heads, head_dim), dtype))
        pv.append(draw(rng, (n, num_kv_heads, head_dim), dtype))
        ps.append(slots_of(page_table, r, np.arange(n), page_size))
        bs.append(slots_of(page_table, r, np.arange(n, n + block), page_size))
    passes = []
    for _ in range(num_passes):
        passes.append((draw(rng, (B * block, num_kv_heads, head_dim), dtype),
                       draw(rng, (B * block, num_kv_heads, head_dim), dtype),
                       draw(rng, (B * block, num_q_heads, head_dim), dtype, q_scale)))
    return LotusCase(layout, num_q_heads, prompt_lens, block, page_table, pk, pv,
                     np.concatenate(ps).astype(np.int32), np.concatenate(bs).astype(np.int32),
                     passes)


def device_normal_(t, seed: int, scale: float = 1.0):
    """Fill a device tensor in place with N(0, scale^2) from a seeded torch
    generator on its device (for pools too large to draw on the host)."""
    import torch

    g = torch.Generator(device=t.device)
    g.manual_seed(seed)
    flat = t.view(-1)
    step = 1 << 28  # draw in slices to bound the temporary
    for i in range(0, flat.numel(), step):
        flat[i:i + step].normal_(0.0, scale, generator=g)
    return t
