"""Brute-force attention on the logical (never paged) K/V, for pinning the oracle.

Dense masked softmax as matrix products: S = scale * Q K^T, keys after a query's
position masked to -inf, normalised with scipy's logsumexp. It never sees a
page table or a slot, so a mistake in the oracle's paging (gather, layout,
slot arithmetic) or in its head/position mapping shows up as a mismatch.
"""
from __future__ import annotations

import numpy as np
from scipy.special import logsumexp


def to_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, positions: np.ndarray,
              scale: float):
    """q [R, Hq, D] at `positions` [R]; k, v [n, Hkv, D] logical context.

    Returns out [R, Hq, D], lse [R, Hq] (fp64)."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    R, Hq, D = q.shape
    n, Hkv, _ = k.shape
    G = Hq // Hkv
    out = np.zeros((R, Hq, D))
    lse = np.full((R, Hq), -np.inf)
    if n == 0 or R == 0:
        return out, lse
    kk = np.repeat(k, G, axis=1)          # [n, Hq, D]: q head h uses kv head h // G
    vv = np.repeat(v, G, axis=1)
    s = scale * np.einsum("rhd,nhd->rhn", q, kk)
    mask = np.arange(n)[None, None, :] > np.asarray(positions)[:, None, None]
    s = np.where(mask, -np.inf, s)
    lse = logsumexp(s, axis=-1)
    w = np.exp(s - lse[..., None])
    out = np.einsum("rhn,nhd->rhd", w, vv)
    return out, lse
