"""Dense, non-paged attention in NumPy float64: an independent check of the oracle.

``causal_attention`` / ``dense_multi`` do the same for several query tokens
per sequence, with the causal mask applied to a full score matrix (the
oracle instead truncates each row's sum).

TEST INFRASTRUCTURE.  It never sees a pool or a block table: it takes each
sequence's K/V rows in logical order, repeats every kv-head G times for the
query heads that share it, and evaluates softmax(q K^T * scale) V with NumPy
matmuls (a different summation order from the oracle's loops).
"""
from __future__ import annotations

import numpy as np
import torch


def _f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def attention(q_row: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q k^T * scale) v for one query row q [D], keys k [L, D], values v [L, D]."""
    if k.shape[0] == 0:
        return np.zeros(q_row.shape[-1])
    z = (k @ q_row) * float(scale)
    w = np.exp(z - z.max())
    return (w @ v) / w.sum()


def dense_case(case) -> np.ndarray:
    """[S, Hq, D] float64 from the drawn logical rows of ``case``."""
    q = _f64(case.q)
    out = np.zeros((case.S, case.Hq, case.D))
    for s in range(case.S):
        k, v = case.logical_kv(s)
        k = np.repeat(_f64(k), case.G, axis=1)  # [L, Hq, D]
        v = np.repeat(_f64(v), case.G, axis=1)
        for h in range(case.Hq):
            out[s, h] = attention(q[s, h], k[:, h, :], v[:, h, :], case.scale)
    return out


def causal_attention(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """The n newest positions of a sequence attending causally, as one masked
    matrix product per head: q_rows [n, D], k and v [L, D] (n <= L); row i sits
    at position L - n + i and may see t <= L - n + i.  Returns [n, D]."""
    n, L = q_rows.shape[0], k.shape[0]
    z = (q_rows @ k.T) * float(scale)  # [n, L]
    pos = np.arange(L)[None, :]
    row_pos = (L - n + np.arange(n))[:, None]
    z = np.where(pos <= row_pos, z, -np.inf)
    w = np.exp(z - z.max(axis=1, keepdims=True))
    return (w @ v) / w.sum(axis=1, keepdims=True)


def dense_multi(mcase) -> np.ndarray:
    """[rows, Hq, D] float64 for a batch with several query tokens per sequence."""
    case = mcase.base
    q = _f64(mcase.q)
    qs = mcase.query_start
    out = np.zeros((int(qs[-1]), case.Hq, case.D))
    for s in range(case.S):
        a, b = int(qs[s]), int(qs[s + 1])
        if a == b:
            continue
        k, v = case.logical_kv(s)
        k = np.repeat(_f64(k), case.G, axis=1)
        v = np.repeat(_f64(v), case.G, axis=1)
        for h in range(case.Hq):
            out[a:b, h] = causal_attention(q[a:b, h], k[:, h, :], v[:, h, :], case.scale)
    return out
