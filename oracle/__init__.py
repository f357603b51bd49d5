"""CPU oracle for paged-KV decode attention (one or several query tokens per
sequence) and the KV-append slot write.

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` use this package.  The HIP library never
imports, links or calls it, and it shares no code with the library.

``pa_oracle.c`` is the float64 definition (its header states it and the
passages it follows); this module builds it with gcc, loads it with ctypes
and marshals torch/numpy host arrays into it.  ``dense.py`` is an
independent NumPy check used to pin the oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
# PA_ORACLE_LIB selects another build of the same source (the sanitizer test builds one).
_LIB_OVERRIDE = os.environ.get("PA_ORACLE_LIB")
_LIB = _LIB_OVERRIDE or os.path.join(_HERE, "liboracle.so")
_DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_lib = None


def build() -> str:
    """Compile the oracle (gcc -O2, no fast-math) in place; returns the .so path."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-std=c11", "-Wall",
                           "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not _LIB_OVERRIDE and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(_LIB)
        P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.oracle_write_kv.argtypes = [P, P, P, P, P, I64, I64, I, I, I, I]
        lib.oracle_write_kv.restype = I
        lib.oracle_decode.argtypes = [P, P, P, P, P, ctypes.c_float, P, I, I, I, I, I, I, I, P, I64, I]
        lib.oracle_decode.restype = I
        lib.oracle_attend.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, I, I, I, I, I, I, I, I]
        lib.oracle_attend.restype = I
        lib.oracle_rope.argtypes = [P, P, P, I64, I, I, I, ctypes.c_double]
        lib.oracle_rope.restype = I
        lib.oracle_round.argtypes = [P, I64, I, P]
        lib.oracle_round.restype = I
        lib.oracle_widen.argtypes = [P, I64, I, P]
        lib.oracle_widen.restype = None
        lib.oracle_rmsnorm.argtypes = [P, P, P, P, P, I64, I, I, ctypes.c_double]
        lib.oracle_rmsnorm.restype = I
        lib.oracle_pool_init.argtypes = [P, P, I]
        lib.oracle_pool_init.restype = None
        lib.oracle_assign_slots.argtypes = [P, P, P, P, P, P, I, I, I]
        lib.oracle_assign_slots.restype = I
        lib.oracle_release_seqs.argtypes = [P, I, P, P, P, P, I, I, I, I]
        lib.oracle_release_seqs.restype = I
        _lib = lib
    return _lib


def _ptr(x):
    if isinstance(x, torch.Tensor):
        assert x.device.type == "cpu" and x.is_contiguous()
        return ctypes.c_void_p(x.data_ptr())
    assert isinstance(x, np.ndarray) and x.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(x.ctypes.data)


def default_threads() -> int:
    """Host threads to use: the CPU affinity set, capped by OMP_NUM_THREADS when that is set."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(cap))) if cap.isdigit() and int(cap) > 0 else n


def widen(x: torch.Tensor) -> np.ndarray:
    """The oracle's exact widening of a stored tensor to float64 (flattened)."""
    x = x.contiguous()
    out = np.empty(x.numel(), dtype=np.float64)
    _load().oracle_widen(_ptr(x), x.numel(), _DTYPE_CODE[x.dtype], _ptr(out))
    return out


def write_kv(k_new: torch.Tensor, v_new: torch.Tensor, slots: np.ndarray,
             k_pool: torch.Tensor, v_pool: torch.Tensor, *, num_blocks: int, B: int) -> None:
    """Scatter [T, Hkv, D] rows into flat host pools in place (float64-free: bit copies)."""
    T, Hkv, D = k_new.shape
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    assert slots.shape == (T,) and v_new.shape == k_new.shape
    assert k_pool.dtype == k_new.dtype == v_pool.dtype == v_new.dtype
    rc = _load().oracle_write_kv(_ptr(k_new.contiguous()), _ptr(v_new.contiguous()), _ptr(slots),
                                 _ptr(k_pool), _ptr(v_pool), T, num_blocks, B, Hkv, D,
                                 _DTYPE_CODE[k_new.dtype])
    if rc:
        raise ValueError("oracle_write_kv: bad argument")


def decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, block_tables: np.ndarray,
           context_lens: np.ndarray, scale: float, *, Hkv: int, B: int,
           pairs: np.ndarray | None = None, threads: int | None = None) -> np.ndarray:
    """float64 attention output: [S, Hq, D], or [len(pairs), D] for (s, h) pairs."""
    S, Hq, D = q.shape
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    assert bt.shape[0] == S and ctx.shape == (S,)
    if pairs is not None:
        pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
        out = np.empty((pairs.shape[0], D), dtype=np.float64)
        pp, npairs = _ptr(pairs), pairs.shape[0]
    else:
        out = np.empty((S, Hq, D), dtype=np.float64)
        pp, npairs = None, 0
    rc = _load().oracle_decode(_ptr(q.contiguous()), _ptr(k_pool), _ptr(v_pool), _ptr(bt), _ptr(ctx),
                               float(np.float32(scale)), _ptr(out), S, Hq, Hkv, D, B, bt.shape[1],
                               _DTYPE_CODE[q.dtype], pp, npairs, threads or default_threads())
    if rc:
        raise ValueError("oracle_decode: bad argument")
    return out


def attend(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, block_tables: np.ndarray,
           context_lens: np.ndarray, query_start: np.ndarray, scale: float, *, Hkv: int, B: int,
           threads: int | None = None) -> np.ndarray:
    """float64 causal attention of several query tokens per sequence: q is
    [rows, Hq, D], sequence s owning rows query_start[s] .. query_start[s+1]-1
    (its newest positions); returns [rows, Hq, D]."""
    rows, Hq, D = q.shape
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    S = ctx.shape[0]
    assert bt.shape[0] == S and qs.shape == (S + 1,) and int(qs[-1]) == rows
    out = np.empty((rows, Hq, D), dtype=np.float64)
    rc = _load().oracle_attend(_ptr(q.contiguous()), _ptr(k_pool), _ptr(v_pool), _ptr(bt), _ptr(ctx), _ptr(qs),
                               float(np.float32(scale)), _ptr(out), S, Hq, Hkv, D, B, bt.shape[1],
                               _DTYPE_CODE[q.dtype], threads or default_threads())
    if rc:
        raise ValueError("oracle_attend: bad argument")
    return out


def rope(x: torch.Tensor, positions: np.ndarray, theta: float) -> np.ndarray:
    """float64 rotary embedding of x [T, H, D] (storage dtype) at positions [T]."""
    T, H, D = x.shape
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    assert pos.shape == (T,)
    out = np.empty((T, H, D), dtype=np.float64)
    rc = _load().oracle_rope(_ptr(x.contiguous()), _ptr(pos), _ptr(out), T, H, D, _DTYPE_CODE[x.dtype], float(theta))
    if rc:
        raise ValueError("oracle_rope: bad argument")
    return out


def round_to(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """x (float64) rounded once, to nearest with ties to even, into dtype."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    rc = _load().oracle_round(_ptr(x), x.size, _DTYPE_CODE[dtype], _ptr(out))
    if rc:
        raise ValueError("oracle_round: bad dtype")
    return torch.from_numpy(out).to(dtype)  # exact: every value is representable


def rope_case(case, theta: float):
    """The decode step of ``case`` with RoPE applied: q and the new token's K rows
    rotated at position ctx - 1 and rounded into the dtype; the prefill rows are
    taken as already rotated.  Returns a copy of the case with those rows."""
    import dataclasses

    pos = np.maximum(case.context_lens.astype(np.int64) - 1, 0).astype(np.int32)
    dt = case.q.dtype
    q = round_to(rope(case.q, pos, theta), dt)
    k_new = round_to(rope(case.k_new, pos, theta), dt)
    return dataclasses.replace(case, q=q, k_new=k_new)


def build_pools(case):
    """Flat host K/V pools after writing every token of ``case`` (prefill, then the new tokens)."""
    k_pool, v_pool = case.nan_pool(), case.nan_pool()
    write_kv(case.k_prefill, case.v_prefill, case.slot_prefill, k_pool, v_pool,
             num_blocks=case.num_blocks, B=case.B)
    write_kv(case.k_new, case.v_new, case.slot_new, k_pool, v_pool, num_blocks=case.num_blocks, B=case.B)
    return k_pool, v_pool


def decode_case(case, k_pool=None, v_pool=None, pairs=None, threads=None) -> np.ndarray:
    """The oracle's answer for one case (pools built by the oracle's own write if not given)."""
    if k_pool is None:
        k_pool, v_pool = build_pools(case)
    return decode(case.q, k_pool, v_pool, case.block_tables, case.context_lens, case.scale,
                  Hkv=case.Hkv, B=case.B, pairs=pairs, threads=threads)


# --- block pool: a stack of free block ids and its state record (see pa_oracle.c) ---

def pool_init(capacity: int, num_free: int):
    """A fresh pool: (free_ids int32[capacity], state int32[8]) with ids 0 .. num_free-1 free."""
    assert 0 <= num_free <= capacity
    free_ids = np.full(capacity, -7, dtype=np.int32)  # entries at and above top are never read
    state = np.zeros(8, dtype=np.int32)
    _load().oracle_pool_init(_ptr(free_ids), _ptr(state), num_free)
    return free_ids, state


def assign_slots(context_lens: np.ndarray, query_start, block_tables: np.ndarray, free_ids: np.ndarray,
                 state: np.ndarray, *, B: int) -> np.ndarray:
    """Blocks for each sequence's new tokens (block_tables and state updated in
    place) and their slots, int64 [rows].  query_start None: one token per sequence."""
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    S = ctx.shape[0]
    assert block_tables.dtype == np.int32 and block_tables.flags["C_CONTIGUOUS"] and block_tables.shape[0] == S
    assert free_ids.dtype == np.int32 and state.dtype == np.int32 and state.shape == (8,)
    if query_start is None:
        qs, rows = None, S
    else:
        qs = np.ascontiguousarray(query_start, dtype=np.int32)
        assert qs.shape == (S + 1,)
        rows = int(qs[-1])
    slots = np.empty(rows, dtype=np.int64)
    rc = _load().oracle_assign_slots(_ptr(ctx), None if qs is None else _ptr(qs), _ptr(block_tables),
                                     _ptr(free_ids), _ptr(state), _ptr(slots), S, block_tables.shape[1], B)
    if rc:
        raise ValueError("oracle_assign_slots: bad argument")
    return slots


def release_seqs(seq_ids, context_lens: np.ndarray, block_tables: np.ndarray, free_ids: np.ndarray,
                 state: np.ndarray, *, B: int) -> None:
    """Return the listed sequences' blocks to the stack (in place); the stack holds at most len(free_ids)."""
    ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    S = ctx.shape[0]
    assert block_tables.dtype == np.int32 and block_tables.flags["C_CONTIGUOUS"] and block_tables.shape[0] == S
    rc = _load().oracle_release_seqs(_ptr(ids), ids.shape[0], _ptr(ctx), _ptr(block_tables), _ptr(free_ids),
                                     _ptr(state), S, block_tables.shape[1], B, free_ids.shape[0])
    if rc:
        raise ValueError("oracle_release_seqs: bad argument")


# --- RMSNorm ---

def rmsnorm(x: torch.Tensor, weight: torch.Tensor, eps: float, residual: torch.Tensor | None = None):
    """float64 RMSNorm of the rows of x ([T, H], storage dtype) with weight [H]:
    returns y [T, H] before rounding, or (y, new_residual) when residual is given
    (new_residual = x + residual rounded to the dtype, the row that is normalised)."""
    T, H = x.shape
    assert weight.shape == (H,) and weight.dtype == x.dtype
    out = np.empty((T, H), dtype=np.float64)
    res = np.empty((T, H), dtype=np.float64) if residual is not None else None
    if residual is not None:
        assert residual.shape == x.shape and residual.dtype == x.dtype
    rc = _load().oracle_rmsnorm(_ptr(x.contiguous()), None if residual is None else _ptr(residual.contiguous()),
                                _ptr(weight.contiguous()), _ptr(out), None if res is None else _ptr(res), T, H,
                                _DTYPE_CODE[x.dtype], float(np.float32(eps)))
    if rc:
        raise ValueError("oracle_rmsnorm: bad argument")
    return out if residual is None else (out, res)
