"""Thin Python binding of libpagedattn (ctypes).

Argument marshalling only: shapes, dtypes, devices and the current HIP stream
are checked and passed through; every step of the computation runs in the
library's kernels.  There is no fallback: if the library is not built,
every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

# PAGEDATTN_LIB selects another build of the library (for example a differently tuned one).
_LIB_PATH = os.environ.get("PAGEDATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                           "libpagedattn.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_CAPACITY = range(6)
# PA_ABI_VERSION of the C interface the signatures below are written for; a
# library built from other sources is refused when it is loaded.
ABI_VERSION = 3
_DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_ELT = {torch.float32: 4, torch.float16: 2, torch.bfloat16: 2}

EXPORTS = (
    "pa_write_kv",
    "pa_decode",
    "pa_decode_noalloc",
    "pa_decode_ex",
    "pa_decode_append",
    "pa_attend",
    "pa_attend_workspace_bytes",
    "pa_rope",
    "pa_decode_rope_append",
    "pa_decode_workspace_bytes",
    "pa_decode_workspace_bytes_ex",
    "pa_pool_init",
    "pa_assign_slots",
    "pa_release_seqs",
    "pa_acct_init",
    "pa_acct_admit",
    "pa_acct_retire",
    "pa_pool_telemetry",
    "pa_rmsnorm",
    "pa_read_probe",
    "pa_workspace_sync_bytes",
    "pa_status_string",
    "pa_abi_version",
)


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class PoolAcct(ctypes.Structure):
    """pa_pool_acct_t: host-side worst-case admission accounting."""
    _fields_ = [(n, ctypes.c_int64) for n in ("num_blocks", "block_size", "bytes_per_block", "reserved_blocks",
                                              "peak_reserved_blocks", "admitted", "refused")]


class PoolTelemetry(ctypes.Structure):
    """pa_pool_telemetry_t."""
    _fields_ = ([(n, ctypes.c_int64) for n in ("capacity_blocks", "free_blocks", "used_blocks", "peak_used_blocks",
                                               "capacity_bytes", "used_bytes", "reserved_blocks",
                                               "peak_reserved_blocks", "admitted", "tokens_stored", "empty_slots")]
                + [("occupancy", ctypes.c_double)]
                + [(n, ctypes.c_int64) for n in ("refused_admissions", "refused_sequences", "refused_releases")])

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _t in self._fields_}


class CapacityError(RuntimeError):
    """An admission the pool cannot promise (PA_ERR_CAPACITY)."""


class PagedAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m paged_kv_decode_slot_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        DP = ctypes.POINTER(CacheDesc)
        L.pa_write_kv.argtypes = [P, P, P, P, P, I32, DP, P]
        L.pa_write_kv.restype = ctypes.c_int
        L.pa_decode.argtypes = [P, P, P, P, P, ctypes.c_float, P, I32, I32, I32, DP, P, SZ, P]
        L.pa_decode.restype = ctypes.c_int
        L.pa_decode_noalloc.argtypes = [P, P, P, P, P, ctypes.c_float, P, I32, I32, I32, DP, P]
        L.pa_decode_noalloc.restype = ctypes.c_int
        L.pa_decode_ex.argtypes = [P, P, P, P, P, ctypes.c_float, P, I32, I32, I32, DP, P, SZ, I32, P]
        L.pa_decode_ex.restype = ctypes.c_int
        L.pa_decode_append.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, P, I32, I32, I32, DP, P, SZ, I32, P]
        L.pa_decode_append.restype = ctypes.c_int
        L.pa_attend.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, I32, I32, I32, I32, I32, DP, P, SZ, I32, P]
        L.pa_attend.restype = ctypes.c_int
        L.pa_attend_workspace_bytes.argtypes = [I32, I32, I32, DP, I32]
        L.pa_rope.argtypes = [P, P, P, I32, I32, I32, I32, I32, ctypes.c_float, P]
        L.pa_rope.restype = ctypes.c_int
        L.pa_decode_rope_append.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_float, P, I32, I32, I32,
                                            DP, P, SZ, I32, P]
        L.pa_decode_rope_append.restype = ctypes.c_int
        L.pa_attend_workspace_bytes.restype = SZ
        L.pa_decode_workspace_bytes.argtypes = [I32, I32, I32, DP]
        L.pa_decode_workspace_bytes.restype = SZ
        L.pa_decode_workspace_bytes_ex.argtypes = [I32, I32, I32, DP, I32]
        L.pa_decode_workspace_bytes_ex.restype = SZ
        L.pa_status_string.argtypes = [ctypes.c_int]
        L.pa_status_string.restype = ctypes.c_char_p
        L.pa_abi_version.argtypes = []
        L.pa_abi_version.restype = I32
        L.pa_read_probe.argtypes = [P, P, ctypes.c_int64, I32, P, I32, P]
        L.pa_read_probe.restype = ctypes.c_int
        L.pa_workspace_sync_bytes.argtypes = []
        L.pa_workspace_sync_bytes.restype = SZ
        L.pa_rmsnorm.argtypes = [P, P, P, P, ctypes.c_int64, I32, ctypes.c_float, I32, P]
        L.pa_rmsnorm.restype = ctypes.c_int
        L.pa_pool_init.argtypes = [P, P, I32, I32, P]
        L.pa_pool_init.restype = ctypes.c_int
        L.pa_assign_slots.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, P]
        L.pa_assign_slots.restype = ctypes.c_int
        L.pa_release_seqs.argtypes = [P, I32, P, P, P, P, I32, I32, I32, I32, P]
        L.pa_release_seqs.restype = ctypes.c_int
        AP = ctypes.POINTER(PoolAcct)
        L.pa_acct_init.argtypes = [AP, ctypes.c_int64, I32, ctypes.c_int64]
        L.pa_acct_init.restype = ctypes.c_int
        L.pa_acct_admit.argtypes = [AP, ctypes.c_int64]
        L.pa_acct_admit.restype = ctypes.c_int
        L.pa_acct_retire.argtypes = [AP, ctypes.c_int64]
        L.pa_acct_retire.restype = ctypes.c_int
        L.pa_pool_telemetry.argtypes = [AP, P, ctypes.c_int64, ctypes.POINTER(PoolTelemetry)]
        L.pa_pool_telemetry.restype = ctypes.c_int
        got = L.pa_abi_version()
        if got != ABI_VERSION:
            raise RuntimeError(f"{_LIB_PATH} has ABI {got}; this binding marshals ABI {ABI_VERSION}: rebuild it")
        _lib = L
    return _lib


def library_path() -> str:
    return _LIB_PATH


def _check(fn: str, status: int) -> None:
    if status != PA_OK:
        msg = lib().pa_status_string(status).decode()
        if status == PA_ERR_CAPACITY:
            raise CapacityError(f"{fn}: {msg} (status {status})")
        if status in (PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE):
            raise ValueError(f"{fn}: {msg} (status {status})")
        raise PagedAttnError(fn, status, msg)


def cache_shapes(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype):
    """Shapes of the K and V pools: [num_blocks, Hkv, block_size/16, 16*head_dim] each.

    The last dimension is one 16-token slab; the element order inside a slab is
    the library's (see include/pagedattn.h).
    """
    if block_size % 16:
        raise ValueError("block_size must be a multiple of 16")
    shape = (num_blocks, num_kv_heads, block_size // 16, 16 * head_dim)
    return shape, shape


def new_cache(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
              dtype: torch.dtype, device) -> tuple[torch.Tensor, torch.Tensor]:
    """Uninitialised K and V pools (torch device memory) in the library's layout."""
    ks, vs = cache_shapes(num_blocks, block_size, num_kv_heads, head_dim, dtype)
    return (torch.empty(ks, dtype=dtype, device=device), torch.empty(vs, dtype=dtype, device=device))


def cache_desc(k_cache: torch.Tensor, v_cache: torch.Tensor) -> CacheDesc:
    """The pool geometry, read from the pools' shapes [NB, Hkv, B/16, 16*D]."""
    if k_cache.dim() != 4 or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache must both be [num_blocks, Hkv, block_size/16, 16*head_dim]")
    if k_cache.dtype not in _DTYPE_CODE or v_cache.dtype != k_cache.dtype:
        raise ValueError("caches must share one of float32/float16/bfloat16")
    NB, Hkv, NS, SL = k_cache.shape
    if SL % 16:
        raise ValueError("the last dimension must be 16 * head_dim")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous")
    return CacheDesc(NB, NS * 16, Hkv, SL // 16, _DTYPE_CODE[k_cache.dtype])


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# Workspaces start zero-filled: their first pa_workspace_sync_bytes() bytes are the
# library's synchronisation words, which must be zero before the first call and
# which every call leaves zero.  One workspace per (device, stream) is kept and
# grown for the calls that do not bring their own; calls on one stream never
# overlap, so they can share it.
_WS_CACHE: dict = {}


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled uint8 workspace of nbytes (at least 1), ready for any call."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _workspace(dev: torch.device, need: int, workspace, own: bool) -> torch.Tensor:
    if workspace is not None:
        if workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the same device")
        return workspace
    if own:  # a prepared call keeps its own (it may be captured in a graph)
        return new_workspace(need, dev)
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    ws = _WS_CACHE.get(key)
    if ws is None or ws.numel() < need:
        ws = new_workspace(max(need, 2 * (0 if ws is None else ws.numel())), dev)
        _WS_CACHE[key] = ws
    return ws


def _dev(*ts: torch.Tensor) -> torch.device:
    d = ts[0].device
    if d.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    for t in ts:
        if t.device != d:
            raise ValueError("all tensors must be on one device")
    return d


def _write_args(k_new, v_new, slot_mapping, k_cache, v_cache):
    desc = cache_desc(k_cache, v_cache)
    dev = _dev(k_new, v_new, slot_mapping, k_cache, v_cache)
    if k_new.shape != v_new.shape or k_new.dim() != 3 or tuple(k_new.shape[1:]) != (desc.num_kv_heads, desc.head_dim):
        raise ValueError("k_new/v_new must be [T, Hkv, D]")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise ValueError("k_new/v_new dtype must match the caches")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (k_new.shape[0],):
        raise ValueError("slot_mapping must be int64 [T]")
    if not (k_new.is_contiguous() and v_new.is_contiguous() and slot_mapping.is_contiguous()):
        raise ValueError("inputs must be contiguous")
    args = (k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            int(k_new.shape[0]), ctypes.byref(desc), _stream(dev))
    return dev, args, (k_new, v_new, slot_mapping, k_cache, v_cache, desc)


def write_kv(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
             k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    """Append: copy each token's K/V rows ([T, Hkv, D]) into slot_mapping[t] (int64; < 0 skips)."""
    dev, args, _keep = _write_args(k_new, v_new, slot_mapping, k_cache, v_cache)
    with torch.cuda.device(dev):
        st = lib().pa_write_kv(*args)
    _check("pa_write_kv", st)


def workspace_bytes(num_seqs: int, num_q_heads: int, max_blocks_per_seq: int, desc: CacheDesc,
                    num_workers: int = 0) -> int:
    return int(lib().pa_decode_workspace_bytes_ex(num_seqs, num_q_heads, max_blocks_per_seq,
                                                  ctypes.byref(desc), num_workers))


def _decode_args(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_workers, workspace,
                 own_workspace=False):
    desc = cache_desc(k_cache, v_cache)
    dev = _dev(q, k_cache, v_cache, block_tables, context_lens)
    if q.dim() != 3 or q.shape[2] != desc.head_dim or q.dtype != k_cache.dtype or not q.is_contiguous():
        raise ValueError("q must be contiguous [S, Hq, D] in the cache dtype")
    S, Hq, D = q.shape
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S \
            or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [S, max_blocks_per_seq]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (S,) or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32 [S]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != dev:
        raise ValueError("out must be contiguous and shaped like q")
    maxblk = int(block_tables.shape[1])
    need = workspace_bytes(S, Hq, maxblk, desc, num_workers)
    workspace = _workspace(dev, need, workspace, own_workspace)
    args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(),
            ctypes.c_float(scale), out.data_ptr(), S, Hq, maxblk, ctypes.byref(desc), workspace.data_ptr(),
            workspace.numel(), int(num_workers), _stream(dev))
    return dev, out, args, (q, k_cache, v_cache, block_tables, context_lens, out, workspace, desc)


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
           context_lens: torch.Tensor, scale: float, out: torch.Tensor | None = None, *,
           num_workers: int = 0, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Decode attention of q [S, Hq, D] over the paged caches; returns out [S, Hq, D].

    num_workers: 0 automatic, -1 one worker per (sequence, kv-head slice), >0 that many
    workers (a worker is a workgroup with one wavefront per kv-head of a slice).
    workspace: optional uint8 device tensor whose first pa_workspace_sync_bytes() bytes
    are zero before its first use (new_workspace() makes one); when not given, a
    zero-filled workspace kept for the current stream is used.
    """
    dev, out, args, _keep = _decode_args(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                                         num_workers, workspace)
    with torch.cuda.device(dev):
        st = lib().pa_decode_ex(*args)
    _check("pa_decode", st)
    return out


def prepare_write_kv(k_new, v_new, slot_mapping, k_cache, v_cache):
    """Validate once; return a no-argument callable that issues the same pa_write_kv
    on the stream that is current now (for tight loops)."""
    _dev_, args, keep = _write_args(k_new, v_new, slot_mapping, k_cache, v_cache)
    fn = lib().pa_write_kv

    def call():
        _check("pa_write_kv", fn(*args))
        return keep

    return call


def prepare_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out=None, *, num_workers=0,
                   workspace=None):
    """Validate once (allocating out and the workspace if not given); return a
    no-argument callable that issues the same pa_decode_ex on the stream that
    is current now, and returns out."""
    _dev_, out, args, keep = _decode_args(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                                          num_workers, workspace, own_workspace=True)
    fn = lib().pa_decode_ex

    def call():
        _check("pa_decode", fn(*args))
        return keep[5]

    return call


def _append_args(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out, num_workers, workspace,
                 own_workspace=False):
    dev, out, dargs, keep = _decode_args(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                                         num_workers, workspace, own_workspace)
    desc = keep[7]
    S = q.shape[0]
    for t in (k_new, v_new):
        if t.device != dev or t.dtype != q.dtype or not t.is_contiguous() \
                or tuple(t.shape) != (S, desc.num_kv_heads, desc.head_dim):
            raise ValueError("k_new/v_new must be contiguous [S, Hkv, D] in the cache dtype on the same device")
    # pa_decode_ex arguments are (q, k, v, bt, ctx, scale, out, S, Hq, maxblk, desc, ws, ws_bytes, workers, stream)
    q_p, k_p, v_p, bt_p, ctx_p, sc, out_p, S_, Hq, maxblk, descp, ws_p, ws_n, wk, st = dargs
    args = (q_p, k_new.data_ptr(), v_new.data_ptr(), k_p, v_p, bt_p, ctx_p, sc, out_p, S_, Hq, maxblk, descp,
            ws_p, ws_n, wk, st)
    return dev, out, args, keep + (k_new, v_new)


def decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                  v_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                  out: torch.Tensor | None = None, *, num_workers: int = 0,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step in one launch: append each sequence's new token (position ctx-1, its
    block-table slot) and attend; same results as write_kv then decode."""
    dev, out, args, _keep = _append_args(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                                         out, num_workers, workspace)
    with torch.cuda.device(dev):
        st = lib().pa_decode_append(*args)
    _check("pa_decode_append", st)
    return out


def prepare_decode_append(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out=None, *,
                          num_workers=0, workspace=None):
    """Validate once; return a no-argument callable issuing the same pa_decode_append."""
    _dev_, out, args, keep = _append_args(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                                          out, num_workers, workspace, own_workspace=True)
    fn = lib().pa_decode_append

    def call():
        _check("pa_decode_append", fn(*args))
        return keep[5]

    return call


def _attend_args(q, k_cache, v_cache, block_tables, context_lens, query_start, max_query_len, scale, out,
                 num_workers, workspace, own_workspace=False):
    desc = cache_desc(k_cache, v_cache)
    dev = _dev(q, k_cache, v_cache, block_tables, context_lens, query_start)
    if q.dim() != 3 or q.shape[2] != desc.head_dim or q.dtype != k_cache.dtype or not q.is_contiguous():
        raise ValueError("q must be contiguous [rows, Hq, D] in the cache dtype")
    _rows, Hq, D = q.shape
    S = int(context_lens.shape[0]) if context_lens.dim() == 1 else -1
    if context_lens.dtype != torch.int32 or S < 0 or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32 [S]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S \
            or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [S, max_blocks_per_seq]")
    if query_start.dtype != torch.int32 or query_start.shape != (S + 1,) or not query_start.is_contiguous():
        raise ValueError("query_start must be contiguous int32 [S + 1]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != dev:
        raise ValueError("out must be contiguous and shaped like q")
    maxblk = int(block_tables.shape[1])
    need = int(lib().pa_attend_workspace_bytes(S, Hq, maxblk, ctypes.byref(desc), int(num_workers)))
    workspace = _workspace(dev, need, workspace, own_workspace)
    args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(),
            query_start.data_ptr(), ctypes.c_float(scale), out.data_ptr(), S, Hq, maxblk, int(max_query_len),
            int(q.shape[0]), ctypes.byref(desc), workspace.data_ptr(), workspace.numel(), int(num_workers),
            _stream(dev))
    return dev, out, args, (q, k_cache, v_cache, block_tables, context_lens, out, workspace, desc, query_start)


def attend(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
           context_lens: torch.Tensor, query_start: torch.Tensor, max_query_len: int, scale: float,
           out: torch.Tensor | None = None, *, num_workers: int = 0,
           workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Causal attention of several query tokens per sequence: q [rows, Hq, D], sequence s
    owning rows query_start[s] .. query_start[s+1]-1 (its newest positions, already
    written to the caches); returns out [rows, Hq, D].  max_query_len bounds every
    sequence's token count (a host value)."""
    dev, out, args, _keep = _attend_args(q, k_cache, v_cache, block_tables, context_lens, query_start,
                                         max_query_len, scale, out, num_workers, workspace)
    with torch.cuda.device(dev):
        st = lib().pa_attend(*args)
    _check("pa_attend", st)
    return out


def prepare_attend(q, k_cache, v_cache, block_tables, context_lens, query_start, max_query_len, scale, out=None, *,
                   num_workers=0, workspace=None):
    """Validate once; return a no-argument callable issuing the same pa_attend."""
    _dev_, out, args, keep = _attend_args(q, k_cache, v_cache, block_tables, context_lens, query_start,
                                          max_query_len, scale, out, num_workers, workspace, own_workspace=True)
    fn = lib().pa_attend

    def call():
        _check("pa_attend", fn(*args))
        return keep[5]

    return call


def rope(q: torch.Tensor, k: torch.Tensor, positions: torch.Tensor, rope_theta: float) -> None:
    """Rotary embedding in place: q [T, Hq, D] and k [T, Hkv, D] at positions (int32 [T])."""
    dev = _dev(q, k, positions)
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2] \
            or q.dtype != k.dtype or not (q.is_contiguous() and k.is_contiguous()):
        raise ValueError("q and k must be contiguous [T, H, D] of one dtype")
    if positions.dtype != torch.int32 or positions.shape != (q.shape[0],) or not positions.is_contiguous():
        raise ValueError("positions must be contiguous int32 [T]")
    T, Hq, D = q.shape
    with torch.cuda.device(dev):
        st = lib().pa_rope(q.data_ptr(), k.data_ptr(), positions.data_ptr(), T, Hq, k.shape[1], D,
                           _DTYPE_CODE[q.dtype], ctypes.c_float(rope_theta), _stream(dev))
    _check("pa_rope", st)


def _rope_append_args(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, rope_theta, out,
                      num_workers, workspace, own_workspace=False):
    dev, out, args, keep = _append_args(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                                        out, num_workers, workspace, own_workspace)
    # pa_decode_append arguments: (q, kn, vn, k, v, bt, ctx, scale, out, S, Hq, maxblk, desc, ws, ws_n, wk, st)
    args = args[:8] + (ctypes.c_float(rope_theta),) + args[8:]
    return dev, out, args, keep


def decode_rope_append(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, rope_theta,
                       out=None, *, num_workers=0, workspace=None):
    """decode_append with the rotary embedding of q and k_new (at position ctx - 1) in the same launch."""
    dev, out, args, _keep = _rope_append_args(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                                              scale, rope_theta, out, num_workers, workspace)
    with torch.cuda.device(dev):
        st = lib().pa_decode_rope_append(*args)
    _check("pa_decode_rope_append", st)
    return out


def prepare_decode_rope_append(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, rope_theta,
                               out=None, *, num_workers=0, workspace=None):
    """Validate once; return a no-argument callable issuing the same pa_decode_rope_append."""
    _dev_, out, args, keep = _rope_append_args(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                                               scale, rope_theta, out, num_workers, workspace, own_workspace=True)
    fn = lib().pa_decode_rope_append

    def call():
        _check("pa_decode_rope_append", fn(*args))
        return keep[5]

    return call


# --- block pool ---

def _int32_vec(t: torch.Tensor, name: str, n: int | None = None) -> None:
    if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous() or (n is not None and t.shape[0] != n):
        raise ValueError(f"{name} must be contiguous int32 [{'' if n is None else n}]")


def pool_init(free_ids: torch.Tensor, pool_state: torch.Tensor, num_free: int) -> None:
    """Fresh pool: ids 0 .. num_free-1 on the stack free_ids (int32 [capacity]), pool_state int32 [8]."""
    dev = _dev(free_ids, pool_state)
    _int32_vec(free_ids, "free_ids")
    _int32_vec(pool_state, "pool_state", 8)
    with torch.cuda.device(dev):
        st = lib().pa_pool_init(free_ids.data_ptr(), pool_state.data_ptr(), num_free, free_ids.shape[0], _stream(dev))
    _check("pa_pool_init", st)


def _assign_args(context_lens, query_start, block_tables, free_ids, pool_state, slot_mapping, block_size):
    ts = [context_lens, block_tables, free_ids, pool_state, slot_mapping] + ([query_start] if query_start is not None else [])
    dev = _dev(*ts)
    _int32_vec(context_lens, "context_lens")
    S = context_lens.shape[0]
    if query_start is not None:
        _int32_vec(query_start, "query_start", S + 1)
    _int32_vec(free_ids, "free_ids")
    _int32_vec(pool_state, "pool_state", 8)
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S \
            or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [S, max_blocks]")
    if slot_mapping.dtype != torch.int64 or slot_mapping.dim() != 1 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous int64 [T]")
    T = slot_mapping.shape[0]
    args = (context_lens.data_ptr(), None if query_start is None else query_start.data_ptr(), block_tables.data_ptr(),
            free_ids.data_ptr(), pool_state.data_ptr(), slot_mapping.data_ptr(), S, block_tables.shape[1],
            block_size, T, free_ids.shape[0], _stream(dev))
    return dev, args


def assign_slots(context_lens: torch.Tensor, query_start, block_tables: torch.Tensor, free_ids: torch.Tensor,
                 pool_state: torch.Tensor, slot_mapping: torch.Tensor, block_size: int) -> None:
    """Blocks and slots for each sequence's new tokens (pa_assign_slots); query_start None: one token each."""
    dev, args = _assign_args(context_lens, query_start, block_tables, free_ids, pool_state, slot_mapping, block_size)
    with torch.cuda.device(dev):
        st = lib().pa_assign_slots(*args)
    _check("pa_assign_slots", st)


def prepare_assign_slots(context_lens, query_start, block_tables, free_ids, pool_state, slot_mapping, block_size):
    """A no-argument callable that repeats assign_slots with pre-marshalled arguments."""
    dev, args = _assign_args(context_lens, query_start, block_tables, free_ids, pool_state, slot_mapping, block_size)
    fn = lib().pa_assign_slots

    def call():
        st = fn(*args)
        if st:
            _check("pa_assign_slots", st)
    return call


def release_seqs(seq_ids: torch.Tensor, context_lens: torch.Tensor, block_tables: torch.Tensor,
                 free_ids: torch.Tensor, pool_state: torch.Tensor, block_size: int) -> None:
    """Push the listed sequences' blocks back on the stack (pa_release_seqs)."""
    dev = _dev(seq_ids, context_lens, block_tables, free_ids, pool_state)
    _int32_vec(seq_ids, "seq_ids")
    _int32_vec(context_lens, "context_lens")
    _int32_vec(free_ids, "free_ids")
    _int32_vec(pool_state, "pool_state", 8)
    S = context_lens.shape[0]
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S \
            or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32 [S, max_blocks]")
    with torch.cuda.device(dev):
        st = lib().pa_release_seqs(seq_ids.data_ptr(), seq_ids.shape[0], context_lens.data_ptr(),
                                   block_tables.data_ptr(), free_ids.data_ptr(), pool_state.data_ptr(), S,
                                   block_tables.shape[1], block_size, free_ids.shape[0], _stream(dev))
    _check("pa_release_seqs", st)


def acct_init(num_blocks: int, block_size: int, bytes_per_block: int) -> PoolAcct:
    a = PoolAcct()
    _check("pa_acct_init", lib().pa_acct_init(ctypes.byref(a), num_blocks, block_size, bytes_per_block))
    return a


def acct_admit(acct: PoolAcct, max_tokens: int) -> None:
    """Reserve for a request of at most max_tokens tokens; CapacityError if the pool cannot promise it."""
    _check("pa_acct_admit", lib().pa_acct_admit(ctypes.byref(acct), max_tokens))


def acct_retire(acct: PoolAcct, max_tokens: int) -> None:
    _check("pa_acct_retire", lib().pa_acct_retire(ctypes.byref(acct), max_tokens))


def pool_telemetry(acct: PoolAcct, state_host, tokens_stored: int) -> dict:
    """Occupancy and bytes from the accounting and a host copy of pool_state (8 int32)."""
    st = torch.as_tensor(state_host, dtype=torch.int32).contiguous().cpu()
    if st.shape != (8,):
        raise ValueError("state_host must hold the 8 int32 of pool_state")
    out = PoolTelemetry()
    _check("pa_pool_telemetry", lib().pa_pool_telemetry(ctypes.byref(acct), ctypes.c_void_p(st.data_ptr()),
                                                        tokens_stored, ctypes.byref(out)))
    return out.as_dict()


# --- RMSNorm ---

def _norm_args(x, weight, eps, out, residual):
    ts = [x, weight, out] + ([residual] if residual is not None else [])
    dev = _dev(*ts)
    if x.dim() != 2 or weight.shape != (x.shape[1],) or out.shape != x.shape:
        raise ValueError("x and out must be [rows, hidden], weight [hidden]")
    if residual is not None and residual.shape != x.shape:
        raise ValueError("residual must be [rows, hidden]")
    if x.dtype not in _DTYPE_CODE or any(t.dtype != x.dtype for t in ts):
        raise ValueError("tensors must share one of float32/float16/bfloat16")
    if not all(t.is_contiguous() for t in ts):
        raise ValueError("tensors must be contiguous")
    args = (x.data_ptr(), None if residual is None else residual.data_ptr(), weight.data_ptr(), out.data_ptr(),
            x.shape[0], x.shape[1], ctypes.c_float(eps), _DTYPE_CODE[x.dtype], _stream(dev))
    return dev, args


def rmsnorm(x: torch.Tensor, weight: torch.Tensor, eps: float, out: torch.Tensor | None = None,
            residual: torch.Tensor | None = None) -> torch.Tensor:
    """RMSNorm of the rows of x (pa_rmsnorm).  With residual, residual <- round(x + residual)
    in place and that row is normalised.  out may be x."""
    if out is None:
        out = torch.empty_like(x)
    dev, args = _norm_args(x, weight, eps, out, residual)
    with torch.cuda.device(dev):
        st = lib().pa_rmsnorm(*args)
    _check("pa_rmsnorm", st)
    return out


def prepare_rmsnorm(x, weight, eps, out, residual=None):
    """A no-argument callable that repeats rmsnorm with pre-marshalled arguments."""
    dev, args = _norm_args(x, weight, eps, out, residual)
    fn = lib().pa_rmsnorm

    def call():
        st = fn(*args)
        if st:
            _check("pa_rmsnorm", st)
    return call


# --- read-bandwidth probe (measurement aid) ---

def prepare_read_probe(src: torch.Tensor, tile_bytes: int, tile_ids: torch.Tensor | None = None,
                       num_waves: int = 8192):
    """A no-argument callable that reads src's tiles of tile_bytes (in tile_ids order, or
    address order) with pa_read_probe, and the sink tensor it writes: returns (call, sink)."""
    dev = _dev(src) if tile_ids is None else _dev(src, tile_ids)
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    nbytes = src.numel() * src.element_size()
    if tile_ids is None:
        num_tiles = nbytes // tile_bytes
    else:
        if tile_ids.dtype != torch.int32 or tile_ids.dim() != 1 or not tile_ids.is_contiguous():
            raise ValueError("tile_ids must be contiguous int32 [n]")
        num_tiles = tile_ids.shape[0]
    sink = torch.empty(num_waves * 64 * 4, dtype=torch.int32, device=dev)
    args = (src.data_ptr(), None if tile_ids is None else tile_ids.data_ptr(), num_tiles, tile_bytes,
            sink.data_ptr(), num_waves, _stream(dev))
    fn = lib().pa_read_probe

    def call():
        st = fn(*args)
        if st:
            _check("pa_read_probe", st)
    call.num_tiles = num_tiles
    return call, sink
