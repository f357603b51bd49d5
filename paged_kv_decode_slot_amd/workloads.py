"""Seeded synthetic inputs for paged-KV decode attention.

This module only draws numbers and places them: context lengths, the
physical placement of each sequence's blocks (the block tables), the query
rows and the K/V rows of every token, and the slot each token is written to.
It holds none of the attention arithmetic, and it is the one module that the
HIP path's tests and the CPU oracle both take their inputs from.

The workloads imitate the batches described on the pages:

* the ForgeLLM README (LLM-inference-server), feature list: physical KV blocks
  reached through per-request logical block tables, grouped-query attention,
  one decode token per running sequence;
* the LLM-Inference-Engine README, request-journey figure and the "why paged
  KV cache" paragraph: fixed-size blocks from a preallocated pool, handed to a
  request as it grows and returned when it finishes.

Draw order, per case, from ``numpy.random.default_rng(seed)``: context
lengths, then placement, then Q, then the K rows of the prefill tokens, then
their V rows, then the new token's K and V rows.  Values are float32 standard
normals rounded to nearest-even into the storage dtype (torch's CPU cast), and
both sides read those rounded values.

``context_lens[s]`` counts the token being decoded: positions
``0 .. ctx-2`` are the prefill (already cached) and position ``ctx-1`` is the
new token whose K/V the decode step appends before attending.

A slot is ``physical_block * block_size + offset_in_block``; a negative slot
marks a padding token that is not written.  Pools start filled with a quiet
NaN, and one extra block (the poison block) is never written: block-table
entries past a sequence's last block point at it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ELT_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
# Quiet-NaN bit patterns used to poison never-written cache bytes.
NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}


@dataclass
class Case:
    """One decode step's inputs, in storage dtype, on the host."""

    name: str
    S: int
    Hq: int
    Hkv: int
    D: int
    B: int
    dtype: str
    num_blocks: int  # pool size, poison block included
    poison_block: int
    context_lens: np.ndarray  # int32 [S]
    block_tables: np.ndarray  # int32 [S, max_blocks_per_seq]
    q: torch.Tensor  # [S, Hq, D]
    k_prefill: torch.Tensor  # [T0, Hkv, D]  positions 0..ctx-2 of every sequence
    v_prefill: torch.Tensor
    slot_prefill: np.ndarray  # int64 [T0]
    k_new: torch.Tensor  # [S, Hkv, D]  position ctx-1 of every sequence
    v_new: torch.Tensor
    slot_new: np.ndarray  # int64 [S]; -1 where ctx == 0
    scale: float  # a float32 value
    meta: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elt(self) -> int:
        return ELT_BYTES[self.dtype]

    @property
    def pool_numel(self) -> int:
        """Elements in one cache (K or V) pool."""
        return self.num_blocks * self.Hkv * self.B * self.D

    def nan_pool(self) -> torch.Tensor:
        """A flat host pool of ``pool_numel`` elements holding the poison NaN."""
        bits = NAN_BITS[self.dtype]
        if self.elt == 4:
            raw = torch.full((self.pool_numel,), bits, dtype=torch.int32)
        else:
            raw = torch.full((self.pool_numel,), bits, dtype=torch.int16)
        return raw.view(DTYPES[self.dtype])

    def logical_kv(self, s: int) -> tuple[torch.Tensor, torch.Tensor]:
        """K and V rows of sequence ``s`` in logical position order, [ctx, Hkv, D].

        Assembled from the drawn arrays (prefill rows, then the new row); no
        cache or block table is involved.
        """
        L = int(self.context_lens[s])
        if L == 0:
            empty = torch.empty((0, self.Hkv, self.D), dtype=DTYPES[self.dtype])
            return empty, empty
        pre = np.concatenate([[0], np.cumsum(np.maximum(self.context_lens.astype(np.int64) - 1, 0))])
        a, b = int(pre[s]), int(pre[s + 1])
        k = torch.cat([self.k_prefill[a:b], self.k_new[s:s + 1]], dim=0)
        v = torch.cat([self.v_prefill[a:b], self.v_new[s:s + 1]], dim=0)
        return k, v

    def all_tokens(self):
        """Prefill and new tokens as one write batch: (k, v, slots)."""
        k = torch.cat([self.k_prefill, self.k_new], dim=0)
        v = torch.cat([self.v_prefill, self.v_new], dim=0)
        slots = np.concatenate([self.slot_prefill, self.slot_new]).astype(np.int64)
        return k, v, slots


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(x).to(DTYPES[dtype])


def _normal(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    return _cast(rng.standard_normal(size=shape, dtype=np.float32), dtype)


def _blocks_needed(ctx: np.ndarray, B: int) -> np.ndarray:
    return (ctx.astype(np.int64) + B - 1) // B


def _shuffled_placement(rng, ctx, B, pool):
    """First ``need`` entries of a seeded permutation of the pool, sequence by sequence."""
    nb = _blocks_needed(ctx, B)
    perm = rng.permutation(pool)
    tables, at = [], 0
    for n in nb:
        tables.append(perm[at:at + n])
        at += n
    return tables


def _lognormal_ctx(rng, n, median=1024.0, sigma=1.0, lo=1, hi=32768):
    return np.clip(np.rint(np.exp(rng.normal(math.log(median), sigma, size=n))), lo, hi).astype(np.int64)


def _churned_placement(rng, ctx, B, pool):
    """Placement after seeded alloc/free churn of a block pool.

    A free stack starts as a seeded permutation.  4*S rounds either admit a
    dummy request (lognormal length) or retire a live one, returning its
    blocks; then all dummies retire.  The real sequences then take half their
    blocks as a prompt, in admission order, and grow one block per turn in
    round-robin until each holds all of its blocks, as sequences do when they
    decode side by side.
    """
    S = len(ctx)
    free = list(rng.permutation(pool))
    live = []
    for _ in range(4 * S):
        if not live or rng.random() < 0.5:
            dctx = int(_lognormal_ctx(rng, 1)[0])
            need = -(-dctx // B)
            if need <= len(free):
                live.append([free.pop() for _ in range(need)])
        else:
            blocks = live.pop(int(rng.integers(len(live))))
            free.extend(reversed(blocks))
    for i in rng.permutation(len(live)):
        free.extend(reversed(live[i]))
    nb = _blocks_needed(ctx, B)
    tables = [[] for _ in range(S)]
    for s in range(S):
        for _ in range(-(-int(ctx[s]) // (2 * B))):
            tables[s].append(free.pop())
    while any(len(tables[s]) < nb[s] for s in range(S)):
        for s in range(S):
            if len(tables[s]) < nb[s]:
                tables[s].append(free.pop())
    return [np.asarray(t, dtype=np.int64) for t in tables]


def make_case(*, S, Hq, Hkv, D, B, dtype, ctx=None, ctx_range=None, seed=0,
              pool=None, pool_factor=1.25, placement="shuffle", scale=None,
              name="custom", max_blocks_per_seq=None) -> Case:
    """Draw one decode step.

    ``ctx`` gives the context lengths directly; otherwise they are drawn as
    integers uniform on the inclusive ``ctx_range``, or lognormal
    (median 1024, sigma 1, clipped to [1, 32768]) when ``ctx_range`` is the
    string ``"lognormal"``.  The pool holds ``pool`` blocks, or
    ``ceil(pool_factor * need)``, plus the poison block.
    """
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    rng = np.random.default_rng(seed)
    if ctx is not None:
        ctx = np.asarray(ctx, dtype=np.int64)
        assert ctx.shape == (S,)
    elif ctx_range == "lognormal":
        ctx = _lognormal_ctx(rng, S)
    else:
        lo, hi = ctx_range
        ctx = rng.integers(lo, hi + 1, size=S).astype(np.int64)
    nb = _blocks_needed(ctx, B)
    need = int(nb.sum())
    if pool is None:
        pool = max(1, math.ceil(pool_factor * need))
    if pool < need:
        raise ValueError("pool smaller than the blocks needed")
    if placement == "shuffle":
        tables = _shuffled_placement(rng, ctx, B, pool)
    elif placement == "churn":
        tables = _churned_placement(rng, ctx, B, pool)
    elif placement == "identity":
        tables, at = [], 0
        for n in nb:
            tables.append(np.arange(at, at + n))
            at += n
    else:
        raise ValueError(placement)
    poison = pool  # the extra block, never written
    num_blocks = pool + 1
    maxblk = max_blocks_per_seq if max_blocks_per_seq is not None else max(1, int(nb.max()) if S else 1)
    assert maxblk >= (int(nb.max()) if S else 0)
    bt = np.full((S, maxblk), poison, dtype=np.int32)
    for s in range(S):
        bt[s, :nb[s]] = tables[s]

    q = _normal(rng, (S, Hq, D), dtype)
    T0 = int(np.maximum(ctx - 1, 0).sum())
    k_pre = _normal(rng, (T0, Hkv, D), dtype)
    v_pre = _normal(rng, (T0, Hkv, D), dtype)
    k_new = _normal(rng, (S, Hkv, D), dtype)
    v_new = _normal(rng, (S, Hkv, D), dtype)

    slot_pre = np.empty(T0, dtype=np.int64)
    slot_new = np.full(S, -1, dtype=np.int64)
    at = 0
    for s in range(S):
        L = int(ctx[s])
        if L == 0:
            continue
        pos = np.arange(L, dtype=np.int64)
        slots = bt[s, pos // B].astype(np.int64) * B + pos % B
        slot_pre[at:at + L - 1] = slots[:-1]
        slot_new[s] = slots[-1]
        at += L - 1

    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    return Case(name=name, S=S, Hq=Hq, Hkv=Hkv, D=D, B=B, dtype=dtype,
                num_blocks=num_blocks, poison_block=poison,
                context_lens=ctx.astype(np.int32), block_tables=bt, q=q,
                k_prefill=k_pre, v_prefill=v_pre, slot_prefill=slot_pre,
                k_new=k_new, v_new=v_new, slot_new=slot_new,
                scale=float(np.float32(scale)), meta={"seed": seed, "pool": pool, "placement": placement})


@dataclass
class MultiCase:
    """Several query tokens per sequence over the pools of ``base``: sequence s
    owns query rows ``query_start[s] .. query_start[s+1]-1``, its newest
    positions (their K/V are among the base case's written rows)."""

    base: Case
    q: torch.Tensor  # [rows, Hq, D]
    query_start: np.ndarray  # int32 [S + 1]

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.query_start)

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.base.S else 0


def with_queries(case: Case, q_lens, seed: int = 0) -> MultiCase:
    """Query rows for ``case``'s sequences: ``q_lens[s]`` of them (clipped to the
    context length), drawn as float32 standard normals rounded into the dtype
    from their own generator (seeded with ``seed``)."""
    n = np.minimum(np.asarray(q_lens, dtype=np.int64), case.context_lens.astype(np.int64))
    n = np.maximum(n, 0)
    assert n.shape == (case.S,)
    rng = np.random.default_rng(seed)
    q = _normal(rng, (int(n.sum()), case.Hq, case.D), case.dtype)
    qs = np.zeros(case.S + 1, dtype=np.int32)
    qs[1:] = np.cumsum(n)
    return MultiCase(base=case, q=q, query_start=qs)


def attend_bytes(mc: MultiCase) -> int:
    """Bytes a multi-query attention call must move: every used K and V row once,
    q read and out written, used block-table entries, lengths and query starts."""
    case = mc.base
    ctx = case.context_lens.astype(np.int64)
    used = mc.q_lens > 0
    kv = int(ctx[used].sum()) * case.Hkv * case.D * case.elt * 2
    rows = int(mc.query_start[-1])
    qo = 2 * rows * case.Hq * case.D * case.elt
    bt = 4 * int(((ctx[used] + case.B - 1) // case.B).sum())
    return kv + qo + bt + 4 * case.S + 4 * (case.S + 1)


# The five workloads.  C1 is the small case the oracle finishes at once;
# C3 and C4 are the Llama-3-8B-shaped ragged batches.
CONFIGS = {
    1: dict(name="C1 tiny fp32: 4 seqs, 4q/2kv, d64, B16, ctx U[1,64], pool 64",
            S=4, Hq=4, Hkv=2, D=64, B=16, dtype="f32", ctx_range=(1, 64), pool=64),
    2: dict(name="C2 TinyLlama-1.1B-shaped fp16: 8 seqs, 32q/4kv, d64, B16, ctx U[128,2048]",
            S=8, Hq=32, Hkv=4, D=64, B=16, dtype="f16", ctx_range=(128, 2048)),
    3: dict(name="C3 Llama-3-8B-shaped bf16: 64 seqs, 32q/8kv, d128, B16, ctx U[512,4096]",
            S=64, Hq=32, Hkv=8, D=128, B=16, dtype="bf16", ctx_range=(512, 4096)),
    4: dict(name="C4 ragged mix bf16: 256 seqs, 32q/8kv, d128, B32, lognormal ctx, churned pool",
            S=256, Hq=32, Hkv=8, D=128, B=32, dtype="bf16", ctx_range="lognormal", placement="churn"),
    5: dict(name="C5 long-context bf16: 8 seqs x 131072, 28q/4kv, d128, B16",
            S=8, Hq=28, Hkv=4, D=128, B=16, dtype="bf16", ctx=[131072] * 8),
}


def config_case(n: int) -> Case:
    """The seeded draw of workload ``n`` (seed = n)."""
    cfg = dict(CONFIGS[n])
    return make_case(seed=n, **cfg)


def twin_case(n: int, dtype: str = "f32") -> Case:
    """Workload ``n`` drawn again with another storage dtype: the same seed, so the
    same lengths, block tables and placement, and the same float32 draws, here
    rounded into ``dtype`` (not rounded at all for f32)."""
    cfg = dict(CONFIGS[n])
    cfg["name"] = f"{cfg['name']} ({dtype} twin)"
    cfg["dtype"] = dtype
    return make_case(seed=n, **cfg)


def decode_bytes(case: Case) -> int:
    """Bytes a decode step must move: every used K and V row, q, out, the used
    block-table entries and the context lengths."""
    ctx = case.context_lens.astype(np.int64)
    kv = int(ctx.sum()) * case.Hkv * case.D * case.elt * 2
    qo = 2 * case.S * case.Hq * case.D * case.elt
    bt = 4 * int(((ctx + case.B - 1) // case.B).sum())
    return kv + qo + bt + 4 * case.S


def kv_read_bytes(case: Case) -> int:
    """K and V bytes a fused step reads from the pools: every cached position's rows
    except the new token's, which come from k_new / v_new."""
    ctx = case.context_lens.astype(np.int64)
    return int(np.maximum(ctx - 1, 0).sum()) * case.Hkv * case.D * case.elt * 2


def step_bytes(case: Case) -> int:
    """Bytes one fused step (append, then decode) must move: the K and V rows of
    the L - 1 cached positions of every sequence, its new token's rows read once
    and stored once, q, out, the used block-table entries and the lengths."""
    ctx = case.context_lens.astype(np.int64)
    row = case.Hkv * case.D * case.elt * 2  # one position's K and V rows, all kv-heads
    new = int((ctx > 0).sum())
    return decode_bytes(case) - new * row + 2 * new * row


def write_bytes(case: Case) -> int:
    """Bytes the KV-append of one new token per sequence must move (read + write of K and V, plus slots)."""
    T = case.S
    return 2 * T * case.Hkv * case.D * case.elt * 2 + 8 * T
