"""The full-size f32 parity bound can see lost work (CPU only).

The GPU tests hold the f32 twins of the three large workloads to a max-abs
error of 1e-5.  This checks, in float64 on the host, that a kernel which lost
the work of any single 16-token block of any sequence (or of a whole split
part) would miss that bound: removing one block's tokens from the softmax
moves some output element by more than 1e-5, for every block of the
Llama-3-8B-shaped batch and of a sequence of the long-context workload.

Dropping block j of a sequence changes out = N / W (N = sum_t w_t v_t,
W = sum_t w_t, w_t = exp(z_t - max z)) into (N - N_j) / (W - W_j), so every
block's effect comes from per-block sums of one dense pass; the dense pass is
the plain definition (it agrees with the oracle, checked below).
"""
import numpy as np
import pytest

import oracle
from paged_kv_decode_slot_amd import workloads as W

F32_BOUND = 1e-5


def _block_sums(q, k, v, scale, G, B):
    """Per kv-head group: the full sums (W [G], N [G, D]) and the per-block sums
    (W_j [G, nblk], N_j [G, nblk, D]).  q [Hq, D], k and v [L, Hkv, D] (float64),
    L a multiple of B."""
    L, Hkv, D = k.shape
    nblk = L // B
    groups = []
    for g in range(Hkv):
        z = scale * (q[g * G:(g + 1) * G] @ k[:, g, :].T)  # [G, L]
        w = np.exp(z - z.max(axis=1, keepdims=True))
        wb = w.reshape(G, nblk, B)
        Wj = wb.sum(axis=2)
        Nj = np.einsum("hjt,jtd->hjd", wb, v[:, g, :].reshape(nblk, B, D))
        groups.append((Wj.sum(axis=1), Nj.sum(axis=1), Wj, Nj))
    return groups


def _shift(groups, drop):
    """max over (head, dim) of |out without the blocks in `drop` - out|, for each
    row of `drop` (a [n, nblk] 0/1 matrix)."""
    worst = np.zeros(drop.shape[0])
    for Wt, Nt, Wj, Nj in groups:
        out = Nt / Wt[:, None]
        Wd = Wj @ drop.T                                  # [G, n]
        Nd = np.einsum("hjd,nj->hnd", Nj, drop)           # [G, n, D]
        dropped = (Nt[:, None, :] - Nd) / (Wt[:, None] - Wd)[:, :, None]
        worst = np.maximum(worst, np.abs(dropped - out[:, None, :]).max(axis=(0, 2)))
    return worst


def _output(groups):
    return np.concatenate([Nt / Wt[:, None] for Wt, Nt, _, _ in groups])


def _per_block(groups):
    """The effect of dropping each single block, without forming a [nblk, nblk] matrix."""
    worst = None
    for Wt, Nt, Wj, Nj in groups:
        out = Nt / Wt[:, None]
        dropped = (Nt[:, None, :] - Nj) / (Wt[:, None] - Wj)[:, :, None]
        w = np.abs(dropped - out[:, None, :]).max(axis=(0, 2))
        worst = w if worst is None else np.maximum(worst, w)
    return worst


def _seq(case, s):
    k, v = case.logical_kv(s)
    L = k.shape[0] // case.B * case.B  # whole blocks only (the last, partial one is left out)
    q = case.q[s].double().numpy()
    return q, k[:L].double().numpy(), v[:L].double().numpy()


def test_llama3_batch_every_block_is_visible():
    case = W.twin_case(3, "f32")
    lows = []
    for s in range(case.S):
        q, k, v = _seq(case, s)
        lows.append(float(_per_block(_block_sums(q, k, v, case.scale, case.G, case.B)).min()))
    print(f"C3 f32 twin: smallest effect of dropping one block, over all {case.S} sequences: {min(lows):.3e}")
    assert min(lows) > 3 * F32_BOUND


def test_long_context_every_block_and_part_is_visible():
    # one sequence of the long-context workload's shape (131072 tokens, 28q/4kv, d128, B16)
    case = W.make_case(S=1, Hq=28, Hkv=4, D=128, B=16, dtype="f32", ctx=[131072], seed=5, name="C5 shape")
    q, k, v = _seq(case, 0)
    groups = _block_sums(q, k, v, case.scale, case.G, case.B)
    worst = _per_block(groups)
    print(f"C5 shape: smallest effect of dropping one block of 8192: {worst.min():.3e}")
    assert worst.min() > 3 * F32_BOUND
    # whole parts of a split of the sequence into 16 runs of 512 blocks
    drop = np.zeros((16, 8192))
    for i in range(16):
        drop[i, 512 * i:512 * (i + 1)] = 1.0
    parts = _shift(groups, drop)
    print(f"C5 shape: smallest effect of dropping a 512-block part: {parts.min():.3e}")
    assert parts.min() > 30 * F32_BOUND


def test_dense_pass_is_the_oracle():
    case = W.make_case(S=2, Hq=8, Hkv=2, D=128, B=16, dtype="f32", ctx=[512, 48], seed=9, name="tie")
    ref = oracle.decode_case(case)
    for s in range(case.S):
        q, k, v = _seq(case, s)
        out = _output(_block_sums(q, k, v, case.scale, case.G, case.B))
        np.testing.assert_allclose(out, ref[s], rtol=0, atol=1e-12)
        # and the per-block formula is a real removal of those tokens
        groups = _block_sums(q, k, v, case.scale, case.G, case.B)
        keep = np.ones(k.shape[0] // 16, dtype=bool)
        keep[1] = False
        kk = k.reshape(-1, 16, 2, 128)[keep].reshape(-1, 2, 128)
        vv = v.reshape(-1, 16, 2, 128)[keep].reshape(-1, 2, 128)
        direct = _output(_block_sums(q, kk, vv, case.scale, case.G, case.B))
        assert abs(float(np.abs(direct - out).max()) - float(_per_block(groups)[1])) < 1e-12
