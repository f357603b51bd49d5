"""Pins of the oracle's block pool (CPU only).

The pool hands out physical blocks from a stack of free ids and turns each
new token's position into its slot.  These tests tie it to facts that do not
come from its own code: closed forms for a fresh pool, a hand-worked refusal
example, the stack's last-in-first-out order, conservation of block ids
through random admit / grow / release churn, and the composition
allocate -> write -> decode against dense attention over the logical rows.
A plausible slip (an off-by-one in the blocks a sequence already holds, pops
from the wrong end, a refusal that is not a prefix, a slot that mixes up the
block and the offset) fails at least one of them.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import dense


def _cdiv(a, b):
    return -(-np.asarray(a, dtype=np.int64) // b)


def _qs(n):
    return np.concatenate([[0], np.cumsum(n)]).astype(np.int32)


@pytest.mark.parametrize("B", [16, 32])
def test_fresh_pool_prefill_closed_form(B):
    # From a fresh pool ids come out 0, 1, 2, ...: sequence s's block j is
    # sum_{r<s} ceil(L_r / B) + j, so its token p has slot base_s * B + p.
    L = np.array([0, 1, B - 1, B, B + 1, 3 * B, 5, 2 * B + 7], dtype=np.int32)
    nb = _cdiv(L, B)
    base = np.concatenate([[0], np.cumsum(nb)[:-1]])
    cap = int(nb.sum()) + 5
    free, st = oracle.pool_init(cap, cap)
    bt = np.full((len(L), 4), -1, dtype=np.int32)
    slots = oracle.assign_slots(L, _qs(L), bt, free, st, B=B)
    want = np.concatenate([base[s] * B + np.arange(L[s]) for s in range(len(L))])
    assert np.array_equal(slots, want)
    for s in range(len(L)):
        assert list(bt[s, :nb[s]]) == list(range(base[s], base[s] + nb[s]))
        assert (bt[s, nb[s]:] == -1).all()
    assert st[0] == cap - nb.sum() and st[2] == st[0] and st[1] == 0 and st[3] == 0


def test_one_sequence_slots_are_its_positions():
    free, st = oracle.pool_init(64, 64)
    bt = np.full((1, 64), -1, dtype=np.int32)
    slots = oracle.assign_slots(np.array([1000]), np.array([0, 1000]), bt, free, st, B=16)
    assert np.array_equal(slots, np.arange(1000))


@pytest.mark.parametrize("L0", [1, 15, 16, 17, 31])
def test_decode_steps_take_a_block_exactly_at_block_starts(L0):
    B, steps = 16, 40
    free, st = oracle.pool_init(20, 20)
    bt = np.full((1, 8), -1, dtype=np.int32)
    oracle.assign_slots(np.array([L0]), np.array([0, L0]), bt, free, st, B=B)
    prev = []
    for k in range(1, steps + 1):
        L = L0 + k
        top = st[0]
        slot = oracle.assign_slots(np.array([L]), None, bt, free, st, B=B)
        p = L - 1
        assert top - st[0] == (1 if p % B == 0 else 0)
        assert slot[0] % B == p % B  # the offset inside the block is the position's
        if p % B and prev:
            assert slot[0] == prev[-1] + 1  # the same block, the next offset
        prev.append(int(slot[0]))
    assert 20 - st[0] == _cdiv(L0 + steps, B)


def test_stack_is_last_in_first_out():
    B = 16
    free, st = oracle.pool_init(12, 12)
    bt = np.full((3, 4), -1, dtype=np.int32)
    L = np.array([40, 20, 0], dtype=np.int32)  # 3 + 2 blocks: ids 0,1,2 and 3,4
    oracle.assign_slots(L, _qs(L), bt, free, st, B=B)
    oracle.release_seqs([0], L, bt, free, st, B=B)  # pushes 0, 1, 2 in block order
    assert (bt[0] == -1).all() and st[0] == 12 - 2
    L2 = np.array([0, 20, 30], dtype=np.int32)  # sequence 2 now takes 2 blocks
    oracle.assign_slots(L2, _qs([0, 0, 30]), bt, free, st, B=B)
    assert list(bt[2, :2]) == [2, 1]  # the last pushed comes off first


def test_refusal_is_a_prefix_of_the_needy_sequences():
    # Worked by hand: 6 free blocks, B = 16.  A first call gives sequence 6 one
    # block (id 0) holding 3 positions, leaving 5.  The second call's needs, in
    # order: s0: 2 (L 20), s1: 0 (no tokens), s2: 4 (L 50), s3: 1 (L 10),
    # s4: 0, s5: 2 (L 17), s6: 0 (its position 3 still fits in block 0).
    # s0 takes ids 1, 2 (3 left); s2 needs 4 > 3 and is refused, and with it
    # s3 and s5 although they would fit; s1, s4 and s6 need nothing and are
    # served.  3 refusals, 3 blocks left.
    B = 16
    free, st = oracle.pool_init(6, 6)
    bt = np.full((7, 4), -1, dtype=np.int32)
    oracle.assign_slots(np.array([0, 0, 0, 0, 0, 0, 3]), _qs([0, 0, 0, 0, 0, 0, 3]), bt, free, st, B=B)
    assert bt[6, 0] == 0 and st[0] == 5
    L = np.array([20, 0, 50, 10, 0, 17, 4], dtype=np.int32)
    n = np.array([20, 0, 50, 10, 0, 17, 1])
    slots = oracle.assign_slots(L, _qs(n), bt, free, st, B=B)
    q = _qs(n)
    assert list(bt[0, :2]) == [1, 2]
    assert np.array_equal(slots[q[0]:q[1]], np.concatenate([16 + np.arange(16), 32 + np.arange(4)]))
    assert (slots[q[2]:q[6]] == -1).all()  # s2, s3, s5 refused
    assert (bt[2] == -1).all() and (bt[3] == -1).all() and (bt[5] == -1).all()
    assert slots[q[6]] == 0 * B + 3  # s6: block 0, offset 3
    assert st[0] == 3 and st[1] == 3 and st[2] == 3


def test_release_that_would_overflow_is_refused_whole():
    B = 16
    free, st = oracle.pool_init(4, 4)
    bt = np.full((2, 2), -1, dtype=np.int32)
    L = np.array([16, 40], dtype=np.int32)
    bt[1] = [9, 9]  # a table the pool never handed out: its release would overflow
    before = (free.copy(), st.copy(), bt.copy())
    oracle.release_seqs([1], L, bt, free, st, B=B)
    assert np.array_equal(free, before[0]) and np.array_equal(bt, before[2])
    assert st[3] == 1 and st[0] == 4


def test_release_skips_ids_outside_the_batch():
    B = 16
    free, st = oracle.pool_init(8, 8)
    bt = np.full((2, 2), -1, dtype=np.int32)
    L = np.array([17, 5], dtype=np.int32)
    oracle.assign_slots(L, _qs(L), bt, free, st, B=B)
    oracle.release_seqs([-1, 7, 1, 2], L, bt, free, st, B=B)
    assert st[0] == 8 - 2 and list(bt[1]) == [-1, -1] and list(bt[0]) == [0, 1]


def _check_conservation(free, st, bt, L, live, cap, B):
    held = []
    for s in live:
        nb = int(_cdiv(L[s], B))
        row = bt[s]
        assert (row[:nb] >= 0).all() and (row[nb:] == -1).all()
        held += list(row[:nb])
    ids = held + list(free[:st[0]])
    assert sorted(ids) == list(range(cap))  # every id exactly once: no leak, no double use


def test_random_churn_conserves_block_ids():
    rng = np.random.default_rng(3)
    B, S, M, cap = 16, 12, 40, 160
    free, st = oracle.pool_init(cap, cap)
    bt = np.full((S, M), -1, dtype=np.int32)
    L = np.zeros(S, dtype=np.int32)
    live = set()
    for it in range(300):
        op = rng.integers(3)
        if op == 0 and len(live) < S:  # admit a prompt, in one or two chunks
            s = min(set(range(S)) - live)
            total = int(rng.integers(1, 200))
            parts = [total] if rng.integers(2) else [total // 2, total - total // 2]
            live.add(s)
            for part in parts:
                n = np.zeros(S, dtype=np.int32)
                n[s] = part
                newL = L.copy()
                newL[s] += part
                slots = oracle.assign_slots(newL, _qs(n), bt, free, st, B=B)
                if st[1]:
                    break
                L = newL
                p = np.arange(L[s] - part, L[s])
                assert np.array_equal(slots // B, bt[s, p // B]) and np.array_equal(slots % B, p % B)
        elif op == 1 and live:  # every live sequence grows by 1..3 tokens
            n = np.zeros(S, dtype=np.int32)
            for s in live:
                n[s] = rng.integers(1, 4)
            newL = (L + n).astype(np.int32)
            if (newL > M * B).any():
                continue
            slots = oracle.assign_slots(newL, _qs(n), bt, free, st, B=B)
            if st[1]:
                break
            L = newL
            assert len(set(slots.tolist())) == len(slots)  # distinct slots
        elif op == 2 and live:
            s = int(rng.choice(sorted(live)))
            oracle.release_seqs([s], L, bt, free, st, B=B)
            live.discard(s)
            L[s] = 0
        if st[1]:
            break  # the pool ran dry: stop before a refused sequence leaves L out of step
        _check_conservation(free, st, bt, L, live, cap, B)
    assert it > 100


def test_allocate_write_decode_matches_dense_attention():
    # Prompts admitted in two chunks and three decode steps on a pool whose
    # free ids were shuffled by earlier churn; every K/V row is written to the
    # slot the pool gave it, then the paged decode must equal dense attention
    # over the rows in logical order.
    rng = np.random.default_rng(9)
    B, D, Hkv, Hq, M = 16, 64, 2, 4, 8
    cap = 30
    free, st = oracle.pool_init(cap, cap)
    junk = np.full((2, M), -1, dtype=np.int32)
    Lj = np.array([70, 45], dtype=np.int32)
    oracle.assign_slots(Lj, _qs(Lj), junk, free, st, B=B)
    oracle.release_seqs([0], Lj, junk, free, st, B=B)
    S = 3
    final = np.array([37, 16, 50], dtype=np.int32)
    k_log = torch.from_numpy(rng.standard_normal((S, 64, Hkv, D)).astype(np.float32))
    v_log = torch.from_numpy(rng.standard_normal((S, 64, Hkv, D)).astype(np.float32))
    kp = torch.zeros(cap * Hkv * B * D, dtype=torch.float32)
    vp = torch.zeros_like(kp)
    bt = np.full((S, M), -1, dtype=np.int32)
    L = np.zeros(S, dtype=np.int32)
    for target in (np.array([20, 10, 33]), final - 3, final - 2, final - 1, final):
        n = (target - L).astype(np.int32)
        slots = oracle.assign_slots(target.astype(np.int32), _qs(n), bt, free, st, B=B)
        rows = [(s, p) for s in range(S) for p in range(L[s], target[s])]
        kn = torch.stack([k_log[s, p] for s, p in rows]) if rows else torch.zeros((0, Hkv, D))
        vn = torch.stack([v_log[s, p] for s, p in rows]) if rows else torch.zeros((0, Hkv, D))
        oracle.write_kv(kn.contiguous(), vn.contiguous(), slots, kp, vp, num_blocks=cap, B=B)
        L = target.astype(np.int32)
    assert st[1] == 0
    q = torch.from_numpy(rng.standard_normal((S, Hq, D)).astype(np.float32))
    scale = float(np.float32(D ** -0.5))
    got = oracle.decode(q, kp, vp, bt, L, scale, Hkv=Hkv, B=B)
    G = Hq // Hkv
    for s in range(S):
        for h in range(Hq):
            ref = dense.attention(q[s, h].double().numpy(), k_log[s, :L[s], h // G].double().numpy(),
                                  v_log[s, :L[s], h // G].double().numpy(), scale)
            assert np.max(np.abs(got[s, h] - ref)) <= 1e-12
