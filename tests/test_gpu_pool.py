"""Block pool on the GPU against the oracle, bit for bit (through the C ABI).

Each step runs pa_assign_slots / pa_release_seqs on the device and the
oracle's assign_slots / release_seqs on host copies of the same inputs; the
slots, block tables, the live part of the free-id stack and the counters
must match exactly after every call.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_slot_amd as pa
from paged_kv_decode_slot_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _qs(n):
    return np.concatenate([[0], np.cumsum(n)]).astype(np.int32)


class Pair:
    """The device pool and the oracle's, driven in lockstep."""

    def __init__(self, S, M, B, capacity, num_free):
        self.S, self.M, self.B, self.cap = S, M, B, capacity
        self.free_h, self.state_h = oracle.pool_init(capacity, num_free)
        self.bt_h = np.full((S, M), -1, dtype=np.int32)
        self.free_d = torch.full((capacity,), -5, dtype=torch.int32, device=DEV)
        self.state_d = torch.full((8,), 77, dtype=torch.int32, device=DEV)
        self.bt_d = torch.from_numpy(self.bt_h.copy()).to(DEV)
        pa.pool_init(self.free_d, self.state_d, num_free)
        self.L = np.zeros(S, dtype=np.int32)
        self.compare("init")

    def assign(self, newL, n, per_token=False):
        newL = np.asarray(newL, dtype=np.int32)
        qs = None if per_token else _qs(n)
        want = oracle.assign_slots(newL, qs, self.bt_h, self.free_h, self.state_h, B=self.B)
        T = self.S if per_token else int(qs[-1])
        slots_d = torch.full((T,), -9, dtype=torch.int64, device=DEV)
        pa.assign_slots(torch.from_numpy(newL).to(DEV), None if per_token else torch.from_numpy(qs).to(DEV),
                        self.bt_d, self.free_d, self.state_d, slots_d, self.B)
        got = slots_d.cpu().numpy()
        assert np.array_equal(got, want), f"slots differ at {np.nonzero(got != want)[0][:10]}"
        self.compare("assign")
        return want

    def release(self, ids):
        ids = np.asarray(ids, dtype=np.int32)
        oracle.release_seqs(ids, self.L, self.bt_h, self.free_h, self.state_h, B=self.B)
        pa.release_seqs(torch.from_numpy(ids).to(DEV), torch.from_numpy(self.L).to(DEV), self.bt_d, self.free_d,
                        self.state_d, self.B)
        self.compare("release")

    def compare(self, what):
        st = self.state_d.cpu().numpy()
        assert np.array_equal(st[:4], self.state_h[:4]), (what, st, self.state_h)
        assert np.array_equal(st[4:], np.zeros(4, dtype=np.int32)), (what, st)  # arrival word back to zero
        top = int(st[0])
        assert np.array_equal(self.free_d[:top].cpu().numpy(), self.free_h[:top]), what
        assert np.array_equal(self.bt_d.cpu().numpy(), self.bt_h), what


def test_fresh_prefill_gives_positions_as_slots():
    print("[pool] fresh prefill", flush=True)
    p = Pair(S=3, M=70, B=16, capacity=200, num_free=200)
    L = np.array([1000, 0, 37], dtype=np.int32)
    slots = p.assign(L, L)
    assert np.array_equal(slots[:1000], np.arange(1000))


@pytest.mark.parametrize("S,B,seed", [(5, 16, 1), (300, 16, 2), (300, 32, 3), (700, 16, 4)])
def test_random_churn_matches_oracle(S, B, seed):
    """Admissions in chunks (some large enough to split a group's rows over
    several workgroups), decode steps of one token each (the per-token form)
    and of several, and releases, over more than one group of 256 sequences."""
    print(f"[pool] churn S={S} B={B} seed={seed}", flush=True)
    rng = np.random.default_rng(seed)
    M = 160
    cap = S * 40
    p = Pair(S=S, M=M, B=B, capacity=cap, num_free=cap - 3)
    live = np.zeros(S, dtype=bool)
    for it in range(14):
        op = it % 4
        if op == 0:  # admit up to a third of the idle sequences, prompts of 1..3000 tokens
            idle = np.nonzero(~live)[0]
            take = rng.choice(idle, size=min(len(idle), max(1, S // 3)), replace=False) if len(idle) else []
            n = np.zeros(S, dtype=np.int32)
            for s in take:
                n[s] = rng.integers(1, 3000) if rng.random() < 0.3 else rng.integers(1, 300)
            newL = np.minimum(p.L + n, M * B).astype(np.int32)
            n = newL - p.L
            p.assign(newL, n)
            if p.state_h[1]:
                break
            live |= n > 0
            p.L = newL
        elif op == 1:  # a decode step: one token for every live sequence (per-token form when all are live)
            n = live.astype(np.int32)
            newL = np.minimum(p.L + n, M * B).astype(np.int32)
            n = newL - p.L
            per_token = bool(live.all()) and bool((n == 1).all())
            p.assign(newL, n, per_token=per_token)
            if p.state_h[1]:
                break
            p.L = newL
        elif op == 2:  # several tokens (drafts or a chunk) for a random subset
            n = np.where(live & (rng.random(S) < 0.5), rng.integers(1, 40, S), 0).astype(np.int32)
            newL = np.minimum(p.L + n, M * B).astype(np.int32)
            n = newL - p.L
            p.assign(newL, n)
            if p.state_h[1]:
                break
            p.L = newL
        else:  # retire a random subset of the live sequences (ids given in a shuffled order)
            ids = np.nonzero(live & (rng.random(S) < 0.4))[0]
            rng.shuffle(ids)
            p.release(ids)
            live[ids] = False
            p.L[ids] = 0


@pytest.mark.parametrize("cfg", [3, 4])
def test_full_size_admission_and_decode_steps(cfg):
    """The workload's whole batch admitted at once (its context lengths as the
    prompts), then 3 decode steps, on a pool of the workload's size."""
    print(f"[pool] full size C{cfg}", flush=True)
    c = W.config_case(cfg)
    M = c.block_tables.shape[1] + 2
    p = Pair(S=c.S, M=M, B=c.B, capacity=c.num_blocks, num_free=c.num_blocks)
    L = c.context_lens.astype(np.int32)
    p.assign(L, L)
    p.L = L
    for _ in range(3):
        newL = (p.L + 1).astype(np.int32)
        p.assign(newL, np.ones(c.S, dtype=np.int32), per_token=True)
        p.L = newL
    assert p.state_h[1] == 0


def test_many_sequences_one_step():
    print("[pool] 5000 sequences", flush=True)
    rng = np.random.default_rng(7)
    S, B, M = 5000, 16, 8
    p = Pair(S=S, M=M, B=B, capacity=S * M, num_free=S * M)
    L = rng.integers(0, 100, S).astype(np.int32)
    p.assign(L, L)
    p.L = L
    newL = np.where(L > 0, L + 1, 0).astype(np.int32)
    p.assign(newL, (newL - L).astype(np.int32))


def test_refusal_and_overflow_match_oracle():
    print("[pool] refusal", flush=True)
    p = Pair(S=7, M=4, B=16, capacity=6, num_free=6)
    p.assign([0, 0, 0, 0, 0, 0, 3], [0, 0, 0, 0, 0, 0, 3])
    p.L = np.array([0, 0, 0, 0, 0, 0, 3], dtype=np.int32)
    p.assign([20, 0, 50, 10, 0, 17, 4], [20, 0, 50, 10, 0, 17, 1])
    assert p.state_h[1] == 3
    # a release that would overflow the 6-id stack is refused whole
    p.L = np.array([20, 0, 0, 0, 0, 0, 4], dtype=np.int32)
    p.bt_h[1, :] = [5, 5, 5, 5]
    p.bt_d[1, :] = 5
    p.L[1] = 64
    p.release([1, 0])
    assert p.state_h[3] == 1


def test_pool_slots_drive_the_fused_decode_step():
    """A decode step whose new blocks come from the pool: pa_assign_slots, then
    pa_decode_append on the updated tables, against the oracle."""
    print("[pool] pool + decode_append", flush=True)
    c = W.config_case(1)
    S, B = c.S, c.B
    M = c.block_tables.shape[1] + 2
    cap = c.num_blocks + 8
    p = Pair(S=S, M=M, B=B, capacity=cap, num_free=cap)
    prompt = (c.context_lens - 1).astype(np.int32)
    p.assign(prompt, prompt)
    p.L = prompt
    kc, vc = pa.new_cache(cap, B, c.Hkv, c.D, W.DTYPES[c.dtype], DEV)
    kc.zero_()
    vc.zero_()
    # the prompt rows (the workload's prefill rows: sequence by sequence, positions < ctx - 1)
    # go to the slots the pool gave them
    slots_prompt = torch.from_numpy(np.concatenate(
        [p.bt_h[s, np.arange(prompt[s]) // B].astype(np.int64) * B + np.arange(prompt[s]) % B
                     for s in range(S)])).to(DEV)
    pa.write_kv(c.k_prefill.to(DEV), c.v_prefill.to(DEV), slots_prompt, kc, vc)
    newL = c.context_lens.astype(np.int32)
    p.assign(newL, np.ones(S, dtype=np.int32), per_token=True)
    p.L = newL
    out = pa.decode_append(c.q.to(DEV), c.k_new.to(DEV), c.v_new.to(DEV), kc, vc, p.bt_d,
                           torch.from_numpy(newL).to(DEV), c.scale)
    kh, vh = kc.cpu().reshape(-1), vc.cpu().reshape(-1)
    want = oracle.decode(c.q, kh, vh, p.bt_h, newL, c.scale, Hkv=c.Hkv, B=B)
    err = np.max(np.abs(out.float().cpu().double().numpy() - want))
    assert err <= 1e-5, err
