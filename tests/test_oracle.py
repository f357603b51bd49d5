"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties one part of the oracle to an independent fact: NumPy dense
attention over the logical rows (no pool, no block table), arbitrary-precision
brute force, closed forms, invariances the definition implies, and other
libraries' float16/bfloat16 conversions.  A plausible slip in the oracle (a
dropped scale, a wrong kv-head for a query head, a transposed pool index, a
missing max shift, a wrong slot split) fails at least one of them.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle
from oracle import dense
from paged_kv_decode_slot_amd import workloads as W


def _case(**kw):
    base = dict(S=3, Hq=4, Hkv=2, D=64, B=16, dtype="f32", ctx_range=(1, 70), seed=11)
    base.update(kw)
    return W.make_case(**base)


# --- P1: the write, against the documented pool shapes (torch views, not the oracle's index code) ---
# Pools hold each block as 16-token slabs of 16*D elements.  Per slab, with
# X = 16/elt and Y = 4/elt: K is [D/X][16][X]; V is [D/(16Y)][16][4][Y][4],
# indexed by (d // 16Y, d % 16, t // 4, (d // 16) % Y, t % 4).

def k_row(c, k_pool, p, o):
    X = 16 // c.elt
    kv = k_pool.view(c.num_blocks, c.Hkv, c.B // 16, c.D // X, 16, X)
    return kv[p, :, o // 16, :, o % 16, :].reshape(c.Hkv, c.D)


def v_row(c, v_pool, p, o):
    Y = 4 // c.elt
    vv = v_pool.view(c.num_blocks, c.Hkv, c.B // 16, 4, c.D // (16 * Y), 16, Y, 4)
    d = torch.arange(c.D)
    t = o % 16
    return vv[p, :, o // 16][:, t // 4, d // (16 * Y), d % 16, (d // 16) % Y, t % 4]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("B", [16, 32])
def test_write_places_rows_at_documented_positions(dtype, B):
    c = _case(dtype=dtype, B=B, D=64, Hkv=2, Hq=4, S=5, ctx_range=(1, 3 * B + 5), seed=3)
    k_pool, v_pool = oracle.build_pools(c)
    k_all, v_all, slots = c.all_tokens()
    written = 0
    for i, sl in enumerate(slots):
        if sl < 0:
            continue
        p, o = int(sl) // c.B, int(sl) % c.B
        got_k = k_row(c, k_pool, p, o)
        got_v = v_row(c, v_pool, p, o)
        assert torch.equal(got_k.contiguous().view(torch.uint8), k_all[i].contiguous().view(torch.uint8))
        assert torch.equal(got_v.contiguous().view(torch.uint8), v_all[i].contiguous().view(torch.uint8))
        written += 1
    # every other element still holds the poison bits
    nan_bits = W.NAN_BITS[dtype]
    ints = torch.int32 if c.elt == 4 else torch.int16
    untouched = int((k_pool.view(ints) == nan_bits).sum())
    assert untouched == c.pool_numel - written * c.Hkv * c.D
    untouched = int((v_pool.view(ints) == nan_bits).sum())
    assert untouched == c.pool_numel - written * c.Hkv * c.D


def test_write_skips_negative_slots_and_is_last_writer_wins():
    c = _case(S=2, ctx=[5, 0], ctx_range=None)
    k_pool, v_pool = c.nan_pool(), c.nan_pool()
    k = torch.randn(3, c.Hkv, c.D)
    v = torch.randn(3, c.Hkv, c.D)
    slots = np.array([-1, 7, 7], dtype=np.int64)
    oracle.write_kv(k, v, slots, k_pool, v_pool, num_blocks=c.num_blocks, B=c.B)
    assert torch.equal(v_row(c, v_pool, 0, 7), v[2])
    assert int(torch.isnan(k_pool).logical_not().sum()) == c.Hkv * c.D


def test_write_rejects_slot_past_pool():
    c = _case(S=1, ctx=[3], ctx_range=None)
    k_pool, v_pool = c.nan_pool(), c.nan_pool()
    k = torch.zeros(1, c.Hkv, c.D)
    with pytest.raises(ValueError):
        oracle.write_kv(k, k, np.array([c.num_blocks * c.B], dtype=np.int64), k_pool, v_pool,
                        num_blocks=c.num_blocks, B=c.B)


# --- widening: the oracle's own fp16/bf16 decoders against NumPy's and torch's ---

def test_widen_f16_all_bit_patterns():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    h = bits.view(torch.float16)
    ref = bits.numpy().view(np.float16).astype(np.float64)
    got = oracle.widen(h)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_widen_bf16_all_bit_patterns():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    b = bits.view(torch.bfloat16)
    ref = b.to(torch.float64).numpy()
    got = oracle.widen(b)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


# --- P2: dense non-paged attention on the same rows ---

@pytest.mark.parametrize("kw", [
    dict(dtype="f32", Hq=4, Hkv=2, D=64, B=16),
    dict(dtype="f16", Hq=8, Hkv=1, D=64, B=16),
    dict(dtype="bf16", Hq=7, Hkv=1, D=128, B=16),
    dict(dtype="bf16", Hq=8, Hkv=2, D=128, B=32),
    dict(dtype="f16", Hq=6, Hkv=6, D=64, B=32),
])
def test_matches_dense_attention(kw):
    c = _case(S=4, ctx_range=(1, 150), seed=5, **kw)
    got = oracle.decode_case(c)
    ref = dense.dense_case(c)
    assert np.abs(got - ref).max() <= 1e-12


def test_dense_covers_ragged_edges():
    # 0 tokens, one token, exactly one block, one past a block, several blocks
    c = _case(S=6, ctx=[0, 1, 16, 17, 48, 63], ctx_range=None, dtype="bf16", Hq=4, Hkv=2, D=64, B=16)
    got = oracle.decode_case(c)
    ref = dense.dense_case(c)
    assert np.abs(got - ref).max() <= 1e-12
    assert np.all(got[0] == 0.0)


# --- P3: a single key returns its value row exactly ---

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_single_key_returns_v(dtype):
    c = _case(S=3, ctx=[1, 1, 1], ctx_range=None, dtype=dtype)
    got = oracle.decode_case(c)
    for s in range(c.S):
        v = c.v_new[s].to(torch.float64).numpy()  # [Hkv, D]
        for h in range(c.Hq):
            assert np.array_equal(got[s, h], v[h // c.G])


# --- P4: moving blocks and rewriting the block table changes nothing ---

def _permuted(c, perm):
    bt = perm[c.block_tables]
    def remap(slots):
        out = slots.copy()
        ok = slots >= 0
        out[ok] = perm[slots[ok] // c.B] * c.B + slots[ok] % c.B
        return out
    return W.Case(**{**c.__dict__, "block_tables": bt.astype(np.int32),
                     "slot_prefill": remap(c.slot_prefill), "slot_new": remap(c.slot_new)})


def test_block_permutation_invariance_bitwise():
    c = _case(S=5, dtype="bf16", Hq=8, Hkv=2, D=128, B=16, ctx_range=(1, 200), seed=9)
    rng = np.random.default_rng(123)
    perm = rng.permutation(c.num_blocks)
    c2 = _permuted(c, perm)
    a = oracle.decode_case(c)
    b = oracle.decode_case(c2)
    assert np.array_equal(a, b)
    assert not np.array_equal(c.block_tables, c2.block_tables)


# --- P5: arbitrary-precision brute force on tiny inputs ---

def _brute(q, ks, vs, scale):
    getcontext().prec = 50
    z = [Decimal(float(scale)) * sum(Decimal(float(a)) * Decimal(float(b)) for a, b in zip(q, k)) for k in ks]
    e = [zz.exp() for zz in z]  # no max shift: exact arithmetic does not need it
    den = sum(e)
    return [float(sum(ei * Decimal(float(v[d])) for ei, v in zip(e, vs)) / den) for d in range(len(q))]


@pytest.mark.parametrize("dtype,D", [("f32", 16), ("f16", 32), ("bf16", 32)])
def test_bruteforce_tiny(dtype, D):
    c = _case(S=2, Hq=2, Hkv=1, D=D, B=16, dtype=dtype, ctx=[5, 3], ctx_range=None, seed=21)
    got = oracle.decode_case(c)
    for s in range(c.S):
        k, v = c.logical_kv(s)
        k = k.to(torch.float64).numpy()
        v = v.to(torch.float64).numpy()
        for h in range(c.Hq):
            q = c.q[s, h].to(torch.float64).numpy()
            ref = np.array(_brute(q, k[:, h // c.G], v[:, h // c.G], c.scale))
            assert np.allclose(got[s, h], ref, rtol=1e-14, atol=1e-15)


# --- P6: closed forms ---

def test_zero_query_gives_mean_of_values():
    c = _case(S=3, dtype="f32", ctx_range=(2, 60), seed=2)
    c.q.zero_()
    got = oracle.decode_case(c)
    for s in range(c.S):
        _, v = c.logical_kv(s)
        mean = v.to(torch.float64).mean(0).numpy()
        for h in range(c.Hq):
            assert np.allclose(got[s, h], mean[h // c.G], rtol=0, atol=1e-14)


def test_zero_scale_gives_mean_of_values():
    c = _case(S=2, dtype="bf16", ctx_range=(2, 60), seed=4, scale=0.0)
    got = oracle.decode_case(c)
    for s in range(c.S):
        _, v = c.logical_kv(s)
        mean = v.to(torch.float64).mean(0).numpy()
        for h in range(c.Hq):
            assert np.allclose(got[s, h], mean[h // c.G], rtol=0, atol=1e-14)


def test_constant_values_return_the_constant():
    c = _case(S=2, dtype="f16", ctx_range=(3, 90), seed=6)
    c.v_prefill.fill_(1.5)
    c.v_new.fill_(1.5)
    got = oracle.decode_case(c)
    assert np.abs(got - 1.5).max() <= 1e-14


def test_two_keys_sigmoid():
    c = _case(S=1, Hq=2, Hkv=1, ctx=[2], ctx_range=None, dtype="f32", seed=8)
    got = oracle.decode_case(c)
    k, v = c.logical_kv(0)
    k = k.to(torch.float64).numpy()[:, 0]
    v = v.to(torch.float64).numpy()[:, 0]
    for h in range(2):
        q = c.q[0, h].to(torch.float64).numpy()
        z0, z1 = c.scale * (q @ k[0]), c.scale * (q @ k[1])
        sig = lambda x: 1.0 / (1.0 + np.exp(-x))
        ref = sig(z0 - z1) * v[0] + sig(z1 - z0) * v[1]
        assert np.allclose(got[0, h], ref, rtol=0, atol=1e-14)


# --- P7: grouped-query heads equal multi-head attention with repeated kv-heads ---

def test_gqa_equals_mha_with_repeated_heads():
    c = _case(S=3, dtype="bf16", Hq=6, Hkv=2, D=64, B=16, ctx_range=(1, 80), seed=12)
    rep = lambda t: t.repeat_interleave(c.G, dim=1).contiguous()
    m = W.Case(**{**c.__dict__, "Hkv": c.Hq, "k_prefill": rep(c.k_prefill), "v_prefill": rep(c.v_prefill),
                  "k_new": rep(c.k_new), "v_new": rep(c.v_new)})
    assert np.array_equal(oracle.decode_case(c), oracle.decode_case(m))


def test_mqa_single_kv_head():
    c = _case(S=2, dtype="f16", Hq=5, Hkv=1, D=64, B=16, ctx_range=(1, 40), seed=13)
    rep = lambda t: t.repeat_interleave(c.G, dim=1).contiguous()
    m = W.Case(**{**c.__dict__, "Hkv": c.Hq, "k_prefill": rep(c.k_prefill), "v_prefill": rep(c.v_prefill),
                  "k_new": rep(c.k_new), "v_new": rep(c.v_new)})
    assert np.array_equal(oracle.decode_case(c), oracle.decode_case(m))


# --- P8: a log-sum-exp merge of partition results equals the unsplit answer ---

def test_partition_merge_identity():
    rng = np.random.default_rng(0)
    L, D = 300, 16
    q = rng.standard_normal(D)
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    scale = 0.25
    whole = dense.attention(q, k, v, scale)
    cuts = [0, 1, 17, 150, 151, 299, 300]
    o_p, lse_p = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        z = (k[a:b] @ q) * scale
        m = z.max()
        o_p.append(dense.attention(q, k[a:b], v[a:b], scale))
        lse_p.append(m + np.log(np.exp(z - m).sum()))
    # an empty partition carries lse = -inf and weight 0
    o_p.append(np.zeros(D))
    lse_p.append(-np.inf)
    lse_p = np.array(lse_p)
    M = lse_p.max()
    w = np.exp(lse_p - M)
    merged = (w[:, None] * np.array(o_p)).sum(0) / w.sum()
    assert np.abs(merged - whole).max() <= 1e-14


# --- P9: large logits stay finite and approach the arg-max row ---

@pytest.mark.parametrize("factor", [1e2, 1e3])
def test_large_logits_are_finite(factor):
    c = _case(S=2, dtype="f32", Hq=2, Hkv=1, D=64, B=16, ctx_range=(5, 40), seed=14)
    c.q.mul_(factor)
    got = oracle.decode_case(c)
    assert np.isfinite(got).all()
    if factor == 1e3:
        for s in range(c.S):
            k, v = c.logical_kv(s)
            for h in range(c.Hq):
                z = k[:, 0].to(torch.float64).numpy() @ c.q[s, h].to(torch.float64).numpy()
                assert np.allclose(got[s, h], v[int(np.argmax(z)), 0].to(torch.float64).numpy(), atol=1e-6)


# --- P10: NaN in tail slots and padding blocks never reaches the output ---

def test_nan_poison_does_not_leak():
    c = _case(S=4, dtype="bf16", Hq=4, Hkv=2, D=64, B=16, ctx=[3, 17, 31, 40], ctx_range=None, seed=15,
              max_blocks_per_seq=6)
    poisoned = oracle.decode_case(c)
    k0, v0 = torch.zeros_like(c.nan_pool()), torch.zeros_like(c.nan_pool())
    oracle.write_kv(*c.all_tokens(), k0, v0, num_blocks=c.num_blocks, B=c.B)
    clean = oracle.decode_case(c, k0, v0)
    assert np.isfinite(poisoned).all()
    assert np.array_equal(poisoned, clean)


def test_thread_count_does_not_change_bits():
    c = _case(S=5, dtype="f16", Hq=8, Hkv=2, D=64, B=16, ctx_range=(1, 120), seed=16)
    k, v = oracle.build_pools(c)
    a = oracle.decode_case(c, k, v, threads=1)
    b = oracle.decode_case(c, k, v, threads=7)
    assert np.array_equal(a, b)


def test_pairs_match_full_output():
    c = _case(S=4, dtype="bf16", Hq=8, Hkv=2, D=128, B=32, ctx_range=(1, 100), seed=17)
    k, v = oracle.build_pools(c)
    full = oracle.decode_case(c, k, v)
    pairs = np.array([[3, 7], [0, 0], [2, 5]])
    part = oracle.decode_case(c, k, v, pairs=pairs)
    for i, (s, h) in enumerate(pairs):
        assert np.array_equal(part[i], full[s, h])


# --- the seeded draws are the ones the workload recipe fixes ---

def test_seeded_context_lengths():
    assert list(W.config_case(1).context_lens) == [31, 33, 49, 61]
    c2 = W.make_case(seed=2, **{k: v for k, v in W.CONFIGS[2].items()})
    assert list(c2.context_lens) == [1736, 630, 337, 701, 922, 1692, 994, 304]
    assert c2.num_blocks - 1 == 577 and int(((c2.context_lens + 15) // 16).sum()) == 461


# --- Several query tokens per sequence (causal): the oracle's attend ---

def _attend(mc, threads=None):
    k_pool, v_pool = oracle.build_pools(mc.base)
    c = mc.base
    return oracle.attend(mc.q, k_pool, v_pool, c.block_tables, c.context_lens, mc.query_start, c.scale,
                         Hkv=c.Hkv, B=c.B, threads=threads)


def test_attend_with_one_token_per_sequence_is_decode():
    c = _case(S=4, Hq=8, Hkv=2, D=64, B=16, dtype="bf16", ctx_range=(1, 90), seed=31)
    mc = W.MultiCase(base=c, q=c.q.clone(), query_start=np.arange(c.S + 1, dtype=np.int32))
    assert np.array_equal(_attend(mc), oracle.decode_case(c))


@pytest.mark.parametrize("kw,q_lens", [
    (dict(S=3, Hq=4, Hkv=2, D=64, B=16, dtype="f32", ctx_range=(20, 70), seed=41), [1, 5, 20]),
    (dict(S=4, Hq=8, Hkv=2, D=128, B=32, dtype="bf16", ctx_range=(1, 90), seed=42), [4, 4, 4, 4]),
    (dict(S=3, Hq=7, Hkv=1, D=64, B=16, dtype="f16", ctx_range=(30, 50), seed=43), [0, 7, 30]),
    (dict(S=2, Hq=16, Hkv=1, D=128, B=16, dtype="bf16", ctx=[17, 33], ctx_range=None, seed=44), [17, 2]),
    (dict(S=5, Hq=4, Hkv=4, D=64, B=32, dtype="f32", ctx_range=(1, 40), seed=45), [3, 1, 0, 9, 40]),
])
def test_attend_matches_dense_causal(kw, q_lens):
    c = _case(**kw)
    mc = W.with_queries(c, q_lens, seed=kw["seed"] + 100)
    got = _attend(mc)
    ref = dense.dense_multi(mc)
    assert got.shape == ref.shape and np.max(np.abs(got - ref)) <= 1e-12


def test_attend_row_is_decode_over_its_visible_prefix():
    # Query token i of a sequence with n tokens and context L is the decode of
    # the same sequence cut to length L - n + i + 1: the same block table, the
    # query row moved into a one-token batch.
    c = _case(S=3, Hq=8, Hkv=2, D=64, B=16, dtype="bf16", ctx_range=(10, 60), seed=51)
    mc = W.with_queries(c, [6, 1, 10], seed=52)
    got = _attend(mc)
    k_pool, v_pool = oracle.build_pools(c)
    qs = mc.query_start
    for s in range(c.S):
        n = int(qs[s + 1] - qs[s])
        for i in range(n):
            row = int(qs[s]) + i
            cut = np.array([int(c.context_lens[s]) - n + i + 1], dtype=np.int32)
            ref = oracle.decode(mc.q[row:row + 1], k_pool, v_pool, c.block_tables[s:s + 1], cut, c.scale,
                                Hkv=c.Hkv, B=c.B)
            assert np.array_equal(got[row], ref[0])


@pytest.mark.parametrize("dtype,D", [("f32", 16), ("bf16", 32)])
def test_attend_bruteforce_tiny(dtype, D):
    c = _case(S=2, Hq=2, Hkv=1, D=D, B=16, dtype=dtype, ctx=[5, 3], ctx_range=None, seed=61)
    mc = W.with_queries(c, [3, 2], seed=62)
    got = _attend(mc)
    qs = mc.query_start
    for s in range(c.S):
        k, v = c.logical_kv(s)
        k = k.to(torch.float64).numpy()
        v = v.to(torch.float64).numpy()
        L, n = int(c.context_lens[s]), int(qs[s + 1] - qs[s])
        for i in range(n):
            row = int(qs[s]) + i
            vis = L - n + i + 1
            for h in range(c.Hq):
                q = mc.q[row, h].to(torch.float64).numpy()
                ref = np.array(_brute(q, k[:vis, h // c.G], v[:vis, h // c.G], c.scale))
                assert np.allclose(got[row, h], ref, rtol=1e-14, atol=1e-15)


def test_attend_zero_query_gives_mean_of_visible_prefix():
    # Closed form: with q = 0 every visible key weighs the same, so query row i
    # of a sequence returns the plain mean of V over positions 0 .. L - n + i.
    c = _case(S=3, Hq=4, Hkv=2, D=64, B=16, dtype="f32", ctx_range=(12, 50), seed=71)
    mc = W.with_queries(c, [12, 1, 5], seed=72)
    mc.q.zero_()
    got = _attend(mc)
    qs = mc.query_start
    for s in range(c.S):
        _, v = c.logical_kv(s)
        v = v.to(torch.float64).numpy()
        L, n = int(c.context_lens[s]), int(qs[s + 1] - qs[s])
        for i in range(n):
            for h in range(c.Hq):
                ref = v[:L - n + i + 1, h // c.G].mean(axis=0)
                assert np.max(np.abs(got[int(qs[s]) + i, h] - ref)) <= 1e-13


def test_attend_rejects_more_queries_than_context():
    c = _case(S=2, Hq=4, Hkv=2, D=64, B=16, dtype="f32", ctx=[3, 5], ctx_range=None, seed=81)
    q = torch.zeros((7, c.Hq, c.D), dtype=torch.float32)
    k_pool, v_pool = oracle.build_pools(c)
    with pytest.raises(ValueError):
        oracle.attend(q, k_pool, v_pool, c.block_tables, c.context_lens, np.array([0, 4, 7], dtype=np.int32),
                      c.scale, Hkv=c.Hkv, B=c.B)


def test_attend_thread_count_does_not_change_bits():
    c = _case(S=4, Hq=8, Hkv=2, D=64, B=16, dtype="f16", ctx_range=(5, 80), seed=91)
    mc = W.with_queries(c, [3, 5, 1, 4], seed=92)
    assert np.array_equal(_attend(mc, threads=1), _attend(mc, threads=7))


# --- RoPE (rotate-half pairing) and the single rounding into the dtype ---

def _rope_np(x, pos, theta):
    """The same rotation as complex multiplication: (x_i + i x_{i+D/2}) * exp(i p w_i)."""
    D = x.shape[-1]
    w = theta ** (-2.0 * np.arange(D // 2) / D)
    z = (x[..., :D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * pos[:, None, None] * w[None, None, :])
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128), ("f16", 128)])
def test_rope_matches_complex_rotation(dtype, D):
    rng = np.random.default_rng(5)
    x = W._normal(rng, (7, 3, D), dtype)
    pos = np.array([0, 1, 2, 17, 1000, 4095, 131071], dtype=np.int32)
    got = oracle.rope(x, pos, 10000.0)
    ref = _rope_np(x.double().numpy(), pos.astype(np.float64), 10000.0)
    assert np.max(np.abs(got - ref)) <= 1e-9 * np.max(np.abs(ref))


def test_rope_position_zero_is_identity_and_pairs_keep_their_norm():
    rng = np.random.default_rng(6)
    x = W._normal(rng, (5, 2, 64), "f32")
    pos = np.array([0, 3, 9, 100, 5000], dtype=np.int32)
    got = oracle.rope(x, pos, 500000.0)
    xd = x.double().numpy()
    assert np.array_equal(got[0], xd[0])
    n_in = xd[..., :32] ** 2 + xd[..., 32:] ** 2
    n_out = got[..., :32] ** 2 + got[..., 32:] ** 2
    assert np.max(np.abs(n_in - n_out)) <= 1e-12 * np.max(n_in)


def test_rope_first_pair_turns_by_the_position_in_radians():
    # w_0 = theta^0 = 1: dims 0 and D/2 rotate by exactly p radians.
    x = torch.zeros((3, 1, 64), dtype=torch.float32)
    x[:, 0, 0] = 1.0
    pos = np.array([1, 2, 3], dtype=np.int32)
    got = oracle.rope(x, pos, 10000.0)
    for t, p in enumerate(pos):
        assert got[t, 0, 0] == pytest.approx(np.cos(p), abs=1e-15)
        assert got[t, 0, 32] == pytest.approx(np.sin(p), abs=1e-15)
    # the last pair turns at w = theta^(-(D-2)/D)
    x = torch.zeros((1, 1, 64), dtype=torch.float32)
    x[0, 0, 31] = 1.0
    got = oracle.rope(x, np.array([1000], dtype=np.int32), 10000.0)
    w = 10000.0 ** (-62 / 64)
    assert got[0, 0, 31] == pytest.approx(np.cos(1000 * w), abs=1e-13)
    assert got[0, 0, 63] == pytest.approx(np.sin(1000 * w), abs=1e-13)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(7)
    q = W._normal(rng, (1, 1, 128), "f32")
    k = W._normal(rng, (1, 1, 128), "f32")
    def score(m, n):
        a = oracle.rope(q, np.array([m], dtype=np.int32), 10000.0)[0, 0]
        b = oracle.rope(k, np.array([n], dtype=np.int32), 10000.0)[0, 0]
        return float(a @ b)
    for m, n in [(5, 2), (40, 37), (1003, 1000)]:
        assert score(m, n) == pytest.approx(score(m - n, 0), rel=1e-10, abs=1e-10)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_round_matches_single_rounding_of_floats(dtype):
    # For values a float holds exactly, one rounding from double must equal
    # torch's float -> dtype rounding (itself to nearest, ties to even).
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(200000) * rng.choice([1e-6, 1e-3, 1.0, 30.0, 3e4], 200000)).astype(np.float32)
    # add exact ties: midpoints between neighbouring dtype values
    a = torch.from_numpy(x[:1000]).to(dtype)
    b = torch.nextafter(a.float(), torch.full_like(a.float(), float("inf"))).to(dtype)
    mids = ((a.double() + b.double()) / 2).float().numpy()
    x = np.concatenate([x, mids])
    got = oracle.round_to(x.astype(np.float64), dtype)
    ref = torch.from_numpy(x).to(dtype)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_round_is_one_step_from_double():
    # 1 + 2^-8 + 2^-30 lies just above the bf16 midpoint 1 + 2^-8: one rounding
    # gives 1 + 2^-7; rounding to float first would land on the midpoint and
    # then round to even, 1.
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30, -(1.0 + 2.0 ** -8 + 2.0 ** -30)])
    got = oracle.round_to(x, torch.bfloat16).double().numpy()
    assert list(got) == [1.0 + 2.0 ** -7, -(1.0 + 2.0 ** -7)]
