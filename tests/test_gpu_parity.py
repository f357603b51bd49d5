"""GPU parity: the HIP library against the float64 CPU oracle, through the C ABI.

pa_write_kv must reproduce the oracle's pools byte for byte (NaN poison in
every unwritten byte included); pa_decode must agree with the oracle within
the stated bound per dtype (max-abs 1e-5 fp32, 2e-3 fp16, 1.5e-2 bf16) on
every output element, for every work split, on all five workloads at full
size and on small shapes that cover the edges.  The 16-bit workloads are
also held to a per-element bound derived from the kernel's arithmetic, and
the three large ones run again as f32 twins (same lengths, tables and draws,
not rounded) at 1e-5, where losing a single 16-token block of a sequence
already moves the output by far more than the bound.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_slot_amd as pa
from paged_kv_decode_slot_amd import workloads as W
from tests.gpu_helpers import (TOL, GpuCase, check_output, dev_bits, flat_bits, log, max_abs_err,
                               oracle_pools)

pytestmark = pytest.mark.gpu

# The five workloads, then f32 twins of the three large ones.
WORKLOADS = [1, 2, 3, 4, 5, "3f", "4f", "5f"]

_memo = {}


def workload_case(n):
    return W.twin_case(int(n[0]), "f32") if isinstance(n, str) else W.config_case(n)


def config_state(n):
    """Case, GPU side (appended), oracle pools, oracle output and the oracle's
    softmax average of |V| for workload n; one workload held at a time."""
    if n not in _memo:
        _memo.clear()
        torch.cuda.empty_cache()
        log(f"[setup] workload {n}: drawing inputs")
        case = workload_case(n)
        g = GpuCase(case)
        g.append()
        torch.cuda.synchronize()
        log(f"[setup] workload {n}: oracle pools and output")
        kp, vp = oracle_pools(case)
        ref = oracle.decode_case(case, kp, vp)
        abs_v = oracle.decode_case(case, kp, vp.abs())
        _memo[n] = (case, g, kp, vp, ref, abs_v)
    return _memo[n]


@pytest.mark.parametrize("n", WORKLOADS)
def test_write_kv_pools_bitexact(n):
    case, g, kp, vp, _, _ = config_state(n)
    log(f"[write] workload {n}: comparing {case.pool_numel * case.elt * 2 / 1e9:.2f} GB of pool bytes")
    assert torch.equal(flat_bits(g.k_cache), flat_bits(kp))
    assert torch.equal(flat_bits(g.v_cache), flat_bits(vp))


@pytest.mark.parametrize("workers", [0, -1, 7, 3000])
@pytest.mark.parametrize("n", WORKLOADS)
def test_decode_parity_workloads(n, workers):
    case, g, _, _, ref, abs_v = config_state(n)
    log(f"[decode] workload {n} workers={workers}")
    out = g.decode(num_workers=workers)
    torch.cuda.synchronize()
    check_output(out, ref, abs_v, case.dtype, f"[decode] workload {n} workers={workers}")


@pytest.mark.parametrize("n", [3, 4, 5, "3f", "5f"])
def test_pa_decode_entry_point(n):
    """pa_decode itself (the automatic split), called through ctypes with a
    workspace sized by pa_decode_workspace_bytes: within the bounds, and bitwise
    the same as pa_decode_ex with num_workers = 0."""
    case, g, _, _, ref, abs_v = config_state(n)
    L = pa.lib()
    desc = pa.cache_desc(g.k_cache, g.v_cache)
    need = int(L.pa_decode_workspace_bytes(case.S, case.Hq, case.max_blocks_per_seq, ctypes.byref(desc)))
    assert need >= int(L.pa_workspace_sync_bytes())
    ws = pa.new_workspace(need, g.q.device)
    out = torch.empty_like(g.q)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    log(f"[pa_decode] workload {n}: workspace {need} bytes")
    st = L.pa_decode(g.q.data_ptr(), g.k_cache.data_ptr(), g.v_cache.data_ptr(), g.bt.data_ptr(), g.ctx.data_ptr(),
                     ctypes.c_float(case.scale), out.data_ptr(), case.S, case.Hq, case.max_blocks_per_seq,
                     ctypes.byref(desc), ws.data_ptr(), need, stream)
    assert st == 0, L.pa_status_string(st)
    torch.cuda.synchronize()
    check_output(out, ref, abs_v, case.dtype, f"[pa_decode] workload {n}")
    assert int(ws[:int(L.pa_workspace_sync_bytes())].count_nonzero()) == 0  # synchronisation words back at zero
    assert torch.equal(dev_bits(out), dev_bits(g.decode(num_workers=0)))


@pytest.mark.parametrize("n", [3, 4])
def test_decode_leaves_caches_and_inputs_unchanged(n):
    case, g, kp, vp, _, _ = config_state(n)
    kb, vb = g.k_cache.clone(), g.v_cache.clone()
    qb, btb, cb = g.q.clone(), g.bt.clone(), g.ctx.clone()
    g.decode()
    torch.cuda.synchronize()
    assert torch.equal(dev_bits(g.k_cache), dev_bits(kb)) and torch.equal(dev_bits(g.v_cache), dev_bits(vb))
    assert torch.equal(dev_bits(g.q), dev_bits(qb)) and torch.equal(g.bt, btb) and torch.equal(g.ctx, cb)


@pytest.mark.parametrize("n", [2, 3])
def test_decode_bitwise_deterministic(n):
    _, g, _, _, _, _ = config_state(n)
    for workers in (0, -1, 123):
        a = g.decode(num_workers=workers)
        b = g.decode(num_workers=workers)
        torch.cuda.synchronize()
        assert torch.equal(dev_bits(a), dev_bits(b))


SMALL = [
    dict(S=5, Hq=8, Hkv=2, D=128, B=16, dtype="bf16", ctx_range=(1, 300)),
    dict(S=3, Hq=16, Hkv=1, D=64, B=32, dtype="f16", ctx_range=(1, 200)),  # G = 16
    dict(S=7, Hq=3, Hkv=3, D=128, B=32, dtype="bf16", ctx_range=(1, 100)),  # G = 1
    dict(S=4, Hq=7, Hkv=1, D=128, B=16, dtype="f32", ctx_range=(1, 90)),
    dict(S=6, Hq=4, Hkv=2, D=64, B=32, dtype="f32", ctx_range=(1, 150)),
    dict(S=9, Hq=12, Hkv=4, D=64, B=16, dtype="f16", ctx_range=(1, 700)),
    dict(S=8, Hq=6, Hkv=2, D=128, B=32, dtype="bf16", ctx=[0, 1, 15, 16, 17, 32, 33, 0], max_blocks_per_seq=4),
    dict(S=6, Hq=4, Hkv=4, D=64, B=16, dtype="f32", ctx=[0, 0, 0, 1, 0, 2]),
    dict(S=1, Hq=5, Hkv=1, D=64, B=16, dtype="bf16", ctx=[3000]),
    dict(S=40, Hq=2, Hkv=1, D=128, B=16, dtype="f16", ctx_range=(1, 40), max_blocks_per_seq=9),
    dict(S=5, Hq=24, Hkv=12, D=64, B=16, dtype="bf16", ctx_range=(1, 400)),  # six slices of 2 kv-heads
    dict(S=3, Hq=32, Hkv=16, D=128, B=32, dtype="f16", ctx_range=(1, 500)),  # eight slices of 2 kv-heads
    dict(S=4, Hq=12, Hkv=6, D=64, B=16, dtype="f32", ctx_range=(1, 300)),  # three slices of 2 kv-heads
]


@pytest.mark.parametrize("workers", [0, -1, 1, 3, 50, 10000])
@pytest.mark.parametrize("idx", range(len(SMALL)))
def test_decode_parity_small_shapes(idx, workers):
    kw = dict(SMALL[idx])
    case = W.make_case(seed=100 + idx, **kw)
    log(f"[small] {idx} {kw} workers={workers}")
    g = GpuCase(case)
    g.append()
    kp, vp = oracle_pools(case)
    assert torch.equal(flat_bits(g.k_cache), flat_bits(kp)) and torch.equal(flat_bits(g.v_cache), flat_bits(vp))
    ref = oracle.decode_case(case, kp, vp)
    out = g.decode(num_workers=workers)
    torch.cuda.synchronize()
    err = max_abs_err(out, ref)
    log(f"[small] {idx} workers={workers}: max abs err {err:.3e}")
    assert err <= TOL[case.dtype]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_single_key_returns_v_exactly(dtype):
    case = W.make_case(S=5, Hq=8, Hkv=2, D=64, B=16, dtype=dtype, ctx=[1, 1, 1, 1, 1], seed=7)
    g = GpuCase(case)
    g.append()
    for workers in (0, -1):
        out = g.decode(num_workers=workers).cpu()
        expect = case.v_new.repeat_interleave(case.G, dim=1)
        assert torch.equal(dev_bits(out), dev_bits(expect))


def test_block_permutation_invariance_bitwise():
    case = W.make_case(S=6, Hq=8, Hkv=2, D=128, B=16, dtype="bf16", ctx_range=(100, 900), seed=31)
    perm = np.random.default_rng(5).permutation(case.num_blocks)

    def remap(slots):
        out = slots.copy()
        ok = slots >= 0
        out[ok] = perm[slots[ok] // case.B] * case.B + slots[ok] % case.B
        return out

    moved = W.Case(**{**case.__dict__, "block_tables": perm[case.block_tables].astype(np.int32),
                      "slot_prefill": remap(case.slot_prefill), "slot_new": remap(case.slot_new)})
    a, b = GpuCase(case), GpuCase(moved)
    a.append()
    b.append()
    for workers in (0, -1, 17):
        oa, ob = a.decode(num_workers=workers), b.decode(num_workers=workers)
        torch.cuda.synchronize()
        assert torch.equal(dev_bits(oa), dev_bits(ob))


@pytest.mark.parametrize("factor", [10.0, 100.0])
def test_large_logits_stay_finite(factor):
    case = W.make_case(S=4, Hq=8, Hkv=2, D=128, B=16, dtype="bf16", ctx_range=(50, 400), seed=41)
    case.q = (case.q.float() * factor).to(case.q.dtype)
    g = GpuCase(case)
    g.append()
    ref = oracle.decode_case(case)
    for workers in (0, -1, 200):
        out = g.decode(num_workers=workers)
        torch.cuda.synchronize()
        assert max_abs_err(out, ref) <= TOL["bf16"]


def test_write_kv_padding_slots_skipped():
    case = W.make_case(S=6, Hq=4, Hkv=2, D=64, B=16, dtype="f16", ctx=[5, 0, 9, 0, 1, 30], seed=51)
    assert (case.slot_new < 0).sum() == 2
    g = GpuCase(case)
    g.append()
    kp, vp = oracle_pools(case)
    assert torch.equal(flat_bits(g.k_cache), flat_bits(kp)) and torch.equal(flat_bits(g.v_cache), flat_bits(vp))


def test_zero_sequences_is_a_noop():
    case = W.make_case(S=2, Hq=4, Hkv=2, D=64, B=16, dtype="bf16", ctx=[3, 4], seed=1)
    g = GpuCase(case)
    g.append()
    import paged_kv_decode_slot_amd as pa
    out = pa.decode(g.q[:0], g.k_cache, g.v_cache, g.bt[:0], g.ctx[:0], case.scale)
    assert out.shape == (0, 4, 64)


def _split_case():
    return W.make_case(S=12, Hq=8, Hkv=2, D=128, B=16, dtype="bf16", ctx_range=(200, 1500), seed=61)


def _sync_bytes():
    return int(pa.lib().pa_workspace_sync_bytes())


def test_workspace_partials_need_no_initialisation():
    """Only the synchronisation words must start at zero: the partial-result
    area may hold anything, and every call leaves the words at zero."""
    case = _split_case()
    g = GpuCase(case)
    g.append()
    ref = oracle.decode_case(case)
    desc = pa.cache_desc(g.k_cache, g.v_cache)
    sync = _sync_bytes()
    for workers in (0, 37, 700):
        need = pa.workspace_bytes(case.S, case.Hq, case.max_blocks_per_seq, desc, workers)
        fills = [torch.full((need,), f, dtype=torch.uint8, device="cuda:0") for f in (0x00, 0xFF, 0x5A)]
        fills.append(torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda:0"))
        first = None
        for ws in fills:
            ws[:sync].zero_()
            for _ in range(3):  # the same workspace again and again
                out = pa.decode(g.q, g.k_cache, g.v_cache, g.bt, g.ctx, case.scale, num_workers=workers,
                                workspace=ws)
                torch.cuda.synchronize()
                assert max_abs_err(out, ref) <= TOL["bf16"]
                assert int(ws[:sync].count_nonzero()) == 0
                if first is None:
                    first = out.clone()
                assert torch.equal(dev_bits(out), dev_bits(first))


def test_workspace_reused_across_shapes():
    """One workspace, zeroed once, serves calls of different shapes in turn: a
    later call's synchronisation words never land on an earlier call's
    partial results (they sit at a fixed place at the start)."""
    cases = [W.make_case(S=S, Hq=8, Hkv=2, D=128, B=16, dtype="bf16", ctx_range=(50, 1200), seed=70 + S)
             for S in (3, 40, 9, 120)]
    gs = []
    for c in cases:
        g = GpuCase(c)
        g.append()
        gs.append((c, g, oracle.decode_case(c)))
    desc = pa.cache_desc(gs[0][1].k_cache, gs[0][1].v_cache)
    plans = [(0, 3000, 5, 1000), (3000, 0, 777, 64)]
    need = max(pa.workspace_bytes(c.S, c.Hq, c.max_blocks_per_seq, pa.cache_desc(g.k_cache, g.v_cache), w)
               for workers in plans for (c, g, _), w in zip(gs, workers))
    ws = pa.new_workspace(need, "cuda:0")
    for rnd, workers in enumerate(plans):
        for (c, g, ref), w in zip(gs, workers):
            log(f"[workspace] round {rnd}: S={c.S} workers={w}")
            out = pa.decode(g.q, g.k_cache, g.v_cache, g.bt, g.ctx, c.scale, num_workers=w, workspace=ws)
            torch.cuda.synchronize()
            assert max_abs_err(out, ref) <= TOL["bf16"]
            assert int(ws[:_sync_bytes()].count_nonzero()) == 0


def test_graph_replay_matches_eager():
    """A captured decode replays correctly: each replay finds the synchronisation words at zero again."""
    import paged_kv_decode_slot_amd as pa
    case = _split_case()
    g = GpuCase(case)
    g.append()
    out = torch.empty_like(g.q)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call = pa.prepare_decode(g.q, g.k_cache, g.v_cache, g.bt, g.ctx, case.scale, out, num_workers=300)
        call()
        stream.synchronize()
        eager = out.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            call()
    for i in range(4):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dev_bits(out), dev_bits(eager)), f"replay {i}"
        # eager work on the same workspace between replays
        call()
        torch.cuda.synchronize()


# ---- the fused step (pa_decode_append) against the two calls it replaces ----

@pytest.mark.parametrize("workers", [0, -1, 37])
@pytest.mark.parametrize("n", WORKLOADS)
def test_decode_append_matches_write_then_decode(n, workers):
    case, g, kp, vp, ref, abs_v = config_state(n)
    log(f"[fused] workload {n} workers={workers}")
    f = GpuCase(case)  # prefill only; the step appends
    out_f = f.decode_append(num_workers=workers)
    out_s = g.decode(num_workers=workers)
    torch.cuda.synchronize()
    assert torch.equal(dev_bits(out_f), dev_bits(out_s))
    assert torch.equal(dev_bits(f.k_cache), dev_bits(g.k_cache)) and torch.equal(dev_bits(f.v_cache),
                                                                                 dev_bits(g.v_cache))
    check_output(out_f, ref, abs_v, case.dtype, f"[fused] workload {n} workers={workers}")
    del f
    torch.cuda.empty_cache()


@pytest.mark.parametrize("workers", [0, -1, 3, 10000])
@pytest.mark.parametrize("idx", range(len(SMALL)))
def test_decode_append_small_shapes(idx, workers):
    kw = dict(SMALL[idx])
    case = W.make_case(seed=200 + idx, **kw)
    log(f"[fused small] {idx} {kw} workers={workers}")
    f = GpuCase(case)
    out_f = f.decode_append(num_workers=workers)
    g = GpuCase(case)
    g.append()
    out_s = g.decode(num_workers=workers)
    torch.cuda.synchronize()
    assert torch.equal(dev_bits(out_f), dev_bits(out_s))
    kp, vp = oracle_pools(case)
    assert torch.equal(flat_bits(f.k_cache), flat_bits(kp)) and torch.equal(flat_bits(f.v_cache), flat_bits(vp))
    assert max_abs_err(out_f, oracle.decode_case(case, kp, vp)) <= TOL[case.dtype]
