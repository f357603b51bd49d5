"""GPU parity of pa_attend (several query tokens per sequence, causal) against
the oracle, through the C ABI.  Pools hold every position (prefill and new
tokens), written by the library's pa_write_kv; the oracle builds its own."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_slot_amd as pa
from paged_kv_decode_slot_amd import workloads as W
from tests.gpu_helpers import TOL, GpuCase, check_output, dev_bits, log, max_abs_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu(case: W.Case) -> GpuCase:
    g = GpuCase(case)
    g.append()  # every position is in the cache before attend
    return g


def _attend(g: GpuCase, mc: W.MultiCase, workers=0):
    qs = torch.from_numpy(mc.query_start).to(DEV)
    return pa.attend(mc.q.to(DEV), g.k_cache, g.v_cache, g.bt, g.ctx, qs, mc.max_q_len, g.case.scale,
                     num_workers=workers)


def _oracle(mc: W.MultiCase, with_abs_v: bool = False):
    """The oracle's answer, and with with_abs_v also its softmax average of |V|
    (the same attention with |V| in place of V), which the derived bound uses."""
    c = mc.base
    kp, vp = oracle.build_pools(c)
    ref = oracle.attend(mc.q, kp, vp, c.block_tables, c.context_lens, mc.query_start, c.scale, Hkv=c.Hkv, B=c.B)
    if not with_abs_v:
        return ref
    return ref, oracle.attend(mc.q, kp, vp.abs(), c.block_tables, c.context_lens, mc.query_start, c.scale,
                              Hkv=c.Hkv, B=c.B)


def _q_lens(case: W.Case, kind: str, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    ctx = case.context_lens.astype(np.int64)
    if kind == "one":
        return np.ones(case.S, dtype=np.int64)
    if kind == "spec4":
        return np.full(case.S, 4)
    if kind == "full":  # the whole context is the prompt
        return ctx.copy()
    # a mix of decode tokens, short drafts and prompt chunks
    return rng.choice([0, 1, 1, 2, 3, 5, 16, 17, 40], size=case.S)


SHAPES = [
    (dict(S=5, Hq=8, Hkv=2, D=128, B=16, dtype="bf16", ctx_range=(1, 300)), "mix"),
    (dict(S=3, Hq=16, Hkv=1, D=64, B=32, dtype="f16", ctx_range=(1, 200)), "mix"),  # G = 16: one token a pair
    (dict(S=7, Hq=3, Hkv=3, D=128, B=32, dtype="bf16", ctx_range=(1, 100)), "spec4"),  # G = 1: 16 tokens a pair
    (dict(S=4, Hq=7, Hkv=1, D=128, B=16, dtype="f32", ctx_range=(1, 90)), "mix"),  # G = 7: 2 tokens, 14 columns
    (dict(S=6, Hq=4, Hkv=2, D=64, B=32, dtype="f32", ctx_range=(1, 150)), "full"),
    (dict(S=8, Hq=6, Hkv=2, D=128, B=32, dtype="bf16", ctx=[0, 1, 15, 16, 17, 32, 33, 0],
          max_blocks_per_seq=4), "full"),
    (dict(S=9, Hq=12, Hkv=4, D=64, B=16, dtype="f16", ctx_range=(1, 700)), "mix"),
    (dict(S=1, Hq=4, Hkv=1, D=64, B=16, dtype="bf16", ctx=[3000]), "spec4"),
]


@pytest.mark.parametrize("workers", [0, -1, 3, 10000])
@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_attend_small_shapes(idx, workers):
    kw, kind = SHAPES[idx]
    case = W.make_case(seed=300 + idx, name=f"mq{idx}", **kw)
    mc = W.with_queries(case, _q_lens(case, kind, 400 + idx), seed=500 + idx)
    log(f"[attend] shape {idx} ({kind}) workers {workers} q_lens {mc.q_lens.tolist()[:10]}")
    out = _attend(_gpu(case), mc, workers)
    torch.cuda.synchronize()
    assert max_abs_err(out, _oracle(mc)) <= TOL[case.dtype]


@pytest.mark.parametrize("workers", [0, 37])
def test_attend_one_token_each_is_decode_bitwise(workers):
    case = W.config_case(3)
    g = _gpu(case)
    mc = W.MultiCase(base=case, q=case.q.clone(), query_start=np.arange(case.S + 1, dtype=np.int32))
    log(f"[attend] one token each, C3, workers {workers}")
    a = _attend(g, mc, workers)
    d = g.decode(num_workers=workers)
    torch.cuda.synchronize()
    assert torch.equal(dev_bits(a), dev_bits(d))


def test_attend_speculative_verify_llama3_shape():
    # Four draft tokens per sequence on the Llama-3-8B-shaped batch: one launch,
    # every K/V row read once.
    case = W.config_case(3)
    mc = W.with_queries(case, np.full(case.S, 4), seed=601)
    log("[attend] C3 with 4 query tokens per sequence")
    out = _attend(_gpu(case), mc)
    torch.cuda.synchronize()
    assert max_abs_err(out, _oracle(mc)) <= TOL[case.dtype]


def test_attend_prompt_chunks_mixed_with_decode():
    case = W.make_case(S=6, Hq=32, Hkv=8, D=128, B=16, dtype="bf16", ctx_range=(300, 2000), seed=611, name="mix")
    mc = W.with_queries(case, [1, 1, 64, 300, 1, 17], seed=612)
    log(f"[attend] chunked prompts with decode, q_lens {mc.q_lens.tolist()}")
    g = _gpu(case)
    out = _attend(g, mc)
    again = _attend(g, mc)
    torch.cuda.synchronize()
    assert max_abs_err(out, _oracle(mc)) <= TOL[case.dtype]
    assert torch.equal(dev_bits(out), dev_bits(again))  # run to run, bitwise


def test_attend_no_query_tokens_is_a_noop():
    case = W.make_case(S=3, Hq=4, Hkv=2, D=64, B=16, dtype="f16", ctx_range=(5, 40), seed=621, name="none")
    g = _gpu(case)
    qs = torch.zeros(case.S + 1, dtype=torch.int32, device=DEV)
    q = torch.empty((0, case.Hq, case.D), dtype=torch.float16, device=DEV)
    out = pa.attend(q, g.k_cache, g.v_cache, g.bt, g.ctx, qs, 0, case.scale)
    torch.cuda.synchronize()
    assert out.shape == (0, case.Hq, case.D)


def test_attend_query_start_is_clamped_to_the_rows():
    """query_start values outside [0, num_q_rows] are clamped: a first entry
    below 0 and a last entry past the rows give exactly the answer of the
    well-formed call, and rows past num_q_rows (guard rows here) stay untouched."""
    case = W.make_case(S=5, Hq=8, Hkv=2, D=128, B=16, dtype="bf16", ctx_range=(40, 300), seed=631, name="clamp")
    mc = W.with_queries(case, [3, 1, 7, 2, 5], seed=632)
    g = _gpu(case)
    R = int(mc.query_start[-1])
    qs = torch.from_numpy(mc.query_start).to(DEV)
    good = pa.attend(mc.q.to(DEV), g.k_cache, g.v_cache, g.bt, g.ctx, qs, mc.max_q_len, case.scale)
    bad = mc.query_start.copy()
    bad[0], bad[-1] = -4, R + 5
    log(f"[attend] clamped query_start {bad.tolist()} over {R} rows")
    q_full = torch.empty((R + 2, case.Hq, case.D), dtype=torch.bfloat16, device=DEV)
    q_full[:R] = mc.q.to(DEV)
    q_full[R:] = float("nan")
    out_full = torch.full((R + 2, case.Hq, case.D), 7.0, dtype=torch.bfloat16, device=DEV)
    pa.attend(q_full[:R], g.k_cache, g.v_cache, g.bt, g.ctx, torch.from_numpy(bad).to(DEV), mc.max_q_len,
              case.scale, out=out_full[:R])
    torch.cuda.synchronize()
    assert torch.equal(dev_bits(out_full[:R]), dev_bits(good))
    assert bool((out_full[R:] == 7.0).all())


# ---- prompt chunks: sequences with more query tokens than one chunk_kernel wave holds ----

CHUNK_SHAPES = [
    # Llama-3-8B-shaped layer: prompt chunks of 64 to 512 tokens beside decode tokens and drafts
    (dict(S=12, Hq=32, Hkv=8, D=128, B=16, dtype="bf16", ctx_range=(600, 2500)),
     [1, 1, 64, 128, 1, 256, 512, 1, 3, 17, 300, 1]),
    # Qwen2-like G = 7 (2 tokens, 14 columns a tile), block 32, fp16
    (dict(S=6, Hq=28, Hkv=4, D=128, B=32, dtype="f16", ctx_range=(300, 1400)), [1, 200, 33, 1, 96, 5]),
    # TinyLlama-like G = 8, d64, f32 (two column tiles a wave)
    (dict(S=5, Hq=32, Hkv=4, D=64, B=16, dtype="f32", ctx_range=(100, 700)), [70, 1, 2, 150, 9]),
    # G = 1 (16 tokens a tile): whole prompts, lengths at block edges
    (dict(S=6, Hq=4, Hkv=4, D=64, B=32, dtype="bf16", ctx=[65, 64, 129, 200, 31, 300]), [65, 64, 129, 200, 31, 300]),
    # G = 16 (one token a tile), prompt longer than a block
    (dict(S=3, Hq=16, Hkv=1, D=128, B=16, dtype="bf16", ctx=[90, 400, 17]), [90, 40, 17]),
    # G = 4: 5..8 tokens fill one query block (the chunk kernel's single-block form),
    # 9 and 16 two, 1 goes to the split path
    (dict(S=7, Hq=32, Hkv=8, D=128, B=16, dtype="bf16", ctx_range=(20, 900)), [5, 6, 7, 8, 1, 9, 16]),
    # G = 2, 64-dim f16 rows (four column tiles: 32 tokens a block), block 32
    (dict(S=4, Hq=8, Hkv=4, D=64, B=32, dtype="f16", ctx_range=(100, 600)), [9, 40, 1, 100]),
]


@pytest.mark.parametrize("idx", range(len(CHUNK_SHAPES)))
def test_attend_prompt_chunks(idx):
    kw, q_lens = CHUNK_SHAPES[idx]
    case = W.make_case(seed=700 + idx, name=f"chunk{idx}", **kw)
    mc = W.with_queries(case, q_lens, seed=800 + idx)
    log(f"[chunks] shape {idx}: q_lens {mc.q_lens.tolist()}, ctx {case.context_lens.tolist()}")
    g = _gpu(case)
    out = _attend(g, mc)
    again = _attend(g, mc)
    torch.cuda.synchronize()
    check_output(out, *_oracle(mc, True), case.dtype, f"[chunks] shape {idx}")
    assert torch.equal(dev_bits(out), dev_bits(again))  # run to run, bitwise


def test_attend_chunks_on_llama3_batch():
    """The Llama-3-8B-shaped batch with 8 of its 64 sequences carrying prompt
    chunks of 64 to 512 tokens and the rest one decode token each."""
    case = W.config_case(3)
    q_lens = np.ones(case.S, dtype=np.int64)
    q_lens[::8] = [64, 96, 128, 200, 256, 300, 400, 512]
    mc = W.with_queries(case, q_lens, seed=901)
    log(f"[chunks] C3 with prompt chunks {mc.q_lens[::8].tolist()}")
    out = _attend(_gpu(case), mc)
    torch.cuda.synchronize()
    check_output(out, *_oracle(mc, True), case.dtype, "[chunks] C3 mixed")


def test_attend_drafts_on_llama3_batch():
    """Eight draft tokens on each of the 64 sequences of the Llama-3-8B-shaped batch:
    every sequence is one query block of the prompt-chunk kernel."""
    case = W.config_case(3)
    mc = W.with_queries(case, np.full(case.S, 8), seed=911)
    log("[chunks] C3 with 8 query tokens per sequence")
    g = _gpu(case)
    out = _attend(g, mc)
    again = _attend(g, mc)
    torch.cuda.synchronize()
    check_output(out, *_oracle(mc, True), case.dtype, "[chunks] C3 8 each")
    assert torch.equal(dev_bits(out), dev_bits(again))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attend_negative_scale(dtype):
    """A negative scale (the softmax of -q.k) on both paths: draft tokens on the
    split path and prompt chunks on the prompt-chunk kernel."""
    case = W.make_case(S=5, Hq=8, Hkv=2, D=128, B=16, dtype=dtype, ctx_range=(40, 700), seed=931, name="neg")
    mc = W.with_queries(case, [2, 40, 1, 17, 9], seed=932)
    neg = -case.scale
    g = _gpu(case)
    qs = torch.from_numpy(mc.query_start).to(DEV)
    log(f"[attend] negative scale {neg}, {dtype}, q_lens {mc.q_lens.tolist()}")
    out = pa.attend(mc.q.to(DEV), g.k_cache, g.v_cache, g.bt, g.ctx, qs, mc.max_q_len, neg)
    torch.cuda.synchronize()
    kp, vp = oracle.build_pools(case)
    ref = oracle.attend(mc.q, kp, vp, case.block_tables, case.context_lens, mc.query_start, neg, Hkv=case.Hkv, B=case.B)
    assert max_abs_err(out, ref) <= TOL[case.dtype]


@pytest.mark.parametrize("S,D", [(4096, 64), (8192, 128)])
def test_decode_and_attend_at_the_sequence_cap(S, D):
    """Thousands of sequences, up to 8192 (the most one call takes: every workgroup
    holds per-sequence tables in LDS), through pa_decode_ex and through pa_attend
    with prompt chunks on every 512th sequence."""
    case = W.make_case(S=S, Hq=8, Hkv=2, D=D, B=16, dtype="bf16", ctx_range=(1, 40), seed=41 + D, name="cap")
    g = _gpu(case)
    log(f"[cap] {S} sequences, D {D}: decode")
    out = g.decode(num_workers=0)
    torch.cuda.synchronize()
    kp, vp = oracle.build_pools(case)
    check_output(out, oracle.decode_case(case, kp, vp), oracle.decode_case(case, kp, vp.abs()), case.dtype,
                 f"[cap] decode D {D}")
    ql = np.where(np.arange(case.S) % 512 == 0, np.minimum(case.context_lens, 20), 1)
    mc = W.with_queries(case, ql, seed=7)
    log(f"[cap] {S} sequences, D {D}: attend, q_lens up to {mc.max_q_len}")
    out = _attend(g, mc)
    torch.cuda.synchronize()
    check_output(out, *_oracle(mc, True), case.dtype, f"[cap] attend D {D}")


def test_attend_graph_replay_matches_eager():
    """pa_attend with prompt chunks and decode tokens (both launches) captured in a
    graph: every replay finds the item counters and arrival words at zero again."""
    case = W.make_case(S=6, Hq=32, Hkv=8, D=128, B=16, dtype="bf16", ctx_range=(300, 2000), seed=941, name="graph")
    mc = W.with_queries(case, [1, 3, 64, 200, 1, 17], seed=942)
    g = _gpu(case)
    q = mc.q.to(DEV)
    qs = torch.from_numpy(mc.query_start).to(DEV)
    out = torch.empty_like(q)
    stream = torch.cuda.Stream()
    log(f"[attend] graph replay, q_lens {mc.q_lens.tolist()}")
    with torch.cuda.stream(stream):
        call = pa.prepare_attend(q, g.k_cache, g.v_cache, g.bt, g.ctx, qs, mc.max_q_len, case.scale, out,
                                 num_workers=300)
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
        call()  # eager work on the same workspace between replays
        torch.cuda.synchronize()
    assert max_abs_err(eager, _oracle(mc)) <= TOL[case.dtype]
