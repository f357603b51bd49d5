#!/usr/bin/env python3
"""Decode-step benchmark on one MI355X.

A step is one pass of the whole path over one batch: the KV append of one new
token per sequence and paged decode attention, as one pa_decode_append launch.
The default workload is the Llama-3-8B-shaped layer: 64 sequences, 32 query /
8 kv heads, head_dim 128, block 16, bf16, context lengths uniform on
[512, 4096], shuffled blocks (seed 3).

Steps rotate over several "layers", each with its own K/V pools, so that the
bytes a step reads are not left in the 256 MB last-level cache by the step
before (as in a real model, where every layer has its own cache).  Inputs are
resident in HBM before timing starts.  The timed region is K steps launched
back to back on one stream between two HIP events, synchronized on both
sides; per-launch event pairs (which add each launch's overhead) give the
percentiles, and the same step as two calls (pa_write_kv, pa_decode_ex) is
timed beside it.

Prints one JSON line.  `value` is the algorithmic bytes of a step (K/V rows
of the cached positions, the new token's rows read and stored, q read, out
written, block-table entries and lengths) divided by the step time.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved HBM GB/s (% of peak) and μs per layer-step"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD's published figure
# Dense matrix-core peaks of MI355X (AMD's published figures, without sparsity), TFLOP/s.
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def setup_layers(case, layers, device, num_workers):
    """Per layer: (append call, decode call, fused step call) on that layer's own pools."""
    import torch

    import paged_kv_decode_slot_amd as pa
    from paged_kv_decode_slot_amd import workloads as W

    dt = W.DTYPES[case.dtype]
    q = case.q.to(device)
    bt = torch.from_numpy(case.block_tables).to(device)
    ctx = torch.from_numpy(case.context_lens).to(device)
    k_new, v_new = case.k_new.to(device), case.v_new.to(device)
    slot_new = torch.from_numpy(case.slot_new).to(device)
    ints = torch.int32 if case.elt == 4 else torch.int16
    k0, v0 = pa.new_cache(case.num_blocks, case.B, case.Hkv, case.D, dt, device)
    k0.view(ints).fill_(W.NAN_BITS[case.dtype])
    v0.view(ints).fill_(W.NAN_BITS[case.dtype])
    if case.k_prefill.shape[0]:
        pa.write_kv(case.k_prefill.to(device), case.v_prefill.to(device),
                    torch.from_numpy(case.slot_prefill).to(device), k0, v0)
    steps, pools = [], []
    for i in range(layers):
        kc, vc = (k0, v0) if i == 0 else (k0.clone(), v0.clone())
        out = torch.empty_like(q)
        steps.append((pa.prepare_write_kv(k_new, v_new, slot_new, kc, vc),
                      pa.prepare_decode(q, kc, vc, bt, ctx, case.scale, out, num_workers=num_workers),
                      pa.prepare_decode_append(q, k_new, v_new, kc, vc, bt, ctx, case.scale, out,
                                               num_workers=num_workers)))
        pools.append((kc, vc))
    torch.cuda.synchronize()
    return steps, pools


def _events(n):
    import torch

    return [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]


def time_back_to_back(calls, n_steps, warmup):
    """n_steps launches of calls[i % len(calls)] back to back between two events on the
    launch stream, synchronized on both sides; returns the total in ms."""
    import torch

    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(n_steps):
        calls[i % len(calls)]()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


def time_each(calls, n_steps, warmup):
    """Per-launch event pairs around each call of calls[i % len(calls)] (a list of
    callables run in order per step); returns per-step lists of us, one per callable."""
    import torch

    for i in range(warmup):
        for c in calls[i % len(calls)]:
            c()
    torch.cuda.synchronize()
    k = len(calls[0])
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(k + 1)] for _ in range(n_steps)]
    for i in range(n_steps):
        for j, c in enumerate(calls[i % len(calls)]):
            ev[i][j].record()
            c()
        ev[i][k].record()
    torch.cuda.synchronize()
    return [[ev[i][j].elapsed_time(ev[i][j + 1]) * 1e3 for i in range(n_steps)] for j in range(k)]


def pct(xs, p):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(p / 100 * (len(xs) - 1)))))]


def measure(n, args, device):
    from paged_kv_decode_slot_amd import workloads as W

    t = time.perf_counter()
    case = W.config_case(n)
    log(f"[bench] workload {n}: inputs drawn in {time.perf_counter() - t:.1f}s")
    layer_bytes = 2 * case.pool_numel * case.elt
    layers = args.layers or max(2, math.ceil(2 * 2**30 / layer_bytes))
    steps, _pools = setup_layers(case, layers, device, args.workers)
    K, Wm = args.steps, args.warmup
    log(f"[bench] workload {n}: {layers} layers of {layer_bytes / 1e9:.2f} GB; timing {K} steps")
    # The timed region: K fused steps back to back (the headline).
    fused_ms = time_back_to_back([s[2] for s in steps], K, Wm)
    # Beside it: the decode alone and the two-call step, back to back, and
    # per-launch event pairs for percentiles (these include each launch's overhead).
    decode_ms = time_back_to_back([s[1] for s in steps], K, Wm)
    pairs = [(lambda w=w, d=d: (w(), d())) for (w, d, _) in steps]
    two_ms = time_back_to_back(pairs, K, Wm)
    # Hot cache: one layer's pools over and over (whatever of them the 256 MB MALL keeps).
    hot_ms = time_back_to_back([steps[0][2]], K, Wm)
    (t_step,) = time_each([[s[2]] for s in steps], K, Wm)
    t_write, t_decode = time_each([[s[0], s[1]] for s in steps], K, Wm)
    dec_b, wr_b, st_b = W.decode_bytes(case), W.write_bytes(case), W.step_bytes(case)
    step_us = fused_ms * 1e3 / K
    dec_us = decode_ms * 1e3 / K
    return dict(
        case=case,
        layers=layers,
        decode_bytes=dec_b,
        write_bytes=wr_b,
        step_bytes=st_b,
        # the fused step, pa_decode_append, back to back
        ms_per_step=fused_ms / K,
        step_us_mean=step_us,
        step_gbs=st_b / (step_us * 1e-6) / 1e9,
        seq_heads_per_s=case.S * case.Hq / (step_us * 1e-6),
        step_us_events=dict(mean=statistics.fmean(t_step), p10=pct(t_step, 10), p50=pct(t_step, 50),
                            p90=pct(t_step, 90)),
        # pa_decode_ex alone, and pa_write_kv + pa_decode_ex, back to back
        decode_us_mean=dec_us,
        decode_gbs=dec_b / (dec_us * 1e-6) / 1e9,
        two_call_ms_per_step=two_ms / K,
        t_decode_us_events=dict(mean=statistics.fmean(t_decode), p10=pct(t_decode, 10), p50=pct(t_decode, 50),
                                p90=pct(t_decode, 90)),
        t_write_us_events=dict(mean=statistics.fmean(t_write), p50=pct(t_write, 50)),
        hot_step_us=hot_ms * 1e3 / K,
    )


def measure_attend(n, q_len, args, device):
    """pa_attend with q_len query tokens per sequence (e.g. draft tokens being
    verified) over workload n's pools, K steps back to back."""
    import torch

    import paged_kv_decode_slot_amd as pa
    from paged_kv_decode_slot_amd import workloads as W

    case = W.config_case(n)
    mc = W.with_queries(case, [q_len] * case.S, seed=1000 + n)
    layer_bytes = 2 * case.pool_numel * case.elt
    layers = args.layers or max(2, math.ceil(2 * 2**30 / layer_bytes))
    steps, pools = setup_layers(case, layers, device, args.workers)
    for (w, _d, _f) in steps:  # every position, the query tokens' own included, is in the cache
        w()
    q = mc.q.to(device)
    qs = torch.from_numpy(mc.query_start).to(device)
    bt = torch.from_numpy(case.block_tables).to(device)
    ctx = torch.from_numpy(case.context_lens).to(device)
    out = torch.empty_like(q)
    calls = [pa.prepare_attend(q, kc, vc, bt, ctx, qs, mc.max_q_len, case.scale, out, num_workers=args.workers)
             for (kc, vc) in pools]
    ms = time_back_to_back(calls, args.steps, args.warmup)
    us = ms * 1e3 / args.steps
    b = W.attend_bytes(mc)
    return dict(workload=W.CONFIGS[n]["name"], query_tokens_per_seq=q_len, us=round(us, 2),
                bytes=b, gbs=round(b / (us * 1e-6) / 1e9, 1), frac_of_peak=round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                query_rows_per_s=round(int(mc.query_start[-1]) * case.Hq / (us * 1e-6)),
                traffic=measured_traffic(n, f"attend{q_len}"))


def chunk_q_lens(case):
    """The mixed batch of the chunk leg: every 8th sequence carries a prompt chunk
    (64 to 512 tokens), the others one decode token each."""
    import numpy as np

    q_lens = np.ones(case.S, dtype=np.int64)
    q_lens[::8] = [64, 96, 128, 200, 256, 300, 400, 512][:len(q_lens[::8])]
    return q_lens


def measure_chunks(n, args, device):
    """pa_attend on workload n's pools with a mixed batch: prompt chunks of 64 to 512
    tokens beside decode tokens, K calls back to back.  Reports query rows/s, the
    chunk kernel's matrix-core rate (causal FLOPs of the chunk tokens) and the
    bytes the call must read."""
    import numpy as np
    import torch

    import paged_kv_decode_slot_amd as pa
    from paged_kv_decode_slot_amd import workloads as W

    case = W.config_case(n)
    mc = W.with_queries(case, chunk_q_lens(case), seed=2000 + n)
    layer_bytes = 2 * case.pool_numel * case.elt
    layers = args.layers or max(2, math.ceil(2 * 2**30 / layer_bytes))
    steps, pools = setup_layers(case, layers, device, args.workers)
    for (w, _d, _f) in steps:
        w()
    q = mc.q.to(device)
    qs = torch.from_numpy(mc.query_start).to(device)
    bt = torch.from_numpy(case.block_tables).to(device)
    ctx = torch.from_numpy(case.context_lens).to(device)
    out = torch.empty_like(q)
    calls = [pa.prepare_attend(q, kc, vc, bt, ctx, qs, mc.max_q_len, case.scale, out, num_workers=args.workers)
             for (kc, vc) in pools]
    ms = time_back_to_back(calls, args.steps, args.warmup)
    us = ms * 1e3 / args.steps
    ql = mc.q_lens.astype(np.int64)
    L = case.context_lens.astype(np.int64)
    chunk = ql > 1
    # causal FLOPs: token i of a sequence sees L - n + i + 1 positions; 4 flops per (position, head, dim)
    seen = sum(int(((L[s] - ql[s]) * ql[s] + ql[s] * (ql[s] + 1) // 2)) for s in np.nonzero(chunk)[0])
    flops = 4 * seen * case.Hq * case.D
    b = W.attend_bytes(mc)
    rows = int(mc.query_start[-1])
    tflops = flops / (us * 1e-6) / 1e12
    c = measured_counters(n, "chunks")
    return dict(workload=W.CONFIGS[n]["name"], query_lens=f"{int(chunk.sum())} prompt chunks {ql[chunk].tolist()}, "
                f"{int((~chunk).sum())} decode tokens", us=round(us, 2), query_rows=rows,
                query_rows_per_s=round(rows / (us * 1e-6)), chunk_tflops=round(tflops, 1),
                chunk_frac_of_mfma_peak=round(tflops / MFMA_PEAK_TFLOPS[case.dtype], 4),
                bytes=b, gbs=round(b / (us * 1e-6) / 1e9, 1),
                chunk_kernel_traffic=None if c is None else c["total"],
                chunk_kernel_l2_hit_rate=None if c is None else c["l2_hit_rate"],
                note="one pa_attend call: chunk_kernel for the chunks, the split path for the decode tokens; "
                     "chunk_tflops counts only the chunks' causal FLOPs over the whole call's time, against the "
                     "dense matrix-core peak of the dtype; chunk_kernel_traffic: counter bytes of the chunk "
                     "kernel's launch alone")


def measure_rope(n, theta, args, device):
    """The decode step with the rotary embedding of q and the new K rows fused
    in (pa_decode_rope_append), beside pa_rope + pa_decode_append, K steps back
    to back each."""
    import torch

    import paged_kv_decode_slot_amd as pa
    from paged_kv_decode_slot_amd import workloads as W

    case = W.config_case(n)
    layer_bytes = 2 * case.pool_numel * case.elt
    layers = args.layers or max(2, math.ceil(2 * 2**30 / layer_bytes))
    _steps, pools = setup_layers(case, layers, device, args.workers)
    q = case.q.to(device)
    kn, vn = case.k_new.to(device), case.v_new.to(device)
    bt = torch.from_numpy(case.block_tables).to(device)
    ctx = torch.from_numpy(case.context_lens).to(device)
    pos = torch.clamp(ctx - 1, min=0).to(torch.int32)
    out = torch.empty_like(q)
    fused = [pa.prepare_decode_rope_append(q, kn, vn, kc, vc, bt, ctx, case.scale, theta, out,
                                           num_workers=args.workers) for (kc, vc) in pools]
    q2, kn2 = q.clone(), kn.clone()
    appends = [pa.prepare_decode_append(q2, kn2, vn, kc, vc, bt, ctx, case.scale, out, num_workers=args.workers)
               for (kc, vc) in pools]

    def two(i):
        q2.copy_(q)  # pa_rope works in place
        kn2.copy_(kn)
        pa.rope(q2, kn2, pos, theta)
        appends[i]()

    fused_ms = time_back_to_back(fused, args.steps, args.warmup)
    two_ms = time_back_to_back([(lambda i=i: two(i)) for i in range(len(pools))], args.steps, args.warmup)
    b = W.step_bytes(case)
    us = fused_ms * 1e3 / args.steps
    return dict(workload=W.CONFIGS[n]["name"], rope_theta=theta, us=round(us, 2),
                gbs=round(b / (us * 1e-6) / 1e9, 1), frac_of_peak=round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                traffic=measured_traffic(n, "rope"),
                two_calls_us=round(two_ms * 1e3 / args.steps, 2),
                two_calls_note="copies of q and k_new (pa_rope works in place), pa_rope, pa_decode_append")


def measure_pool(n, args, device):
    """The block pool on workload n: the whole batch admitted by one
    pa_assign_slots call (its context lengths as the prompts), timed over fresh
    pools; then K decode steps, every sequence growing by one token per step on
    the pool as the earlier steps left it, back to back."""
    import numpy as np
    import torch

    import paged_kv_decode_slot_amd as pa
    from paged_kv_decode_slot_amd import workloads as W

    case = W.config_case(n)
    S, B = case.S, case.B
    K, warm = args.steps, args.warmup
    grow = -(-(K + warm) // B) + 1
    M = case.block_tables.shape[1] + grow
    cap = case.num_blocks + S * grow
    i32 = dict(dtype=torch.int32, device=device)
    free = torch.empty(cap, **i32)
    state = torch.empty(8, **i32)
    bt = torch.empty((S, M), **i32)
    L0 = case.context_lens.astype(np.int32)
    qs0 = np.concatenate([[0], np.cumsum(L0)]).astype(np.int32)
    T0 = int(qs0[-1])
    ctx0, qs0_d = torch.from_numpy(L0).to(device), torch.from_numpy(qs0).to(device)
    slots0 = torch.empty(T0, dtype=torch.int64, device=device)
    admit = pa.prepare_assign_slots(ctx0, qs0_d, bt, free, state, slots0, B)

    def reset():
        bt.fill_(-1)
        pa.pool_init(free, state, cap)
    reps = 20
    admit_us = time_each([[reset, admit]], reps, 3)[1]
    reset()
    admit()
    lens = [torch.from_numpy((L0 + k + 1).astype(np.int32)).to(device) for k in range(warm + K)]
    slots = torch.empty(S, dtype=torch.int64, device=device)
    steps = [pa.prepare_assign_slots(lens[k], None, bt, free, state, slots, B) for k in range(warm + K)]
    for k in range(warm):
        steps[k]()
    torch.cuda.synchronize()
    ms = time_back_to_back(steps[warm:], K, 0)
    st = state.cpu().numpy()
    assert st[1] == 0, "the pool refused a sequence"
    a_mean = float(np.mean(admit_us))
    return dict(workload=W.CONFIGS[n]["name"], admit_tokens=T0, admit_us_mean=round(a_mean, 2), admit_us_p50=round(pct(admit_us, 50), 2),
                admit_slots_per_s=round(T0 / (a_mean * 1e-6)),
                decode_step_us=round(ms * 1e3 / K, 2), decode_steps=K, seqs=S,
                pool_blocks=cap, blocks_used_after=int(cap - st[0]),
                note="launch-bound: the decode step reads lengths and writes one int64 slot per sequence")


def measure_norm(args, device):
    """pa_rmsnorm on Llama-3-8B rows (hidden 4096, bf16, eps 1e-5): a prefill
    chunk of 16384 rows (HBM-bound; buffers rotated so the 256 MB MALL holds
    none of a step's inputs) plain and fused with the residual add, and a
    decode batch of 64 rows, K launches back to back each."""
    import torch

    import paged_kv_decode_slot_amd as pa

    H, dt = 4096, torch.bfloat16
    g = torch.Generator(device=device).manual_seed(0)
    w = torch.randn(H, device=device, generator=g).to(dt)
    res = {}
    for rows in (16384, 64):
        sets = 4 if rows > 1024 else 1
        xs = [torch.randn((rows, H), device=device, generator=g).to(dt) for _ in range(sets)]
        rs = [torch.randn((rows, H), device=device, generator=g).to(dt) for _ in range(sets)]
        outs = [torch.empty_like(xs[0]) for _ in range(sets)]
        plain = [pa.prepare_rmsnorm(xs[i], w, 1e-5, outs[i]) for i in range(sets)]
        fused = [pa.prepare_rmsnorm(xs[i], w, 1e-5, outs[i], residual=rs[i]) for i in range(sets)]
        row_bytes = H * 2
        for name, calls, nbytes in (("plain", plain, 2 * rows * row_bytes + row_bytes),
                                    ("fused_residual", fused, 4 * rows * row_bytes + row_bytes)):
            ms = time_back_to_back(calls, args.steps, args.warmup)
            us = ms * 1e3 / args.steps
            res[f"{name}_{rows}"] = dict(us=round(us, 2), bytes=nbytes, gbs=round(nbytes / (us * 1e-6) / 1e9, 1),
                                         frac_of_peak=round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4))
        del xs, rs, outs
    return dict(workload="RMSNorm, Llama-3-8B rows: hidden 4096, bf16, eps 1e-5; 16384 rows (prefill chunk), 64 rows (decode batch)",
                **res)


# Measured HBM traffic of the decode kernel (two rocprofv3 counter passes, scaled by a
# plain copy of known size), kept with the hash of the source it was measured on.
TRAFFIC_FILES = {(3, "fused"): "profiles/decode_append_kernel_C3_llama3-8b_bf16_counters.txt",
                 (3, "decode"): "profiles/decode_kernel_C3_llama3-8b_bf16_counters.txt",
                 (3, "attend4"): "profiles/attend_kernel_C3_llama3-8b_4tokens_bf16_counters.txt",
                 (3, "rope"): "profiles/decode_rope_append_kernel_C3_llama3-8b_bf16_counters.txt",
                 (4, "fused"): "profiles/decode_append_kernel_C4_ragged_bf16_counters.txt",
                 (5, "fused"): "profiles/decode_append_kernel_C5_long_bf16_counters.txt",
                 (3, "chunks"): "profiles/chunk_kernel_C3_prompt_chunks_bf16_counters.txt"}
KERNEL_SOURCE = "paged_kv_decode_slot_amd/csrc/pagedattn.hip"


def measured_counters(config: int, kind: str):
    """{"fetch", "write", "total"} bytes per launch and the L2 hit rate (None when not
    taken) from a counter summary, or None if there is none or the kernel source
    changed since it was taken."""
    import hashlib

    path = TRAFFIC_FILES.get((config, kind))
    if path is None or not os.path.exists(os.path.join(ROOT, path)):
        return None
    fields = {}
    for line in open(os.path.join(ROOT, path)):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    src = hashlib.sha256(open(os.path.join(ROOT, KERNEL_SOURCE), "rb").read()).hexdigest()
    if fields.get("source_sha256") != src or "traffic_bytes_per_launch" not in fields:
        return None
    fetch, write = [int(x.split()[-1]) for x in fields["scaled bytes per launch"].split(",")]
    hit = float(fields["l2_hit_rate"]) if "l2_hit_rate" in fields else None
    return dict(fetch=fetch, write=write, total=int(fields["traffic_bytes_per_launch"]), l2_hit_rate=hit)


def l2_hit_rate(config: int, kind: str):
    c = measured_counters(config, kind)
    return None if c is None else c["l2_hit_rate"]


def measured_traffic(config: int, kind: str):
    """Counter bytes (read + written) per launch, or None."""
    c = measured_counters(config, kind)
    return None if c is None else c["total"]


def kv_share(case, config: int, kind: str):
    """Algorithmic K/V bytes read over the counter-measured bytes fetched (1.0: no K/V
    byte fetched twice and nothing else fetched), or None without counters."""
    from paged_kv_decode_slot_amd import workloads as W

    c = measured_counters(config, kind)
    return None if c is None else round(W.kv_read_bytes(case) / c["fetch"], 4)


def measure_ceilings(device, args):
    """Read-bandwidth ceilings on this GPU, measured with pa_read_probe over a 4 GiB
    buffer (16 times the MALL): every byte in address order, and whole 4 KB tiles
    in a shuffled order (how the decode reads a paged pool).  Context for the
    decode's fraction of peak, not a target."""
    import torch

    import paged_kv_decode_slot_amd as pa

    nbytes = 4 << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=device)
    buf.fill_(0x01020304)
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    g = torch.Generator(device="cpu").manual_seed(0)
    res = {}
    reps = max(5, args.steps // 10)
    for name, tile, order in (("stream_read", 4096, None), ("random_4k_tiles", 4096, "perm")):
        ids = None
        if order == "perm":
            ids = torch.randperm(nbytes // tile, generator=g).to(torch.int32).to(device)
        # The best of a few launch widths (wavefronts per compute unit): the ceiling.
        by_width = {}
        for per_cu in (2, 4, 8, 16, 32):
            call, _sink = pa.prepare_read_probe(buf, tile, ids, num_waves=per_cu * cus)
            us = time_back_to_back([call], reps, 2) * 1e3 / reps
            by_width[per_cu] = round(nbytes / (us * 1e-6) / 1e9, 1)
        best = max(by_width, key=by_width.get)
        res[name] = dict(gbs=by_width[best], frac_of_peak=round(by_width[best] / PEAK_HBM_GBS, 4),
                         waves_per_cu=best, gbs_by_waves_per_cu=by_width)
        del ids
    del buf
    res["note"] = ("pa_read_probe over 4 GiB, 16-byte non-temporal loads, 4 tiles of 4 KB in flight per "
                   "wavefront, the best of 2..32 wavefronts per CU; tile ids read from memory in the shuffled case")
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(case, min_seconds):
    import oracle
    from paged_kv_decode_slot_amd import workloads as W

    kp, vp = case.nan_pool(), case.nan_pool()
    oracle.write_kv(case.k_prefill, case.v_prefill, case.slot_prefill, kp, vp, num_blocks=case.num_blocks, B=case.B)
    threads = oracle.default_threads()
    reps, t_total = 0, 0.0
    while t_total < min_seconds or reps == 0:
        t = time.perf_counter()
        oracle.write_kv(case.k_new, case.v_new, case.slot_new, kp, vp, num_blocks=case.num_blocks, B=case.B)
        oracle.decode(case.q, kp, vp, case.block_tables, case.context_lens, case.scale, Hkv=case.Hkv, B=case.B,
                      threads=threads)
        t_total += time.perf_counter() - t
        reps += 1
    per_step = t_total / reps
    gbs = W.step_bytes(case) / per_step / 1e9
    return dict(value=round(gbs, 4), unit="GB/s", cores=threads, kind="oracle", cpu_model=cpu_model(),
                sample=f"the whole workload (append + decode of all {case.S} sequences), {reps} reps, "
                       f"{per_step * 1e3:.1f} ms per step, float64 C oracle")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, help="workload 1-5 (default 3)")
    ap.add_argument("--also", default="1,2,4,5", help="comma list of extra workloads reported under 'other'")
    ap.add_argument("--layers", type=int, default=0, help="distinct K/V pools to rotate over (0: enough for 2 GiB)")
    ap.add_argument("--workers", type=int, default=0, help="decode work split (0 automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--attend-q", type=int, default=4,
                    help="also time pa_attend with this many query tokens per sequence (0: skip)")
    ap.add_argument("--rope-theta", type=float, default=500000.0,
                    help="also time the step with the rotary embedding fused in, at this base (0: skip)")
    ap.add_argument("--no-pool", action="store_true", help="skip the block-pool leg")
    ap.add_argument("--no-chunks", action="store_true", help="skip the prompt-chunk leg")
    ap.add_argument("--no-norm", action="store_true", help="skip the RMSNorm leg")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the read-bandwidth ceilings")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size kernel for counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this path runs on one GPU (asked for {max(args.gpus, world)}); "
              "runs across several GPUs are not implemented.", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_decode_slot_amd as pa
    from paged_kv_decode_slot_amd import workloads as W

    pa.lib()  # fail loudly before any setup if the library is missing
    device = torch.device("cuda:0")
    if args.calib_copy_mb:
        n = args.calib_copy_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {n} bytes done")
        del src, dst
    main_res = measure(args.config, args, device)
    case = main_res.pop("case")

    other = {}
    for n in [int(x) for x in args.also.split(",") if x.strip()]:
        if n == args.config:
            continue
        r = measure(n, args, device)
        c = r.pop("case")
        other[f"C{n}"] = dict(
            workload=W.CONFIGS[n]["name"],
            step_us=round(r["step_us_mean"], 2), step_gbs=round(r["step_gbs"], 1),
            step_frac_of_peak=round(r["step_gbs"] / PEAK_HBM_GBS, 4),
            decode_us=round(r["decode_us_mean"], 2), decode_gbs=round(r["decode_gbs"], 1),
            decode_frac_of_peak=round(r["decode_gbs"] / PEAK_HBM_GBS, 4),
            two_call_us=round(r["two_call_ms_per_step"] * 1e3, 2),
            hot_step_us=round(r["hot_step_us"], 2),
            seq_heads_per_s=round(r["seq_heads_per_s"]), layers=r["layers"],
            step_bytes=r["step_bytes"], decode_bytes=r["decode_bytes"], context_tokens=int(c.context_lens.sum()),
            traffic=measured_traffic(n, "fused"), kv_share=kv_share(c, n, "fused"))
        del c, r
        torch.cuda.empty_cache()

    attend = None
    if args.attend_q > 0:
        attend = measure_attend(args.config, args.attend_q, args, device)
        torch.cuda.empty_cache()

    chunks = None
    if not args.no_chunks:
        chunks = measure_chunks(args.config, args, device)
        torch.cuda.empty_cache()

    rope = None
    if args.rope_theta > 0:
        rope = measure_rope(args.config, args.rope_theta, args, device)
        torch.cuda.empty_cache()

    norm = None
    if not args.no_norm:
        norm = measure_norm(args, device)
        torch.cuda.empty_cache()

    ceilings = None
    if not args.no_ceilings:
        ceilings = measure_ceilings(device, args)
        torch.cuda.empty_cache()

    pool = None
    if not args.no_pool:
        pool = measure_pool(args.config, args, device)
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on the host")
        cpu = cpu_baseline(case, args.cpu_seconds)

    step_bytes = main_res["step_bytes"]
    r2 = lambda d: {k: round(v, 2) for k, v in d.items()}
    line = {
        "metric": METRIC,
        "value": round(main_res["step_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic (seeded; no model weights or datasets)",
        "config": {
            "workload": W.CONFIGS[args.config]["name"],
            "seqs": case.S, "q_heads": case.Hq, "kv_heads": case.Hkv, "head_dim": case.D,
            "block_size": case.B, "context_tokens": int(case.context_lens.sum()),
            "step": "pa_decode_append: KV append of one token per sequence + decode attention, one launch",
            "layers_rotated": main_res["layers"], "workers": args.workers,
        },
        "roofline": {
            "kernel": "decode_kernel with append (the single launch of pa_decode_append)",
            "bound": "hbm",
            "achieved": round(main_res["step_gbs"], 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(main_res["step_gbs"] / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(args.config, "fused"),
            "traffic_unit": "bytes per launch",
            "kv_share": kv_share(case, args.config, "fused"),
            "l2_hit_rate": l2_hit_rate(args.config, "fused"),
            "bytes_per_launch": step_bytes,
            "launch_us_mean": round(main_res["step_us_mean"], 2),
            "timing": "HIP events around the K back-to-back launches on the launch stream",
        },
        "cpu_baseline": cpu,
        "detail": {
            "seq_heads_per_s": round(main_res["seq_heads_per_s"]),
            "step_bytes": step_bytes,
            "hot_step_us": round(main_res["hot_step_us"], 2),
            "ceilings": ceilings,
            "step_us_per_launch_events": r2(main_res["step_us_events"]),
            "decode_alone": {
                "us": round(main_res["decode_us_mean"], 2),
                "gbs": round(main_res["decode_gbs"], 1),
                "frac_of_peak": round(main_res["decode_gbs"] / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(args.config, "decode"),
            },
            "two_calls": {
                "ms_per_step": round(main_res["two_call_ms_per_step"], 5),
                "t_write_us_per_launch_events": r2(main_res["t_write_us_events"]),
                "t_decode_us_per_launch_events": r2(main_res["t_decode_us_events"]),
            },
            "attend": attend,
            "chunks": chunks,
            "rope": rope,
            "pool": pool,
            "rmsnorm": norm,
            "other": other,
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
