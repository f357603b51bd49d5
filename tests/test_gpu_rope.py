"""GPU checks of the rotary embedding: pa_rope against the oracle's float64
rotation (within one unit in the last place of the dtype), and the fused
pa_decode_rope_append against pa_rope + pa_decode_append (bitwise) and the
oracle (within the attention tolerance)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_slot_amd as pa
from paged_kv_decode_slot_amd import workloads as W
from tests.gpu_helpers import TOL, GpuCase, dev_bits, log, max_abs_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MANT = {torch.float32: 23, torch.float16: 10, torch.bfloat16: 7}
EMIN = {torch.float32: -126, torch.float16: -14, torch.bfloat16: -126}


def _ulp(x: np.ndarray, dtype) -> np.ndarray:
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-300)))
    return np.exp2(np.maximum(e, EMIN[dtype]) - MANT[dtype])


def _check_rotated(gpu: torch.Tensor, src: torch.Tensor, pos: np.ndarray, theta: float):
    ref = oracle.rope(src, pos, theta)
    got = gpu.double().cpu().numpy()
    D = ref.shape[-1]
    x = src.double().numpy()
    pair = np.sqrt(x[..., :D // 2] ** 2 + x[..., D // 2:] ** 2)
    pair = np.concatenate([pair, pair], axis=-1)
    # one unit in the last place of the stored value, plus the float arithmetic
    tol = _ulp(ref, gpu.dtype) + 4e-7 * pair
    assert np.all(np.abs(got - ref) <= tol), float(np.max(np.abs(got - ref) - tol))


@pytest.mark.parametrize("dtype,D,theta", [(torch.bfloat16, 128, 500000.0), (torch.float16, 64, 10000.0),
                                           (torch.float32, 128, 10000.0)])
def test_rope_matches_oracle(dtype, D, theta):
    rng = np.random.default_rng(11)
    T, Hq, Hkv = 9, 8, 2
    q = W._normal(rng, (T, Hq, D), {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[dtype])
    k = W._normal(rng, (T, Hkv, D), {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[dtype])
    pos = np.array([0, 1, 2, 15, 16, 1000, 4095, 65535, 131071], dtype=np.int32)
    qg, kg = q.to(DEV), k.to(DEV)
    log(f"[rope] {dtype} D={D} theta={theta}")
    pa.rope(qg, kg, torch.from_numpy(pos).to(DEV), theta)
    torch.cuda.synchronize()
    _check_rotated(qg, q, pos, theta)
    _check_rotated(kg, k, pos, theta)


def _rope_two_calls(case: W.Case, theta: float, workers: int):
    """pa_rope on copies of q and k_new (at ctx - 1), then pa_decode_append."""
    g = GpuCase(case)
    q, kn = g.q.clone(), g.k_new.clone()
    pos = torch.clamp(g.ctx - 1, min=0).to(torch.int32)
    pa.rope(q, kn, pos, theta)
    out = pa.decode_append(q, kn, g.v_new, g.k_cache, g.v_cache, g.bt, g.ctx, case.scale, num_workers=workers)
    return g, out


def _rope_fused(case: W.Case, theta: float, workers: int):
    g = GpuCase(case)
    q0, kn0 = g.q.clone(), g.k_new.clone()
    out = pa.decode_rope_append(g.q, g.k_new, g.v_new, g.k_cache, g.v_cache, g.bt, g.ctx, case.scale, theta,
                                num_workers=workers)
    torch.cuda.synchronize()
    assert torch.equal(dev_bits(g.q), dev_bits(q0)) and torch.equal(dev_bits(g.k_new), dev_bits(kn0))
    return g, out


@pytest.mark.parametrize("workers", [0, -1, 37])
@pytest.mark.parametrize("n", [2, 3, 4])
def test_fused_rope_matches_rope_then_decode_append(n, workers):
    case = W.config_case(n)
    theta = 500000.0
    log(f"[rope] fused vs two calls, workload {n}, workers {workers}")
    g2, out2 = _rope_two_calls(case, theta, workers)
    g1, out1 = _rope_fused(case, theta, workers)
    torch.cuda.synchronize()
    assert torch.equal(dev_bits(out1), dev_bits(out2))
    assert torch.equal(dev_bits(g1.k_cache), dev_bits(g2.k_cache))
    assert torch.equal(dev_bits(g1.v_cache), dev_bits(g2.v_cache))


@pytest.mark.parametrize("n,theta", [(2, 10000.0), (3, 500000.0), (5, 500000.0)])
def test_fused_rope_matches_oracle(n, theta):
    case = W.config_case(n)
    log(f"[rope] fused vs oracle, workload {n}")
    g, out = _rope_fused(case, theta, 0)
    rc = oracle.rope_case(case, theta)
    kp, vp = oracle.build_pools(rc)
    ref = oracle.decode(rc.q, kp, vp, rc.block_tables, rc.context_lens, rc.scale, Hkv=rc.Hkv, B=rc.B)
    assert max_abs_err(out, ref) <= TOL[case.dtype]
    # V pools bitwise; K pools bitwise except the rotated new rows, which are within one unit in the last place
    assert torch.equal(dev_bits(g.v_cache).cpu(), vp.contiguous().view(-1).view(torch.int16))
    gk = g.k_cache.cpu().contiguous().view(-1)
    ok = kp.contiguous().view(-1)
    diff = torch.nonzero(gk.view(torch.int16) != ok.view(torch.int16)).view(-1)
    assert diff.numel() <= case.S * case.Hkv * case.D
    if diff.numel():
        a, b = gk[diff].double().numpy(), ok[diff].double().numpy()
        assert np.all(np.abs(a - b) <= _ulp(b, case.k_new.dtype) * 1.0001)


def test_fused_rope_small_shapes():
    for idx, kw in enumerate([dict(S=5, Hq=8, Hkv=2, D=128, B=16, dtype="bf16", ctx_range=(1, 300)),
                              dict(S=3, Hq=16, Hkv=1, D=64, B=32, dtype="f16", ctx_range=(1, 200)),
                              dict(S=8, Hq=6, Hkv=2, D=128, B=32, dtype="bf16", ctx=[0, 1, 15, 16, 17, 32, 33, 0],
                                   max_blocks_per_seq=4)]):
        case = W.make_case(seed=700 + idx, name=f"rope{idx}", **kw)
        for workers in (0, -1, 3):
            log(f"[rope] small shape {idx}, workers {workers}")
            g2, out2 = _rope_two_calls(case, 10000.0, workers)
            g1, out1 = _rope_fused(case, 10000.0, workers)
            assert torch.equal(dev_bits(out1), dev_bits(out2))
            assert torch.equal(dev_bits(g1.k_cache), dev_bits(g2.k_cache))
