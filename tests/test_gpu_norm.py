"""pa_rmsnorm on the GPU against the oracle (through the C ABI).

The oracle's y is exact to double precision; the kernel computes in float32
and rounds once, so a 16-bit output may differ from round(y) only where y is
within float32 error of a rounding midpoint: within one spacing of the dtype
at |y|.  float32 outputs are held to max-abs 1e-5.  The stored residual of
the fused form is compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_slot_amd as pa

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MANT = {torch.float16: (10, -14), torch.bfloat16: (7, -126)}


def _rand(shape, dtype, seed, spread=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * spread).to(dtype)


def _check(got: torch.Tensor, ref: np.ndarray):
    g = got.float().cpu().double().numpy()
    if got.dtype == torch.float32:
        err = np.max(np.abs(g - ref)) if ref.size else 0.0
        assert err <= 1e-5, err
        return
    m, emin = MANT[got.dtype]
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    spacing = np.exp2(np.maximum(e, emin) - m)
    bad = np.abs(g - ref) > spacing
    assert not bad.any(), (np.argwhere(bad)[:5], g[bad][:5], ref[bad][:5])


SHAPES = [
    (1, 4, torch.float32), (3, 64, torch.float32), (4, 4096, torch.float32),
    (1, 8, torch.bfloat16), (64, 4096, torch.bfloat16), (5, 5120, torch.bfloat16), (2, 3584, torch.bfloat16),
    (9, 8192, torch.bfloat16), (7, 2048, torch.float16), (3, 8192, torch.float16), (300, 512, torch.float16),
]


@pytest.mark.parametrize("T,H,dtype", SHAPES)
@pytest.mark.parametrize("fused", [False, True])
def test_rmsnorm_matches_oracle(T, H, dtype, fused):
    print(f"[norm] T={T} H={H} {dtype} residual={fused}", flush=True)
    x = _rand((T, H), dtype, 1, spread=2.0)
    w = _rand((H,), dtype, 2)
    r = _rand((T, H), dtype, 3, spread=0.5) if fused else None
    xd, wd = x.to(DEV), w.to(DEV)
    rd = r.to(DEV) if fused else None
    out = pa.rmsnorm(xd, wd, 1e-5, residual=rd)
    if fused:
        ref, res = oracle.rmsnorm(x, w, 1e-5, residual=r)
        assert np.array_equal(rd.float().cpu().double().numpy(), res)
    else:
        ref = oracle.rmsnorm(x, w, 1e-5)
    _check(out, ref)


def test_large_batch_sampled_rows():
    """16384 rows of 4096 (a prefill chunk of Llama-3-8B): the launch the
    benchmark times; every 97th row checked against the oracle."""
    print("[norm] 16384 x 4096 bf16", flush=True)
    T, H = 16384, 4096
    x = _rand((T, H), torch.bfloat16, 4)
    w = _rand((H,), torch.bfloat16, 5)
    out = pa.rmsnorm(x.to(DEV), w.to(DEV), 1e-5)
    rows = np.arange(0, T, 97)
    ref = oracle.rmsnorm(x[rows].contiguous(), w, 1e-5)
    _check(out[torch.from_numpy(rows).to(DEV)], ref)


def test_in_place_and_repeatable():
    print("[norm] in place", flush=True)
    x = _rand((33, 4096), torch.bfloat16, 6).to(DEV)
    w = _rand((4096,), torch.bfloat16, 7).to(DEV)
    a = pa.rmsnorm(x, w, 1e-6)
    b = pa.rmsnorm(x, w, 1e-6)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    y = x.clone()
    pa.rmsnorm(y, w, 1e-6, out=y)
    assert torch.equal(y.view(torch.int16), a.view(torch.int16))


def test_empty_and_rejected():
    x = torch.empty((0, 4096), dtype=torch.bfloat16, device=DEV)
    w = torch.ones(4096, dtype=torch.bfloat16, device=DEV)
    pa.rmsnorm(x, w, 1e-5)
    with pytest.raises(ValueError):
        pa.rmsnorm(torch.ones((2, 12), dtype=torch.bfloat16, device=DEV),
                   torch.ones(12, dtype=torch.bfloat16, device=DEV), 1e-5)  # 12 is not a multiple of 8
    with pytest.raises(ValueError):
        pa.rmsnorm(torch.ones((2, 16384), dtype=torch.bfloat16, device=DEV),
                   torch.ones(16384, dtype=torch.bfloat16, device=DEV), 1e-5)  # wider than 8192
