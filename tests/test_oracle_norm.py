"""Pins of the oracle's RMSNorm (CPU only).

Facts that do not come from the oracle's own code: the mean square of the
output, a constant row, one-hot weights, scale invariance, permutation
equivariance, 50-digit decimal arithmetic on a short row, and torch's
float32 addition for the residual form.  A dropped 1/H, eps outside the
square root, a weight on the wrong dimension, or a residual normalised before
rounding fails one of them.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle

DT = [torch.float32, torch.float16, torch.bfloat16]


def _x(T, H, dtype, seed, spread=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(T, H, generator=g) * spread).to(dtype)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.3])
def test_mean_square_of_the_output(dtype, eps):
    # With unit weights, mean_d y_d^2 = ms / (ms + eps).
    x = _x(5, 256, dtype, 1)
    y = oracle.rmsnorm(x, torch.ones(256, dtype=dtype), eps)
    ms = np.mean(x.double().numpy() ** 2, axis=1)
    e = float(np.float32(eps))
    assert np.allclose(np.mean(y ** 2, axis=1), ms / (ms + e), rtol=1e-13, atol=0)


@pytest.mark.parametrize("dtype", DT)
def test_constant_row(dtype):
    # x = 1 everywhere, eps = 3: y = w / sqrt(1 + 3) = w / 2, exactly.
    H = 96
    w = _x(1, H, dtype, 2)[0]
    y = oracle.rmsnorm(torch.ones(2, H, dtype=dtype), w, 3.0)
    assert np.array_equal(y, np.broadcast_to(w.double().numpy() / 2, (2, H)))


def test_one_hot_weight_picks_one_dimension():
    H, d0 = 128, 37
    x = _x(3, H, torch.float32, 3)
    w = torch.zeros(H)
    w[d0] = 2.0
    y = oracle.rmsnorm(x, w, 1e-6)
    xd = x.double().numpy()
    rms = np.sqrt(np.mean(xd ** 2, axis=1) + float(np.float32(1e-6)))
    assert np.all(y[:, np.arange(H) != d0] == 0)
    assert np.allclose(y[:, d0], 2 * xd[:, d0] / rms, rtol=1e-14, atol=0)


def test_scale_invariance_without_eps():
    x = _x(4, 200, torch.float32, 4)
    w = _x(1, 200, torch.float32, 5)[0]
    assert np.allclose(oracle.rmsnorm(x * 8, w, 0.0), oracle.rmsnorm(x, w, 0.0), rtol=1e-14, atol=0)


def test_permutation_equivariance():
    x = _x(2, 64, torch.bfloat16, 6)
    w = _x(1, 64, torch.bfloat16, 7)[0]
    perm = torch.randperm(64, generator=torch.Generator().manual_seed(8))
    y = oracle.rmsnorm(x, w, 1e-5)
    yp = oracle.rmsnorm(x[:, perm].contiguous(), w[perm].contiguous(), 1e-5)
    assert np.allclose(yp, y[:, perm.numpy()], rtol=1e-14, atol=0)


def test_decimal_brute_force():
    getcontext().prec = 50
    x = _x(1, 12, torch.float32, 9, spread=3.0)
    w = _x(1, 12, torch.float32, 10)[0]
    eps = float(np.float32(1e-5))
    y = oracle.rmsnorm(x, w, 1e-5)[0]
    xs = [Decimal(float(v)) for v in x[0]]
    ms = sum(v * v for v in xs) / Decimal(12)
    r = Decimal(1) / (ms + Decimal(eps)).sqrt()
    ref = [float(xs[d] * Decimal(float(w[d])) * r) for d in range(12)]
    assert np.allclose(y, ref, rtol=1e-15, atol=0)


@pytest.mark.parametrize("dtype", DT)
def test_residual_is_the_rounded_sum_and_is_what_gets_normalised(dtype):
    x = _x(6, 512, dtype, 11, spread=4.0)
    r = _x(6, 512, dtype, 12, spread=0.01)  # wide exponent gaps between the two addends
    w = _x(1, 512, dtype, 13)[0]
    y, res = oracle.rmsnorm(x, w, 1e-5, residual=r)
    ref = (x.float() + r.float()).to(dtype)
    assert np.array_equal(res, ref.double().numpy())
    assert np.array_equal(y, oracle.rmsnorm(ref, w, 1e-5))
