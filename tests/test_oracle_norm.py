"""Pins of the oracle's residual add + RMSNorm (O9).  Each checks what the
definition fixes independently of the oracle's code: the fp32 add against
numpy's IEEE single-precision addition, exact small cases, the eps term,
the weight, power-of-two scale invariance, the unit mean square, and the
exact result computed with 60-digit decimal arithmetic."""
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle


def test_residual_add_is_one_fp32_rounding():
    rng = np.random.default_rng(1)
    h = (rng.standard_normal(4096) * 10 ** rng.uniform(-8, 8, 4096)).astype(np.float32)
    r = (rng.standard_normal(4096) * 10 ** rng.uniform(-8, 8, 4096)).astype(np.float32)
    g = np.ones(4096, np.float32)
    h_out, _ = oracle.residual_rmsnorm(h, r, g, 1e-6)
    assert np.array_equal(h_out, h + r)  # numpy float32 + float32: IEEE single rounding
    h_out2, _ = oracle.residual_rmsnorm(h, None, g, 1e-6)
    assert np.array_equal(h_out2, h)


@pytest.mark.parametrize("h,g,eps,want", [
    ([2, 0, 0, 0], [1, 1, 1, 1], 0.0, [2, 0, 0, 0]),        # mean square 1
    ([3, -3, 3, -3], [1, 1, 1, 1], 0.0, [1, -1, 1, -1]),    # rms 3
    ([1, 1, 1, 1], [1, 1, 1, 1], 3.0, [0.5, 0.5, 0.5, 0.5]),  # eps inside the root, added to the mean
    ([1, 1, 1, 1], [1, 2, 3, 4], 0.0, [1, 2, 3, 4]),        # the weight multiplies per channel
    ([0, 0, 0, 0], [1, 1, 1, 1], 1e-6, [0, 0, 0, 0]),       # an all-zero input stays zero
])
def test_exact_cases(h, g, eps, want):
    _, y = oracle.residual_rmsnorm(np.array(h, np.float32), None, np.array(g, np.float32), eps)
    assert np.array_equal(y, np.array(want, np.float64))


def test_power_of_two_scale_invariance():
    rng = np.random.default_rng(2)
    h = rng.standard_normal(1024).astype(np.float32)
    g = rng.uniform(0.5, 2, 1024).astype(np.float32)
    _, y = oracle.residual_rmsnorm(h, None, g, 0.0)
    for e in (-20, -3, 5, 30):
        _, ys = oracle.residual_rmsnorm(h * np.float32(2.0 ** e), None, g, 0.0)
        assert np.array_equal(ys, y), e


def test_unit_mean_square():
    rng = np.random.default_rng(3)
    h = (rng.standard_normal(5120) * 7).astype(np.float32)
    _, y = oracle.residual_rmsnorm(h, None, np.ones(5120, np.float32), 0.0)
    assert abs(np.mean(y * y) - 1.0) < 1e-14


def test_matches_60_digit_arithmetic():
    getcontext().prec = 60
    rng = np.random.default_rng(4)
    k = 96
    h = rng.standard_normal(k).astype(np.float32)
    r = rng.standard_normal(k).astype(np.float32)
    g = rng.uniform(-2, 2, k).astype(np.float32)
    eps = 1e-6
    h_out, y = oracle.residual_rmsnorm(h, r, g, eps)
    hd = [Decimal(float(v)) for v in h_out]
    ms = sum(v * v for v in hd) / k + Decimal(float(np.float64(eps)))
    s = 1 / ms.sqrt()
    for i in range(k):
        exact = hd[i] * s * Decimal(float(g[i]))
        assert abs(Decimal(float(y[i])) - exact) <= abs(exact) * Decimal(2) ** -50 + Decimal(10) ** -300, i
