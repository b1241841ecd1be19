"""Pins of the oracle's SwiGLU epilogue (O10) and its tolerance, against
what mathematics and a library routine fix (no GPU):

* silu(x) u equals x * scipy.special.expit(x) * u (the logistic function
  from a library) to fp64 rounding, on random and extreme x;
* closed forms: silu(0) = 0; silu(x) - silu(-x) = x (the logistic function
  satisfies s(x) + s(-x) = 1); silu(x) -> x for large x and -> -0 for very
  negative x, with no NaN; y is linear in u (exact under power-of-two scaling);
  the gate is the first argument (swapping the halves changes the result);
* the slope bound 1.1 used by the tolerance holds (finite differences on a
  dense grid) and is nearly tight;
* the tolerance is achievable: a plain fp32 evaluation from perturbed
  inputs stays inside it, and a 4x larger perturbation of g does not."""
import numpy as np
from scipy.special import expit

import oracle


def test_matches_library_logistic():
    rng = np.random.default_rng(1010)
    g = np.concatenate([rng.normal(0, 3, 100000), rng.uniform(-60, 60, 10000),
                        [0.0, 1e-300, -1e-300, 5e-324, 700.0, -700.0, 36.0, -36.0]])
    u = rng.normal(0, 2, g.size)
    y = oracle.swiglu(g, u)
    ref = g * expit(g) * u
    assert np.all(np.abs(y - ref) <= 8e-16 * np.abs(ref) + 1e-320)  # a few fp64 roundings apart


def test_closed_forms():
    assert oracle.swiglu([0.0], [3.0])[0] == 0.0
    assert oracle.swiglu([2.0], [0.0])[0] == 0.0
    x = np.linspace(-30, 30, 60001)
    odd = oracle.swiglu(x, np.ones_like(x)) - oracle.swiglu(-x, np.ones_like(x))
    assert np.all(np.abs(odd - x) <= 2e-15 * np.maximum(np.abs(x), 1.0))
    big = oracle.swiglu([40.0, 1000.0, 1e6], [1.0, 1.0, 1.0])
    assert big[0] == 40.0 and big[1] == 1000.0 and big[2] == 1e6
    neg = oracle.swiglu([-1000.0, -1e6], [1.0, 1.0])
    assert np.all(neg == 0.0) and not np.any(np.isnan(neg))
    rng = np.random.default_rng(7)
    g, u = rng.normal(0, 3, 1000), rng.normal(0, 3, 1000)
    assert np.array_equal(oracle.swiglu(g, 2.0 * u), 2.0 * oracle.swiglu(g, u))
    assert not np.allclose(oracle.swiglu(g, u), oracle.swiglu(u, g))


def test_slope_bound():
    x = np.linspace(-40, 40, 800001)
    s = oracle.swiglu(x, np.ones_like(x))
    slope = np.abs(np.diff(s) / np.diff(x))
    assert slope.max() <= oracle.SILU_SLOPE_MAX
    assert slope.max() >= 1.09  # the bound is nearly tight


def test_tolerance_is_achievable_and_not_loose():
    rng = np.random.default_rng(2024)
    n = 200000
    g = rng.normal(0, 3, n)
    u = rng.normal(0, 3, n)
    tol_g = 1e-4 * (np.abs(g) + 1.0)
    tol_u = 1e-4 * (np.abs(u) + 1.0)
    y_ref = oracle.swiglu(g, u)
    tol = oracle.swiglu_tolerance(g, u, tol_g, tol_u)
    # perturbed inputs within their bounds, then a plain fp32 epilogue
    g2 = (g + rng.uniform(-1, 1, n) * tol_g).astype(np.float32)
    u2 = (u + rng.uniform(-1, 1, n) * tol_u).astype(np.float32)
    with np.errstate(over="ignore"):
        y32 = (g2 / (np.float32(1.0) + np.exp(-g2)) * u2).astype(np.float32)
    assert np.all(np.abs(y32.astype(np.float64) - y_ref) <= tol)
    # exact inputs: the epilogue's own rounding alone
    gf, uf = g.astype(np.float32), u.astype(np.float32)
    y_exact = oracle.swiglu(gf.astype(np.float64), uf.astype(np.float64))
    with np.errstate(over="ignore"):
        y32 = (gf / (np.float32(1.0) + np.exp(-gf)) * uf).astype(np.float32)
    tol0 = oracle.swiglu_tolerance(gf, uf, 0.0, 0.0)
    assert np.all(np.abs(y32.astype(np.float64) - y_exact) <= tol0)
    # a gate error four times its bound is caught somewhere
    g4 = g + 4.0 * tol_g * np.sign(u)
    assert np.any(np.abs(oracle.swiglu(g4, u) - y_ref) > tol)
