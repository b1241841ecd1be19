"""Pins for the oracle's three GEMV forms (y = W.x at batch 1;
emit_qwen38_generate, "Where the speed comes from"; GPU Kernel Lab,
"Decode integration") against exact rational brute force, library
matrix products, one-hot columns and sign-definite cases.  Shapes are
non-square so that a transposed operand fails."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

ONE_F16 = 0x3C00


def _rand_q8(rng, n, k, exps=(-10, -4)):
    q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    e = rng.integers(exps[0], exps[1], size=(n, k // 32))
    mant = rng.integers(1024, 2048, size=(n, k // 32))
    d = np.ldexp(mant.astype(np.float64), e - 10).astype(np.float16).view(np.uint16)
    return d, q


def _deq(d, q):
    n, k = q.shape
    dd = oracle.f16_bits_to_f64(d)
    return np.repeat(dd, 32, axis=1) * q.astype(np.float64)


# ------------------------------------------------------------ int8 form (O3)

def test_int8_form_unit_scales_is_integer_matvec():
    rng = np.random.default_rng(1)
    n, k = 37, 160
    qw = rng.integers(-127, 128, (n, k)).astype(np.int8)
    qx = rng.integers(-127, 128, k).astype(np.int8)
    dw = np.full((n, k // 32), ONE_F16, np.uint16)
    dx = np.full(k // 32, ONE_F16, np.uint16)
    y, den, dots = oracle.gemv_q8_act_q8(dw, qw, dx, qx, want_dots=True)
    ref = qw.astype(np.int64) @ qx.astype(np.int64)
    assert np.array_equal(y, ref.astype(np.float64))
    ref_dots = np.einsum("rbi,bi->rb", qw.reshape(n, k // 32, 32).astype(np.int64),
                         qx.reshape(k // 32, 32).astype(np.int64))
    assert np.array_equal(dots, ref_dots)


def test_int8_form_exact_rational_bruteforce():
    rng = np.random.default_rng(2)
    n, k = 3, 64
    dw, qw = _rand_q8(rng, n, k)
    dx, qx = _rand_q8(rng, 1, k)
    dx, qx = dx[0], qx[0]
    y, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
    # dequantize both operands exactly and take the plain matrix-vector product
    for r in range(n):
        acc = Fraction(0)
        mag = Fraction(0)
        for i in range(k):
            w = Fraction(float(oracle.f16_bits_to_f64(dw[r, i // 32]))) * int(qw[r, i])
            xv = Fraction(float(oracle.f16_bits_to_f64(dx[i // 32]))) * int(qx[i])
            acc += w * xv
        assert float(acc) == pytest.approx(y[r], rel=1e-15, abs=1e-300)


def test_int8_form_vs_dequantized_matmul():
    rng = np.random.default_rng(3)
    n, k = 45, 352
    dw, qw = _rand_q8(rng, n, k)
    dx, qx = _rand_q8(rng, 1, k)
    y, den = oracle.gemv_q8_act_q8(dw, qw, dx[0], qx[0])
    ref = _deq(dw, qw) @ _deq(dx, qx)[0]
    assert np.all(np.abs(y - ref) <= 1e-13 * den)
    # den is the sum of |term| per block: >= |y|, and equal when all terms agree in sign
    assert np.all(den >= np.abs(y))


def test_int8_form_sign_definite_den_equals_y():
    rng = np.random.default_rng(4)
    n, k = 5, 96
    qw = rng.integers(1, 128, (n, k)).astype(np.int8)
    qx = rng.integers(1, 128, k).astype(np.int8)
    dw, _ = _rand_q8(rng, n, k)
    dx, _ = _rand_q8(rng, 1, k)
    y, den = oracle.gemv_q8_act_q8(dw, qw, dx[0], qx)
    assert np.array_equal(y, den)


def test_int8_form_dot_extremes_fit_int32():
    n, k = 2, 64
    qw = np.full((n, k), -127, np.int8)
    qw[1] = 127
    qx = np.full(k, -127, np.int8)
    dw = np.full((n, 2), ONE_F16, np.uint16)
    dx = np.full(2, ONE_F16, np.uint16)
    _, _, dots = oracle.gemv_q8_act_q8(dw, qw, dx, qx, want_dots=True)
    assert dots.tolist() == [[516128, 516128], [-516128, -516128]]


# ------------------------------------------------------ dequant form (O4)

def test_f32_form_vs_dequantized_matmul():
    rng = np.random.default_rng(5)
    n, k = 29, 416
    dw, qw = _rand_q8(rng, n, k)
    x = rng.standard_normal(k).astype(np.float32)
    y, den = oracle.gemv_q8_act_f32(dw, qw, x)
    W = _deq(dw, qw)
    ref = W @ x.astype(np.float64)
    assert np.all(np.abs(y - ref) <= 1e-13 * den)
    assert np.allclose(den, np.abs(W) @ np.abs(x.astype(np.float64)), rtol=1e-13, atol=0)


def test_f32_form_one_hot_is_a_column():
    rng = np.random.default_rng(6)
    n, k = 17, 128
    dw, qw = _rand_q8(rng, n, k)
    for j in (0, 31, 32, 77, 127):
        x = np.zeros(k, np.float32)
        x[j] = 1.0
        y, _ = oracle.gemv_q8_act_f32(dw, qw, x)
        col = oracle.f16_bits_to_f64(dw[:, j // 32]) * qw[:, j].astype(np.float64)
        assert np.array_equal(y, col)


def test_f32_form_exact_rational_bruteforce():
    rng = np.random.default_rng(7)
    n, k = 3, 64
    dw, qw = _rand_q8(rng, n, k)
    x = np.ldexp(rng.integers(-1000, 1000, k).astype(np.float64), -9).astype(np.float32)
    y, _ = oracle.gemv_q8_act_f32(dw, qw, x)
    for r in range(n):
        acc = sum(Fraction(float(oracle.f16_bits_to_f64(dw[r, i // 32]))) * int(qw[r, i]) *
                  Fraction(float(x[i])) for i in range(k))
        assert float(acc) == y[r]  # dyadic inputs with few bits: the fp64 sum is exact


# ------------------------------------------------------------ BF16 (O5)

def test_bf16_form_vs_torch():
    rng = np.random.default_rng(8)
    n, k = 33, 520
    w32 = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    wb = oracle.f32_to_bf16_rows(w32)
    x = rng.standard_normal(k).astype(np.float32)
    y, den = oracle.gemv_bf16(wb, x)
    tw = torch.from_numpy(w32).to(torch.bfloat16).to(torch.float64)
    ref = (tw @ torch.from_numpy(x).to(torch.float64)).numpy()
    assert np.all(np.abs(y - ref) <= 1e-13 * den)
    assert np.allclose(den, (tw.abs() @ torch.from_numpy(np.abs(x)).double()).numpy(), rtol=1e-13)


def test_bf16_form_one_hot_and_rational():
    rng = np.random.default_rng(9)
    n, k = 4, 40
    w = oracle.f32_to_bf16_rows(rng.standard_normal((n, k)).astype(np.float32))
    for j in (0, 17, 39):
        x = np.zeros(k, np.float32)
        x[j] = -2.0
        y, _ = oracle.gemv_bf16(w, x)
        assert np.array_equal(y, -2.0 * oracle.bf16_bits_to_f64(w[:, j]))
    x = np.ldexp(rng.integers(-64, 64, k).astype(np.float64), -3).astype(np.float32)
    y, _ = oracle.gemv_bf16(w, x)
    for r in range(n):
        acc = sum(Fraction(float(oracle.bf16_bits_to_f64(w[r, i]))) * Fraction(float(x[i]))
                  for i in range(k))
        assert float(acc) == y[r]


# ---------------------------------------------- tolerance achievability (O7)

@pytest.mark.parametrize("k", [1024, 5120, 17408])
def test_naive_fp32_sequential_meets_q8_tolerances(k):
    """A plain sequential fp32 implementation passes the acceptance bounds,
    so they are achievable (int8 form: chain of K/32 block terms; f32 form:
    per-block sums of 32 then K/32 block terms)."""
    rng = np.random.default_rng(k)
    n = 8
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = rng.standard_normal(k).astype(np.float32)
    dw, qw = oracle.quantize_q8_0(w)
    dx, qx = oracle.quantize_q8_0(x)
    y, den, dots = oracle.gemv_q8_act_q8(dw, qw, dx, qx, want_dots=True)
    dwf = oracle.f16_bits_to_f64(dw).astype(np.float32)
    dxf = oracle.f16_bits_to_f64(dx).astype(np.float32)
    for r in range(n):
        acc = np.float32(0)
        for b in range(k // 32):
            acc = np.float32(acc + np.float32(dwf[r, b] * dxf[b]) * np.float32(dots[r, b]))
        assert abs(float(acc) - y[r]) <= oracle.q8_tolerance(den[r])
    y2, den2 = oracle.gemv_q8_act_f32(dw, qw, x)
    for r in range(n):
        acc = np.float32(0)
        for b in range(k // 32):
            t = np.cumsum(qw[r, 32 * b:32 * b + 32].astype(np.float32) * x[32 * b:32 * b + 32],
                          dtype=np.float32)[-1]
            acc = np.float32(acc + np.float32(dwf[r, b]) * t)
        assert abs(float(acc) - y2[r]) <= oracle.q8_tolerance(den2[r])


def test_naive_fp32_sequential_meets_bf16_tolerance():
    rng = np.random.default_rng(11)
    n, k = 8, 4096
    w = oracle.f32_to_bf16_rows((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    x = rng.standard_normal(k).astype(np.float32)
    y, den = oracle.gemv_bf16(w, x)
    wf = oracle.bf16_bits_to_f64(w).astype(np.float32)
    for r in range(n):
        acc = np.cumsum(wf[r] * x, dtype=np.float32)[-1]
        assert abs(float(acc) - y[r]) <= oracle.bf16_tolerance(den[r])


def test_rejects_bad_shapes():
    with pytest.raises(AssertionError):
        oracle.gemv_q8_act_f32(np.zeros((2, 1), np.uint16), np.zeros((2, 32), np.int8),
                               np.zeros(31, np.float32))
