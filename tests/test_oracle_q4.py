"""Pins of the oracle's 4-bit block quantizer (O11), against what the
rule and arithmetic fix (no GPU):

* the scale is numpy's fp32 max|x| / 7 rounded to fp16; codes lie in
  [-7, 7], and the block maximum gets |q| = 7 when that scale is exact;
* the round trip |d16 q - x| <= d16 (1/2 + 2^-17) for every value (one fp32
  rounding of the quotient);
* exact .5 quotients round away from zero (not to even);
* zero and underflowing blocks give d = +0, q = 0; a block of d q values
  re-quantizes to itself;
* the codes differ from the 8-bit rule's (a check that 7, not 127, is
  used), and the block-dot GEMV over them equals a numpy integer matvec
  when every scale is 1."""
import numpy as np

import oracle


def test_scale_codes_and_round_trip():
    rng = np.random.default_rng(404)
    x = (rng.normal(0, 0.02, (64, 4096)) * np.exp(rng.normal(0, 1, (64, 1)))).astype(np.float32)
    d, q = oracle.quantize_q4_0(x)
    xb = x.reshape(64, -1, 32)
    want_d = (np.abs(xb).max(axis=2) / np.float32(7.0)).astype(np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(d, want_d)
    assert q.min() >= -7 and q.max() <= 7
    df = oracle.f16_bits_to_f64(d)[..., None]
    err = np.abs(df * q.reshape(64, -1, 32) - xb)
    assert np.all(err <= df * (0.5 + 2.0 ** -17))
    q8 = oracle.quantize_q8_0(x)[1]
    assert not np.array_equal(q, q8)


def test_max_element_and_half_quotients():
    d16 = np.float16(2.0 ** -6)
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 7 * float(d16)            # the maximum: q = 7, scale exact
    x[0, 1] = 2.5 * float(d16)          # exact .5 quotient: away from zero -> 3
    x[0, 2] = -2.5 * float(d16)         # -> -3
    x[0, 3] = 0.5 * float(d16)          # -> 1
    x[0, 4] = -6.5 * float(d16)         # -> -7
    d, q = oracle.quantize_q4_0(x)
    assert d[0, 0] == d16.view(np.uint16)
    assert q[0, :5].tolist() == [7, 3, -3, 1, -7]


def test_zero_underflow_and_requantization():
    x = np.zeros((2, 64), np.float32)
    x[1, 32:] = 1e-12                   # max / 7 underflows fp16
    d, q = oracle.quantize_q4_0(x)
    assert np.all(d == 0) and np.all(q == 0)
    rng = np.random.default_rng(5)
    d16 = (np.abs(rng.normal(0, 0.01, (8, 4))) + 1e-3).astype(np.float16)
    codes = rng.integers(-7, 8, (8, 128)).astype(np.int8)
    codes.reshape(8, 4, 32)[:, :, 0] = 7  # each block reaches the maximum
    x = (np.repeat(d16.astype(np.float64), 32, axis=1) * codes).astype(np.float32)
    d2, q2 = oracle.quantize_q4_0(x)
    assert np.array_equal(d2, d16.view(np.uint16)) and np.array_equal(q2, codes)


def test_block_dot_gemv_over_4bit_codes():
    rng = np.random.default_rng(9)
    q = rng.integers(-7, 8, (5, 96)).astype(np.int8)
    qx = rng.integers(-127, 128, 96).astype(np.int8)
    one = np.float16(1.0).view(np.uint16)
    y, _ = oracle.gemv_q8_act_q8(np.full((5, 3), one, np.uint16), q, np.full(3, one, np.uint16), qx)
    assert np.array_equal(y, q.astype(np.int64) @ qx.astype(np.int64))
