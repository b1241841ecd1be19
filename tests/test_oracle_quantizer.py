"""Pins for the oracle's Q8_0 block quantizer (llama.cpp-style blocks of 32
int8 codes and one fp16 scale; emit_qwen38_generate, "Where the speed comes
from": Q8_0 weights and int8-quantized activations).

The readings pinned here: d16 = fp16_RNE(max|x| / 127) with an IEEE fp32
divide; q = clamp(round_half_away(x / d16), -127, 127) against the stored
scale; an all-zero (or underflowing) block stores d = +0, q = 0."""
import numpy as np
import pytest

import oracle


def _blocks(rng, nblk, scale):
    x = (rng.standard_normal((nblk, 32)) * scale).astype(np.float32)
    return x


@pytest.mark.parametrize("scale", [0.02, 1.0, 20.0, 1e-2, 1000.0])
def test_roundtrip_error_bound(scale):
    rng = np.random.default_rng(int(scale * 1000) + 1)
    x = _blocks(rng, 4000, scale)
    d, q = oracle.quantize_q8_0(x.reshape(1, -1))
    d = d.reshape(-1)
    q = q.reshape(-1, 32).astype(np.float64)
    d64 = oracle.f16_bits_to_f64(d)
    assert np.all((d & 0x7C00) != 0), "all scales normal for these magnitudes"
    err = np.abs(d64[:, None] * q - x.astype(np.float64))
    assert np.all(err <= d64[:, None] * (0.5 + 2.0 ** -17))
    assert np.all(np.abs(q) <= 127)
    # signs follow the input (a dropped sign would fail the bound anyway)
    nz = q != 0
    assert np.all(np.sign(q[nz]) == np.sign(x[nz]))


def test_scale_matches_library_division_and_rounding():
    rng = np.random.default_rng(5)
    x = _blocks(rng, 5000, 0.7)
    d, _ = oracle.quantize_q8_0(x.reshape(1, -1))
    amax = np.max(np.abs(x), axis=1).astype(np.float32)
    ref = (amax / np.float32(127.0)).astype(np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(d.reshape(-1), ref)


def test_max_element_maps_to_127_when_scale_exact():
    # amax = 127 * 2^-7 makes d = 2^-7 exactly; that element must be +-127
    x = np.zeros((2, 32), np.float32)
    x[0, 5] = 127 * 2.0 ** -7
    x[1, 31] = -127 * 2.0 ** -7
    x[0, 6] = 0.25
    d, q = oracle.quantize_q8_0(x.reshape(1, 64))
    assert d.tolist() == [[0x2000, 0x2000]]  # 2^-7 in binary16
    assert q[0, 5] == 127 and q[0, 32 + 31] == -127
    assert q[0, 6] == 32


def test_half_quotients_round_away_from_zero():
    s = 2.0 ** -7
    vals = [2.5, -2.5, 0.5, -0.5, 1.5, 126.5, -126.5, 3.5, 4.5]
    x = np.zeros(32, np.float32)
    x[0] = 127 * s  # fixes d16 = 2^-7 exactly
    x[1:1 + len(vals)] = np.array(vals, np.float64) * s
    d, q = oracle.quantize_q8_0(x.reshape(1, 32))
    assert d.tolist() == [[0x2000]]
    assert q[0, 1:1 + len(vals)].tolist() == [3, -3, 1, -1, 2, 127, -127, 4, 5]


def test_zero_and_underflow_blocks():
    x = np.zeros((1, 96), np.float32)
    x[0, 32:64] = 1e-12   # d = 7.9e-15 underflows binary16 to zero
    x[0, 64] = -0.0
    d, q = oracle.quantize_q8_0(x)
    assert d.tolist() == [[0, 0, 0]]
    assert not q.any()


def test_subnormal_scale_clamps():
    # amax/127 in the fp16 subnormal range: codes still within [-127, 127]
    x = np.full((1, 32), 3e-4, np.float32)
    x[0, 0] = 2.5e-3
    d, q = oracle.quantize_q8_0(x)
    assert (d[0, 0] & 0x7C00) == 0 and d[0, 0] != 0
    assert np.abs(q.astype(int)).max() <= 127


def test_requantize_is_identity():
    # x = d16 * q with some |q| = 127 per block quantizes back to (d16, q)
    rng = np.random.default_rng(9)
    nb = 300
    q0 = rng.integers(-127, 128, size=(nb, 32)).astype(np.int8)
    q0[np.arange(nb), rng.integers(0, 32, nb)] = rng.choice([-127, 127], nb)
    e = rng.integers(-12, 3, size=nb)
    mant = rng.integers(1024, 2048, size=nb)
    d0 = (np.ldexp(mant.astype(np.float64), e - 10)).astype(np.float16)
    x = (d0.astype(np.float64)[:, None] * q0.astype(np.float64)).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), d0.astype(np.float64)[:, None] * q0)
    d, q = oracle.quantize_q8_0(x.reshape(1, -1))
    assert np.array_equal(d.reshape(-1), d0.view(np.uint16))
    assert np.array_equal(q.reshape(nb, 32), q0)


def test_never_minus_128():
    rng = np.random.default_rng(3)
    x = _blocks(rng, 2000, 5.0)
    _, q = oracle.quantize_q8_0(x.reshape(1, -1))
    assert q.min() >= -127


def test_rows_are_independent():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((3, 128)) * 0.02).astype(np.float32)
    d, q = oracle.quantize_q8_0(x)
    for r in range(3):
        dr, qr = oracle.quantize_q8_0(x[r:r + 1])
        assert np.array_equal(d[r], dr[0]) and np.array_equal(q[r], qr[0])


def test_rejects_ragged_k_and_nonfinite():
    with pytest.raises(ValueError):
        oracle.quantize_q8_0(np.zeros((1, 33), np.float32))
    x = np.zeros((1, 32), np.float32)
    x[0, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.quantize_q8_0(x)
