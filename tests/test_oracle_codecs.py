"""Pins for the oracle's binary16 / bfloat16 codecs against library
conversions (numpy's float16, torch's bfloat16), exhaustively where the
format is small, and on constructed round-to-nearest-even midpoints."""
import numpy as np
import torch

import oracle


def _all_f16_bits():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_f16_decode_exhaustive_vs_numpy():
    h = _all_f16_bits()
    ours = oracle.f16_bits_to_f64(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signs of zeros
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0x0000])


def test_f16_encode_roundtrip_exhaustive():
    h = _all_f16_bits()
    vals = h.view(np.float16).astype(np.float32)
    finite = np.isfinite(vals)
    back = oracle.f32_to_f16_bits(vals[finite])
    assert np.array_equal(back, h[finite])


def test_f16_encode_midpoints_ties_to_even():
    # every midpoint between adjacent non-negative finite fp16 values is
    # exact in f32 (12 significant bits) and must round to the even code
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    got = oracle.f32_to_f16_bits(mid)
    even = np.where(h % 2 == 0, h, h + 1).astype(np.uint16)
    assert np.array_equal(got, even)
    assert np.array_equal(got, mid.astype(np.float16).view(np.uint16))
    # and the negatives mirror them
    gotn = oracle.f32_to_f16_bits(-mid)
    assert np.array_equal(gotn, even | 0x8000)


def test_f16_encode_random_vs_numpy():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # concentrate half of the samples on the fp16 range, including subnormals
    y = (rng.standard_normal(1_000_000) * np.exp2(rng.integers(-30, 17, 1_000_000))).astype(np.float32)
    for arr in (x, y):
        with np.errstate(over="ignore"):
            ref = arr.astype(np.float16).view(np.uint16)
        assert np.array_equal(oracle.f32_to_f16_bits(arr), ref)


def test_f16_overflow_and_specials():
    got = oracle.f32_to_f16_bits(np.array([65504, 65519.99, 65520, 1e6, -1e6, np.inf, -np.inf],
                                          np.float32))
    assert got.tolist() == [0x7BFF, 0x7BFF, 0x7C00, 0x7C00, 0xFC00, 0x7C00, 0xFC00]
    n = oracle.f32_to_f16_bits(np.array([np.nan], np.float32))[0]
    assert (n & 0x7C00) == 0x7C00 and (n & 0x3FF) != 0


def test_bf16_decode_exhaustive_vs_torch():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_bits_to_f64(h)
    ref = torch.from_numpy(h.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_encode_vs_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    y = (rng.standard_normal(500_000) * 0.02).astype(np.float32)
    # exact midpoints between adjacent bf16 values, incl. the subnormal range
    hb = rng.integers(0, 0x7F7F, size=200_000).astype(np.uint32)
    mid_bits = (hb << 16) | 0x8000
    z = mid_bits.astype(np.uint32).view(np.float32)
    for arr in (x, y, z, -z):
        ref = torch.from_numpy(arr.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(oracle.f32_to_bf16_bits(arr), ref)


def test_bf16_ties_to_even_constructed():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to the even code (1.0)
    # 1 + 3*2^-8 lies halfway between 1+2^-7 and 1+2^-6: rounds up to 1+2^-6
    got = oracle.f32_to_bf16_bits(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8], np.float32))
    assert got.tolist() == [0x3F80, 0x3F82]
