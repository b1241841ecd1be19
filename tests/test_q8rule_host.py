"""The HIP library's divide-free Q8_0 code rules (csrc/q8rule.hpp: the exact
boundary test, and the branch-free form that defers to it next to a
boundary), built for the host, give exactly the oracle's codes (an IEEE fp32 divide by the
stored scale, rounded half away from zero) on random values, on values
planted at and one ulp around every rounding boundary m + 1/2, and across
normal and subnormal fp16 scales."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


# the GPU compiler may fuse a multiply and an add into one FMA; the rules must
# hold with and without that contraction
@pytest.fixture(scope="module", params=[("fast_codes", "off"), ("fast_split_codes", "off"),
                                        ("fast_codes", "fma"), ("fast_split_codes", "fma")])
def fast(tmp_path_factory, request):
    name, contract = request.param
    out = str(tmp_path_factory.mktemp("q8rule") / "libq8rule_host.so")
    flags = ["-ffp-contract=off"] if contract == "off" else ["-ffp-contract=fast", "-mfma"]
    subprocess.run(["g++", "-std=c++17", "-O2", *flags, "-fno-fast-math", "-fPIC", "-shared",
                    "-I", os.path.join(ROOT, "weight_streaming_gemv_q8_amd", "csrc"),
                    os.path.join(HERE, "cpp", "q8rule_host.cpp"), "-o", out], check=True)
    L = ctypes.CDLL(out)
    fn = getattr(L, name)
    fn.restype = None
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]

    def run(v, d16):
        v = np.ascontiguousarray(v, np.float32)
        d16 = np.ascontiguousarray(d16, np.uint16)
        o = np.empty(v.shape, np.int8)
        fn(v.ctypes.data, d16.ctypes.data, v.size, o.ctypes.data)
        return o
    return run


def _scales(rng, n):
    # positive fp16 scales: normal (exponent 1..30) and subnormal (exponent 0)
    ex = rng.integers(0, 31, n)
    fr = rng.integers(0, 1024, n)
    fr[(ex == 0) & (fr == 0)] = 1
    return ((ex << 10) | fr).astype(np.uint16)


def test_random_values(fast):
    rng = np.random.default_rng(0)
    n = 4_000_000
    d16 = _scales(rng, n)
    d = d16.view(np.float16).astype(np.float64)
    # values spread over |v/d| in [0, 130) (and a few beyond, which clamp)
    v = (rng.uniform(-130, 130, n) * d).astype(np.float32)
    assert np.array_equal(fast(v, d16), oracle.q8_codes(v, d16))


def test_planted_boundaries(fast):
    rng = np.random.default_rng(1)
    n_d = 20_000
    d16 = _scales(rng, n_d)
    d = d16.view(np.float16).astype(np.float64)
    m = rng.integers(0, 128, n_d)
    b = (m + 0.5) * d  # the exact boundary value (may not be a float)
    cand = []
    for k in range(-3, 4):
        base = b.astype(np.float32)
        step = np.float32(np.inf) if k > 0 else np.float32(0)
        x = base.copy()
        for _ in range(abs(k)):
            x = np.nextafter(x, step)
        cand.append(x)
    v = np.concatenate(cand)
    dd = np.tile(d16, len(cand))
    sign = np.where(rng.random(v.size) < 0.5, -1, 1).astype(np.float32)
    v = v * sign
    assert np.array_equal(fast(v, dd), oracle.q8_codes(v, dd))


def test_quotient_ties_and_binade_edges(fast):
    # exact half quotients (ties round away) and the 0.5 binade edge
    d16 = np.array([0x2000] * 8 + [0x3C00] * 4 + [0x0001] * 3, np.uint16)  # 2^-7, 1.0, 2^-24
    q = np.array([0.5, 1.5, 2.5, 126.5, 127.5, 3.49999, 0.49999997, 0.5000001, 0.5, -0.5, 1e-30, 200.0,
                  0.5, 1.5, 127.0], np.float64)
    v = (q * d16.view(np.float16).astype(np.float64)).astype(np.float32)
    assert np.array_equal(fast(v, d16), oracle.q8_codes(v, d16))
    assert fast(np.array([-0.0], np.float32), np.array([0x3C00], np.uint16))[0] == 0
