"""CPU oracle for the batch-1 decode GEMV weight stream -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (plain C,
fp64, see ``oracle.c``) with numpy in/out; it shares no code with the HIP
library and never imports it.

Every function is pinned by tests in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "liboracle.so")
SRC = os.path.join(_HERE, "oracle.c")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.c with gcc (C11, -O2, no FP contraction, no fast-math)."""
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f16_to_f64.restype = ctypes.c_double
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_bf16_to_f64.restype = ctypes.c_double
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        for nm in ("orc_f32_to_f16_array", "orc_f16_to_f64_array", "orc_f32_to_bf16_array",
                   "orc_bf16_to_f64_array"):
            getattr(L, nm).restype = None
            getattr(L, nm).argtypes = [vp, i64, vp]
        L.orc_q8_code_array.restype = None
        L.orc_q8_code_array.argtypes = [vp, vp, i64, vp]
        L.orc_quantize_q8_0.restype = ctypes.c_int
        L.orc_quantize_q8_0.argtypes = [vp, i64, i64, vp, vp]
        L.orc_gemv_q8_act_q8.restype = ctypes.c_int
        L.orc_gemv_q8_act_q8.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp, vp]
        L.orc_gemv_q8_act_f32.restype = ctypes.c_int
        L.orc_gemv_q8_act_f32.argtypes = [vp, vp, i64, i64, vp, vp, vp]
        L.orc_gemv_bf16.restype = ctypes.c_int
        L.orc_gemv_bf16.argtypes = [vp, i64, i64, vp, vp, vp]
        L.orc_argmax_f64.restype = i64
        L.orc_argmax_f64.argtypes = [vp, i64]
        L.orc_argmax_f32.restype = i64
        L.orc_argmax_f32.argtypes = [vp, i64]
        L.orc_residual_rmsnorm.restype = None
        L.orc_residual_rmsnorm.argtypes = [vp, vp, vp, i64, ctypes.c_double, vp, vp]
        L.orc_quantize_q4_0.restype = ctypes.c_int
        L.orc_quantize_q4_0.argtypes = [vp, i64, i64, vp, vp]
        L.orc_swiglu.restype = None
        L.orc_swiglu.argtypes = [vp, vp, i64, vp]
        _lib = L
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- O1 codecs

def _map(fn_name: str, a: np.ndarray, in_dtype, out_dtype) -> np.ndarray:
    shape = np.shape(a)
    a = _c(a, in_dtype)
    out = np.empty(a.shape, dtype=out_dtype)
    if a.size:
        getattr(lib(), fn_name)(a.ctypes.data, a.size, out.ctypes.data)
    return out.reshape(shape)


def f32_to_f16_bits(x) -> np.ndarray:
    return _map("orc_f32_to_f16_array", np.asarray(x), np.float32, np.uint16)


def f16_bits_to_f64(h) -> np.ndarray:
    return _map("orc_f16_to_f64_array", np.asarray(h), np.uint16, np.float64)


def f32_to_bf16_bits(x) -> np.ndarray:
    return _map("orc_f32_to_bf16_array", np.asarray(x), np.float32, np.uint16)


def bf16_bits_to_f64(h) -> np.ndarray:
    return _map("orc_bf16_to_f64_array", np.asarray(h), np.uint16, np.float64)


# --------------------------------------------------------------- O2 quantizer

def quantize_q8_0(x: np.ndarray):
    """x float32[..., k] (k % 32 == 0) -> (d fp16 bits uint16[..., k/32], q int8[..., k])."""
    x = _c(x, np.float32)
    k = x.shape[-1]
    rows = int(x.size // k) if k else 0
    d = np.empty(x.shape[:-1] + (k // 32,), dtype=np.uint16)
    q = np.empty(x.shape, dtype=np.int8)
    rc = lib().orc_quantize_q8_0(x.ctypes.data, rows, k, d.ctypes.data, q.ctypes.data)
    if rc != 0:
        raise ValueError(f"orc_quantize_q8_0 failed ({rc})")
    return d, q


def quantize_q4_0(x: np.ndarray):
    """4-bit blocks (O11): x float32[..., k] -> (d fp16 bits [..., k/32], q int8 in [-7, 7] [..., k]).
    The GEMV over these codes is gemv_q8_act_q8 (the same block-dot form)."""
    x = _c(x, np.float32)
    k = x.shape[-1]
    rows = int(x.size // k) if k else 0
    d = np.empty(x.shape[:-1] + (k // 32,), dtype=np.uint16)
    q = np.empty(x.shape, dtype=np.int8)
    rc = lib().orc_quantize_q4_0(x.ctypes.data, rows, k, d.ctypes.data, q.ctypes.data)
    if rc != 0:
        raise ValueError(f"orc_quantize_q4_0 failed ({rc})")
    return d, q


def q8_codes(v, d16) -> np.ndarray:
    """Per-value Q8_0 codes against given fp16 scales (the quantizer's inner rule)."""
    v = _c(v, np.float32)
    d16 = _c(d16, np.uint16)
    assert v.shape == d16.shape
    out = np.empty(v.shape, dtype=np.int8)
    if v.size:
        lib().orc_q8_code_array(v.ctypes.data, d16.ctypes.data, v.size, out.ctypes.data)
    return out


# ------------------------------------------------------------------ O3-O5

def gemv_q8_act_q8(dw, qw, dx, qx, want_dots: bool = False):
    dw, qw = _c(dw, np.uint16), _c(qw, np.int8)
    dx, qx = _c(dx, np.uint16), _c(qx, np.int8)
    n, k = qw.shape
    assert dw.shape == (n, k // 32) and qx.shape == (k,) and dx.shape == (k // 32,)
    y = np.empty(n, dtype=np.float64)
    den = np.empty(n, dtype=np.float64)
    dots = np.empty((n, k // 32), dtype=np.int32) if want_dots else None
    rc = lib().orc_gemv_q8_act_q8(dw.ctypes.data, qw.ctypes.data, n, k, dx.ctypes.data,
                                  qx.ctypes.data, y.ctypes.data, den.ctypes.data,
                                  dots.ctypes.data if dots is not None else None)
    if rc != 0:
        raise ValueError(f"orc_gemv_q8_act_q8 failed ({rc})")
    return (y, den, dots) if want_dots else (y, den)


def gemv_q8_act_f32(dw, qw, x):
    dw, qw, x = _c(dw, np.uint16), _c(qw, np.int8), _c(x, np.float32)
    n, k = qw.shape
    assert dw.shape == (n, k // 32) and x.shape == (k,)
    y = np.empty(n, dtype=np.float64)
    den = np.empty(n, dtype=np.float64)
    rc = lib().orc_gemv_q8_act_f32(dw.ctypes.data, qw.ctypes.data, n, k, x.ctypes.data,
                                   y.ctypes.data, den.ctypes.data)
    if rc != 0:
        raise ValueError(f"orc_gemv_q8_act_f32 failed ({rc})")
    return y, den


def gemv_bf16(w_bits, x):
    w, x = _c(w_bits, np.uint16), _c(x, np.float32)
    n, k = w.shape
    assert x.shape == (k,)
    y = np.empty(n, dtype=np.float64)
    den = np.empty(n, dtype=np.float64)
    rc = lib().orc_gemv_bf16(w.ctypes.data, n, k, x.ctypes.data, y.ctypes.data, den.ctypes.data)
    if rc != 0:
        raise ValueError(f"orc_gemv_bf16 failed ({rc})")
    return y, den


def f32_to_bf16_rows(w: np.ndarray) -> np.ndarray:
    """Offline BF16 weight preparation: RNE of every f32 weight (O1)."""
    return f32_to_bf16_bits(w)


# ---------------------------------------------------------------------- O6

def argmax_f64(v) -> int:
    v = _c(v, np.float64)
    return int(lib().orc_argmax_f64(v.ctypes.data, v.size))


def argmax_f32(v) -> int:
    v = _c(v, np.float32)
    return int(lib().orc_argmax_f32(v.ctypes.data, v.size))


# ---------------------------------------------------------------------- O9

def residual_rmsnorm(h, r, g, eps: float):
    """Residual add + RMSNorm (see oracle.c, O9): returns (h' float32[k], the
    fp32 residual stream after the add; y float64[k]).  r may be None."""
    h = _c(h, np.float32)
    g = _c(g, np.float32)
    k = h.size
    assert h.shape == (k,) and g.shape == (k,)
    rp = None
    if r is not None:
        r = _c(r, np.float32)
        assert r.shape == (k,)
        rp = r.ctypes.data
    h_out = np.empty(k, dtype=np.float32)
    y = np.empty(k, dtype=np.float64)
    if k:
        lib().orc_residual_rmsnorm(h.ctypes.data, rp, g.ctypes.data, k, float(eps), h_out.ctypes.data, y.ctypes.data)
    return h_out, y


# --------------------------------------------------------------------- O10

def swiglu(g, u) -> np.ndarray:
    """SwiGLU epilogue (see oracle.c, O10): silu(g) * u in fp64."""
    g = _c(g, np.float64)
    u = _c(u, np.float64)
    assert g.shape == u.shape and g.ndim == 1
    y = np.empty(g.size, dtype=np.float64)
    if g.size:
        lib().orc_swiglu(g.ctypes.data, u.ctypes.data, g.size, y.ctypes.data)
    return y


# ------------------------------------------------------------ tolerances O7

# |silu'(x)| = |s(x) (1 + x (1 - s(x)))| (s the logistic function) peaks at
# ~1.0998 near x = 2.4: the bound used below (pinned in the tests).
SILU_SLOPE_MAX = 1.1
# fp32 rounding of the epilogue itself: expf (a few ulp), one add, one
# divide, one multiply; 2^-20 leaves ~8x margin over their sum.
SWIGLU_REL_TOL = 2.0 ** -20


def swiglu_tolerance(g_ref, u_ref, tol_g, tol_u) -> np.ndarray:
    """Bound on |y - silu(g) u| for y computed in fp32 from g', u' with
    |g' - g| <= tol_g and |u' - u| <= tol_u:
      |silu(g)| tol_u + 1.1 tol_g (|u| + tol_u)           (input errors)
      + 2^-20 (|silu(g)| + 1.1 tol_g)(|u| + tol_u)        (fp32 epilogue)
      + 1e-30 (|u| + tol_u)                               (exp underflow)."""
    g = np.asarray(g_ref, np.float64)
    u = np.abs(np.asarray(u_ref, np.float64))
    tg = np.asarray(tol_g, np.float64)
    tu = np.asarray(tol_u, np.float64)
    s = np.abs(swiglu(g, np.ones_like(g)))
    return s * tu + SILU_SLOPE_MAX * tg * (u + tu) + SWIGLU_REL_TOL * (s + SILU_SLOPE_MAX * tg) * (u + tu) \
        + 1e-30 * (u + tu)

Q8_REL_TOL = 1e-4          # |y - y_ref| <= 1e-4 * sum_b |d_w d_x s_b| (and the f32-x analogue)
BF16_REL_TOL = 2.0 ** -10  # |y - y_ref| <= 2^-10 * sum_i |w_i x_i|


def q8_tolerance(den: np.ndarray) -> np.ndarray:
    return Q8_REL_TOL * np.asarray(den, dtype=np.float64)


def bf16_tolerance(den: np.ndarray) -> np.ndarray:
    return BF16_REL_TOL * np.asarray(den, dtype=np.float64)
