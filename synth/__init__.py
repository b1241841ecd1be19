"""Seeded synthetic inputs shared by the oracle side and the GPU side.

The definition of every draw is in ``synth.h``.  This package builds the
host library ``libsynth.so`` (gcc) and the device library
``libsynth_dev.so`` (hipcc); both implement that one definition.  Nothing
here quantizes, multiplies matrices or reduces: the method's arithmetic
lives in the oracle and in the HIP library, never in this module.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

_host = None
_dev = None


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except Exception:  # pragma: no cover
        return 1


def host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        u64, i64 = ctypes.c_uint64, ctypes.c_int64
        vp = ctypes.c_void_p
        lib.synth_mix64.restype = u64
        lib.synth_mix64.argtypes = [u64]
        lib.synth_word.restype = u64
        lib.synth_word.argtypes = [u64, u64]
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [u64, u64]
        lib.synth_normal_f32.restype = None
        lib.synth_normal_f32.argtypes = [u64, u64, i64, i64, ctypes.c_float, vp, ctypes.c_int]
        lib.synth_normal_rows_f32.restype = None
        lib.synth_normal_rows_f32.argtypes = [u64, u64, i64, vp, i64, ctypes.c_float, vp, ctypes.c_int]
        lib.synth_int8.restype = None
        lib.synth_int8.argtypes = [u64, u64, i64, i64, vp]
        lib.synth_f16_scale.restype = None
        lib.synth_f16_scale.argtypes = [u64, u64, i64, i64, vp]
        lib.synth_choose.restype = None
        lib.synth_choose.argtypes = [u64, u64, i64, i64, vp]
        _host = lib
    return _host


def dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEV_LIB)
        lib.synth_dev_normal_f32.restype = ctypes.c_int
        lib.synth_dev_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                                             ctypes.c_void_p]
        _dev = lib
    return _dev


# ---------------------------------------------------------------- host draws

def mix64(z: int) -> int:
    return int(host_lib().synth_mix64(z & 0xFFFFFFFFFFFFFFFF))


def word(key: int, n: int) -> int:
    return int(host_lib().synth_word(key & 0xFFFFFFFFFFFFFFFF, n))


def key(seed: int, tensor: int) -> int:
    return int(host_lib().synth_key(seed, tensor))


def normal_f32(seed: int, tensor: int, count: int, sigma: float = 1.0, first: int = 0) -> np.ndarray:
    out = np.empty(count, dtype=np.float32)
    if count:
        host_lib().synth_normal_f32(seed, tensor, first, count, sigma, out.ctypes.data, _threads())
    return out


def normal_rows_f32(seed: int, tensor: int, k: int, rows: Sequence[int], sigma: float) -> np.ndarray:
    """Rows of the row-major (n x k) normal matrix of tensor id ``tensor``."""
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((len(r), k), dtype=np.float32)
    if len(r) and k:
        host_lib().synth_normal_rows_f32(seed, tensor, k, r.ctypes.data, len(r), sigma,
                                         out.ctypes.data, _threads())
    return out


def int8_draws(seed: int, tensor: int, count: int, first: int = 0) -> np.ndarray:
    out = np.empty(count, dtype=np.int8)
    if count:
        host_lib().synth_int8(seed, tensor, first, count, out.ctypes.data)
    return out


def f16_scale_draws(seed: int, tensor: int, count: int, first: int = 0) -> np.ndarray:
    out = np.empty(count, dtype=np.uint16)
    if count:
        host_lib().synth_f16_scale(seed, tensor, first, count, out.ctypes.data)
    return out


def choose(seed: int, tensor: int, n: int, m: int) -> np.ndarray:
    m = min(m, n)
    out = np.empty(m, dtype=np.int64)
    if m:
        host_lib().synth_choose(seed, tensor, n, m, out.ctypes.data)
    return out


# ------------------------------------------------------------ composite inputs

def activation(seed: int, tensor: int, k: int, *, outlier_frac: float = 0.0,
               outlier_mult: float = 20.0, rms: bool = False) -> np.ndarray:
    """An f32 activation ~N(0,1).

    ``outlier_frac``: exactly round(frac*k) entries, chosen by a seeded
    partial Fisher-Yates (tensor id ``tensor + 1``), are multiplied by
    ``outlier_mult`` (one fp32 multiply each).
    ``rms``: x <- x / sqrt(mean(x^2) + 1e-6), computed in fp64 and rounded
    to f32 once, with unit gain (the synthetic RMSNorm scaling applied to
    every layer input).
    """
    x = normal_f32(seed, tensor, k, 1.0)
    m = int(round(outlier_frac * k))
    if m:
        idx = choose(seed, tensor + 1, k, m)
        x[idx] = x[idx] * np.float32(outlier_mult)
    if rms:
        x64 = x.astype(np.float64)
        ms = float(np.mean(x64 * x64))
        x = (x64 / np.sqrt(ms + 1e-6)).astype(np.float32)
    return x


def q8_blocks(seed: int, tensor: int, n: int, k: int):
    """Directly drawn Q8_0 blocks (no quantization): fp16 scale bits
    uint16[n, k/32] and int8 codes int8[n, k] in [-127, 127]."""
    assert k % 32 == 0
    d = f16_scale_draws(seed, tensor, n * (k // 32)).reshape(n, k // 32)
    q = int8_draws(seed, tensor + 1, n * k).reshape(n, k)
    return d, q


def blocks_to_aos(d: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Canonical Q8_0 interchange bytes: per row, per 32-block, the fp16
    scale (little-endian) then the 32 int8 codes: 34 bytes per block."""
    n, k = q.shape
    nb = k // 32
    out = np.empty((n, nb, 34), dtype=np.uint8)
    out[:, :, 0:2] = np.ascontiguousarray(d, dtype="<u2").view(np.uint8).reshape(n, nb, 2)
    out[:, :, 2:34] = q.reshape(n, nb, 32).view(np.uint8)
    return out.reshape(n, nb * 34)


# ------------------------------------------------------------- device draws

def dev_normal_f32(ptr: int, seed: int, tensor: int, count: int, sigma: float, first: int = 0,
                   stream: int = 0) -> None:
    rc = dev_lib().synth_dev_normal_f32(seed, tensor, first, count, sigma, ptr, stream)
    if rc != 0:
        raise RuntimeError(f"synth_dev_normal_f32 failed with code {rc}")
