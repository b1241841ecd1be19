"""Helpers for the GPU parity tests: host<->device transfer, a decoder of
the documented Q8_0 device layout, and the acceptance checks."""
from __future__ import annotations

import numpy as np

import oracle

CHUNK_BLOCKS = 64
FULL_CHUNK_BYTES = 2 * CHUNK_BLOCKS + 32 * CHUNK_BLOCKS


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def empty_u8(nbytes: int):
    import torch
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device="cuda")


def row_bytes(k: int) -> int:
    nb = k // 32
    c = (nb + CHUNK_BLOCKS - 1) // CHUNK_BLOCKS
    nl = nb - (c - 1) * CHUNK_BLOCKS
    return (c - 1) * FULL_CHUNK_BYTES + ((2 * nl + 15) // 16) * 16 + 32 * nl


def unpack_device_layout(buf: np.ndarray, n: int, k: int):
    """Decode the packed Q8_0 device layout (see include/wsgemv.h) into
    (d fp16 bits uint16[n, k/32], q int8[n, k]); also returns the scale
    padding bytes, which must be zero."""
    rb = row_bytes(k)
    rows = np.asarray(buf, dtype=np.uint8)[: n * rb].reshape(n, rb)
    nb = k // 32
    c_count = (nb + CHUNK_BLOCKS - 1) // CHUNK_BLOCKS
    d = np.empty((n, nb), np.uint16)
    q = np.empty((n, nb, 32), np.int8)
    pads = []
    for c in range(c_count):
        nbc = min(CHUNK_BLOCKS, nb - c * CHUNK_BLOCKS)
        sb = ((2 * nbc + 15) // 16) * 16
        base = c * FULL_CHUNK_BYTES
        b0 = c * CHUNK_BLOCKS
        d[:, b0:b0 + nbc] = rows[:, base:base + 2 * nbc].copy().view("<u2")
        pads.append(rows[:, base + 2 * nbc:base + sb])
        qa = rows[:, base + sb:base + sb + 16 * nbc].reshape(n, nbc, 16)
        qb = rows[:, base + sb + 16 * nbc:base + sb + 32 * nbc].reshape(n, nbc, 16)
        q[:, b0:b0 + nbc, :16] = qa.view(np.int8)
        q[:, b0:b0 + nbc, 16:] = qb.view(np.int8)
    pad = np.concatenate([p.reshape(n, -1) for p in pads], axis=1) if pads else np.zeros((n, 0), np.uint8)
    return d, q.reshape(n, k), pad


def split_act_q8(buf: np.ndarray, k: int):
    """Planar Q8_0 activation: int8 q[k] then fp16 d[k/32]."""
    b = np.asarray(buf, dtype=np.uint8)
    q = b[:k].view(np.int8).copy()
    d = b[k:k + 2 * (k // 32)].copy().view("<u2")
    return d, q


def assert_within(y_gpu: np.ndarray, y_ref: np.ndarray, tol: np.ndarray, what: str = ""):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, (
        f"{what}: {bad.size} rows out of tolerance; first {bad[:5].tolist()} "
        f"err {err[bad[:5]].tolist()} tol {tol[bad[:5]].tolist()}")


def check_argmax_vs_oracle(idx: int, y_ref: np.ndarray, tol: np.ndarray) -> None:
    """The GPU index must equal the oracle's when the oracle's winner is
    separated from every other row by more than the two rows' tolerances;
    otherwise it must be one of the rows within tolerance of the maximum."""
    ref = oracle.argmax_f64(y_ref)
    if idx == ref:
        return
    m = y_ref[ref]
    close = np.nonzero(y_ref + tol >= m - tol[ref])[0]
    assert idx in set(close.tolist()), (idx, ref, y_ref[idx], m)
