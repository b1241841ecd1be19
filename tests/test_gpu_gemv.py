"""GPU parity of the three GEMV paths against the oracle (batch-1 decode
GEMV, emit_qwen38_generate, "Where the speed comes from"; split-K decode
GEMV, qwen3-8b-rtx4080-cutedsl, "Decode GEMV path").

* int8 path: per-block int32 dot products bit-exact; y within
  1e-4 * sum_b |d_w d_x s_b|.
* fused-requant path: same bytes, so the same dots and bit-identical y.
* dequant path: y within 1e-4 * sum |d_w q x|.
* BF16: y within 2^-10 * sum |w x|.
Shapes span several chunks, ragged last chunks, one-block rows and the
split-K cases (few rows per CU with long rows)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_within, dev, empty_u8, host

pytestmark = pytest.mark.gpu

SEED = 0x5EED0000

# (n, k): configs[0]'s single GEMV, ragged and tiny shapes, and shapes that
# select 1, 2 and 4 waves per row
Q8_SHAPES = [(1024, 1024), (1, 32), (3, 96), (67, 2080), (130, 4128), (257, 5120), (300, 8288),
             (100, 17408), (2048, 1024), (5, 12288)]
BF16_SHAPES = [(4096, 1024), (1, 8), (3, 24), (77, 1032), (129, 3072), (300, 8192), (64, 17416)]


def _weights(n, k, tensor=1):
    return synth.normal_f32(SEED, tensor, n * k, 0.02).reshape(n, k)


def _act(k, tensor=1000):
    return synth.activation(SEED, tensor, k, outlier_frac=0.01)


def _q8_device(wsg, w):
    n, k = w.shape
    packed = empty_u8(wsg.q8_0_packed_bytes(n, k))
    wsg.quantize_q8_0_weights(dev(w), n, k, packed)
    return packed


@pytest.mark.parametrize("n,k", Q8_SHAPES)
def test_q8_int8_path(gpu_lib, n, k):
    import torch
    wsg = gpu_lib
    w, x = _weights(n, k), _act(k)
    dw, qw = oracle.quantize_q8_0(w)
    dx, qx = oracle.quantize_q8_0(x)
    y_ref, den, dots_ref = oracle.gemv_q8_act_q8(dw, qw, dx, qx, want_dots=True)
    tol = oracle.q8_tolerance(den)

    packed = _q8_device(wsg, w)
    xd = dev(x)
    xq = empty_u8(wsg.act_q8_0_bytes(k))
    wsg.quantize_act_q8_0(xd, k, xq)
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    dots = torch.empty(n * (k // 32), dtype=torch.int32, device="cuda")
    wsg.gemv_q8_0(packed, n, k, xq, wsg.ACT_Q8_0, y, dots)
    assert np.array_equal(host(dots).reshape(n, k // 32), dots_ref)
    y0 = host(y)
    assert_within(y0, y_ref, tol, f"int8 path {n}x{k}")

    # production instantiation (no debug output) gives the same bits
    y1 = torch.empty_like(y)
    wsg.gemv_q8_0(packed, n, k, xq, wsg.ACT_Q8_0, y1)
    assert np.array_equal(host(y1).view(np.uint32), y0.view(np.uint32))

    # fused requantization: same activation bytes, same dots, same bits
    y2 = torch.empty_like(y)
    dots2 = torch.empty_like(dots)
    wsg.gemv_q8_0(packed, n, k, xd, wsg.ACT_F32_REQUANT, y2, dots2)
    assert np.array_equal(host(dots2).reshape(n, k // 32), dots_ref)
    assert np.array_equal(host(y2).view(np.uint32), y0.view(np.uint32))


@pytest.mark.parametrize("n,k", Q8_SHAPES)
def test_q8_dequant_path(gpu_lib, n, k):
    import torch
    wsg = gpu_lib
    if k > wsg.MAX_K_F32ACT:
        pytest.skip("k above the f32-activation limit")
    w, x = _weights(n, k, 2), _act(k, 1002)
    dw, qw = oracle.quantize_q8_0(w)
    y_ref, den = oracle.gemv_q8_act_f32(dw, qw, x)
    packed = _q8_device(wsg, w)
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    wsg.gemv_q8_0(packed, n, k, dev(x), wsg.ACT_F32, y)
    assert_within(host(y), y_ref, oracle.q8_tolerance(den), f"dequant path {n}x{k}")


@pytest.mark.parametrize("n,k", BF16_SHAPES)
def test_bf16_path(gpu_lib, n, k):
    import torch
    wsg = gpu_lib
    w = _weights(n, k, 3)
    x = synth.activation(SEED + 1, 1004, k, rms=True)
    wb_ref = oracle.f32_to_bf16_rows(w)
    y_ref, den = oracle.gemv_bf16(wb_ref, x)
    wb = torch.empty(n * k, dtype=torch.int16, device="cuda")
    wsg.convert_bf16(dev(w), n * k, wb)
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    wsg.gemv_bf16(wb, n, k, dev(x), y)
    assert_within(host(y), y_ref, oracle.bf16_tolerance(den), f"bf16 {n}x{k}")


def test_repeat_runs_are_bit_identical(gpu_lib):
    import torch
    wsg = gpu_lib
    n, k = 300, 8288  # split-K across two waves: the LDS stage must be race-free
    w, x = _weights(n, k, 4), _act(k, 1006)
    packed = _q8_device(wsg, w)
    xd = dev(x)
    outs = []
    for fmt in (wsg.ACT_F32_REQUANT, wsg.ACT_F32):
        ys = []
        for _ in range(3):
            y = torch.empty(n, dtype=torch.float32, device="cuda")
            wsg.gemv_q8_0(packed, n, k, xd, fmt, y)
            ys.append(host(y).view(np.uint32))
        assert all(np.array_equal(ys[0], v) for v in ys[1:])
        outs.append(ys[0])


def test_identical_rows_give_identical_outputs(gpu_lib):
    """The reduction order does not depend on the row index (needed for
    exact argmax ties between byte-identical rows)."""
    import torch
    wsg = gpu_lib
    n, k = 1000, 4096
    w = _weights(n, k, 5)
    for r in (1, 333, 998, 999):
        w[r] = w[500]
    x = _act(k, 1008)
    packed = _q8_device(wsg, w)
    for fmt in (wsg.ACT_F32_REQUANT, wsg.ACT_F32):
        y = torch.empty(n, dtype=torch.float32, device="cuda")
        wsg.gemv_q8_0(packed, n, k, dev(x), fmt, y)
        yh = host(y)
        assert len({yh[r].tobytes() for r in (1, 333, 500, 998, 999)}) == 1
    wb = torch.empty(n * k, dtype=torch.int16, device="cuda")
    wsg.convert_bf16(dev(w), n * k, wb)
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    wsg.gemv_bf16(wb, n, k, dev(x), y)
    yh = host(y)
    assert len({yh[r].tobytes() for r in (1, 333, 500, 998, 999)}) == 1


def test_concatenated_projections(gpu_lib):
    """q/k/v stacked by rows into one matrix: one launch gives the stacked
    outputs (emit_qwen38_generate, "Where the speed comes from", item 1)."""
    import torch
    wsg = gpu_lib
    k = 4096
    parts = [(_weights(r, k, 10 + 2 * i)) for i, r in enumerate((4096, 1024, 1024))]
    n = sum(p.shape[0] for p in parts)
    rb = wsg.q8_0_row_bytes(k)
    packed = empty_u8(n * rb)
    r0 = 0
    for p in parts:
        wsg.quantize_q8_0_weights(dev(p), p.shape[0], k, packed.data_ptr() + r0 * rb)
        r0 += p.shape[0]
    x = _act(k, 1010)
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    wsg.gemv_q8_0(packed, n, k, dev(x), wsg.ACT_F32_REQUANT, y)
    dw, qw = oracle.quantize_q8_0(np.concatenate(parts))
    dx, qx = oracle.quantize_q8_0(x)
    y_ref, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
    assert_within(host(y), y_ref, oracle.q8_tolerance(den), "concatenated qkv")


def test_empty_and_zero_k(gpu_lib):
    import torch
    wsg = gpu_lib
    y = torch.full((8,), 7.0, dtype=torch.float32, device="cuda")
    x = torch.zeros(64, dtype=torch.float32, device="cuda")
    w = torch.zeros(64, dtype=torch.uint8, device="cuda")
    wsg.gemv_q8_0(w, 0, 64, x, wsg.ACT_F32, y)       # n == 0: nothing written
    assert host(y).tolist() == [7.0] * 8
    wsg.gemv_q8_0(w, 8, 0, x, wsg.ACT_F32, y)        # k == 0: the empty sum
    assert host(y).tolist() == [0.0] * 8
    y.fill_(7.0)
    wsg.gemv_bf16(w, 8, 0, x, y)
    assert host(y).tolist() == [0.0] * 8


def test_max_k_boundaries(gpu_lib):
    import torch
    wsg = gpu_lib
    for k, fmt in ((wsg.MAX_K_Q8ACT, wsg.ACT_F32_REQUANT), (wsg.MAX_K_F32ACT, wsg.ACT_F32)):
        n = 40
        w, x = _weights(n, k, 30), _act(k, 1012)
        dw, qw = oracle.quantize_q8_0(w)
        if fmt == wsg.ACT_F32:
            y_ref, den = oracle.gemv_q8_act_f32(dw, qw, x)
        else:
            dx, qx = oracle.quantize_q8_0(x)
            y_ref, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
        packed = _q8_device(wsg, w)
        y = torch.empty(n, dtype=torch.float32, device="cuda")
        wsg.gemv_q8_0(packed, n, k, dev(x), fmt, y)
        assert_within(host(y), y_ref, oracle.q8_tolerance(den), f"k={k}")
        with pytest.raises(wsg.WsgError):
            wsg.gemv_q8_0(packed, n, k + 32, dev(np.zeros(k + 32, np.float32)), fmt, y)
