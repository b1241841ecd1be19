"""The int8 Q8_0 GEMV that computes the residual add + RMSNorm +
re-quantization in its own prologue (gemv_q8_0_rmsnorm; emit_qwen38_generate,
"Where the speed comes from", item 3: the re-quantization fused into the
residual + RMSNorm step of the stream, here inside the consuming GEMV).

* its output equals residual_rmsnorm_q8_0 followed by gemv_q8_0 on that
  call's Q8_0 bytes, bit for bit, and its h_out equals the norm call's,
  across hidden sizes whose norm uses 1-7 units per thread, ragged row
  counts, with and without the residual and the weight, on 4-, 8- and
  16-wave workgroups;
* the output matches the oracle fed the norm call's codes (the chain
  parity rule), on every row;
* a 2-layer 8B- and 27B-shaped chain with the residual stream through every
  layer gives the same buffers fused and unfused, and its graph replay
  equals its eager calls;
* what would race is rejected before launch."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_within, dev, empty_u8, host, split_act_q8
from synth import workloads as W

pytestmark = pytest.mark.gpu

EPS = W.RMSNORM_EPS

CASES = [  # (n, k): k spans 1, 2, 3 and 7 norm units per thread
    (300, 1024), (4096, 4096), (2051, 5120), (1000, 8192), (777, 12288), (129, 17408), (64, 57344),
]


def _inputs(n, k, seed, with_r=True, with_g=True):
    import torch
    w = synth.normal_f32(seed, 1, n * k, 0.02).reshape(n, k)
    packed = torch.empty(_pad(k, n), dtype=torch.uint8, device="cuda")
    import weight_streaming_gemv_q8_amd as wsg
    wsg.quantize_q8_0_weights(dev(w), n, k, packed)
    h = synth.normal_f32(seed, 2, k, 1.0)
    r = synth.normal_f32(seed, 3, k, 0.5) if with_r else None
    g = (np.float32(1.0) + synth.normal_f32(seed, 4, k, 0.1)).astype(np.float32) if with_g else None
    return w, packed, h, r, g


def _pad(k, n):
    import weight_streaming_gemv_q8_amd as wsg
    return wsg.q8_0_packed_bytes(n, k)


def _unfused(wsg, packed, n, k, hd, rd, gd):
    import torch
    h_out = torch.empty(k, dtype=torch.float32, device="cuda")
    yq = empty_u8(wsg.act_q8_0_bytes(k))
    wsg.residual_rmsnorm_q8_0(hd, rd, gd, k, EPS, h_out=h_out, y_q8=yq)
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    wsg.gemv_q8_0(packed, n, k, yq, wsg.ACT_Q8_0, y)
    return host(y), host(h_out), host(yq)


@pytest.mark.parametrize("waves", [0, 4, 16])
@pytest.mark.parametrize("n,k", CASES)
def test_fused_equals_norm_then_gemv(gpu_lib, n, k, waves):
    import torch
    wsg = gpu_lib
    if waves:
        wsg.tune(wsg.TUNE_WAVES, waves)
    try:
        w, packed, h, r, g = _inputs(n, k, 0x5EED9000 + k)
        hd, rd, gd = dev(h), dev(r), dev(g)
        y_ref, h_ref, yq = _unfused(wsg, packed, n, k, hd, rd, gd)
        y = torch.full((n,), np.nan, dtype=torch.float32, device="cuda")
        h_out = torch.full((k,), np.nan, dtype=torch.float32, device="cuda")
        wsg.gemv_q8_0_rmsnorm(packed, n, k, hd, rd, gd, EPS, y, h_out=h_out)
        got = host(y)
        assert np.array_equal(got.view(np.uint32), y_ref.view(np.uint32)), "fused GEMV differs from norm + GEMV"
        assert np.array_equal(host(h_out).view(np.uint32), h_ref.view(np.uint32)), "h' differs"
        if waves == 0:
            # chain parity: the oracle fed the norm call's own codes
            dx, qx = split_act_q8(yq, k)
            dw, qw = oracle.quantize_q8_0(w)
            y_or, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
            assert_within(got, y_or, oracle.q8_tolerance(den), f"{n}x{k} fused GEMV vs oracle")
    finally:
        wsg.tune(wsg.TUNE_WAVES, 0)


@pytest.mark.parametrize("with_r,with_g", [(False, True), (True, False), (False, False)])
def test_fused_without_residual_or_weight(gpu_lib, with_r, with_g):
    import torch
    wsg = gpu_lib
    n, k = 1500, 5120
    _, packed, h, r, g = _inputs(n, k, 0x5EED9100, with_r, with_g)
    hd = dev(h)
    rd = dev(r) if r is not None else None
    gd = dev(g) if g is not None else None
    y_ref, h_ref, _ = _unfused(wsg, packed, n, k, hd, rd, gd)
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    wsg.gemv_q8_0_rmsnorm(packed, n, k, hd, rd, gd, EPS, y)  # no h_out
    assert np.array_equal(host(y).view(np.uint32), y_ref.view(np.uint32))


def test_fused_rejects_racy_buffers(gpu_lib):
    import torch
    wsg = gpu_lib
    n, k = 256, 1024
    _, packed, h, r, g = _inputs(n, k, 0x5EED9200)
    buf = torch.zeros(4 * k, dtype=torch.float32, device="cuda")
    hd, rd, gd = buf[:k], buf[k:2 * k], buf[2 * k:3 * k]
    hd.copy_(dev(h))
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    for h_out, yy in ((hd, y), (rd, y), (gd, y), (buf[3 * k:], hd), (buf[3 * k:], buf[3 * k:3 * k + n])):
        with pytest.raises(wsg.WsgError) as e:
            wsg.gemv_q8_0_rmsnorm(packed, n, k, hd, rd, gd, EPS, yy, h_out=h_out)
        assert e.value.status == wsg.ERR_MODE
    with pytest.raises(wsg.WsgError) as e:
        wsg.gemv_q8_0_rmsnorm(packed, n, k, hd, rd, gd, 0.0, y)
    assert e.value.status == wsg.ERR_MODE


@pytest.mark.parametrize("wl_name", ["QWEN3_8B_Q8", "DENSE27B_Q8"])
def test_fused_chain_equals_unfused_chain(gpu_lib, wl_name):
    import torch

    from weight_streaming_gemv_q8_amd.stream import TokenStream
    wl = getattr(W, wl_name)
    layers = 2
    shapes = [(m.n, m.k, m.parts) for m in wl.matrices]
    got = {}
    for fused in (False, True):
        ts = TokenStream(shapes, layers, "q8_0", deq=0, norm_before=(0, 2), eps=EPS, fused_norm=fused)

        def fill(layer, m, part, rows, staging):
            synth.dev_normal_f32(staging.data_ptr(), wl.seed, W.weight_tensor_id(layer, m, part),
                                 rows * wl.matrices[m].k, W.WEIGHT_SIGMA,
                                 stream=torch.cuda.current_stream().cuda_stream)

        ts.fill_weights(fill)
        hidden = ts.hidden
        h0 = synth.normal_f32(wl.seed, W.RESIDUAL_TENSOR_ID, hidden, 1.0)
        gains = np.stack([np.float32(1.0) + synth.normal_f32(wl.seed, W.gain_tensor_id(i), hidden, W.GAIN_SIGMA)
                          for i in range(len(ts.norms))]).astype(np.float32)
        ts.set_residual_input(torch.from_numpy(h0).cuda(), torch.from_numpy(gains).cuda())
        bufs = [s.y for s in ts.slots] + [n.h_out for n in ts.norms]
        ts.run_eager()
        eager = [host(b).view(np.uint32).copy() for b in bufs]
        for b in bufs:
            b.fill_(np.nan)
        plan = ts.capture()
        assert plan.kernel_count == len(ts.slots) + (0 if fused else len(ts.norms))
        for _ in range(2):
            ts.launch()
            rep = [host(b).view(np.uint32).copy() for b in bufs]
            assert all(np.array_equal(a, b) for a, b in zip(eager, rep)), "replay differs from eager"
        got[fused] = eager
        ts.close()
        del ts
        torch.cuda.empty_cache()
    for i, (a, b) in enumerate(zip(got[False], got[True])):
        assert np.array_equal(a, b), f"buffer {i}: fused chain differs from the unfused chain"
