"""The f32-activation (deq 2) forms of the fused GEMVs (emit_qwen38_generate,
"Where the speed comes from", the deq paragraph: deq 2 dequantizes the
weights of every Q8_0 GEMV against f32 activations, removing the
activation quantization error):

* gemv_q8_0_swiglu with f32 activations (the W8A16 dual gate/up projection
  with SwiGLU; GPU Kernel Lab, "Quantization experiments", "Decode
  integration"): each half is reduced as the dequantizing GEMV reduces an
  unsplit row, so the output is silu(g) u of that GEMV's own halves up to
  the epilogue's rounding, and it matches the oracle within the dequant
  bound propagated through the product;
* gemv_q8_0_rmsnorm_f32: the residual add + RMSNorm in the prologue, then
  the dequantizing GEMV on the f32 normalized vector: bit for bit
  residual_rmsnorm_q8_0's y fed to gemv_q8_0 with f32 activations, h_out
  bit for bit the norm call's, and the oracle fed that y;
* a 2-layer chain at deq 2 with the residual stream, fused norms and the
  W8A16 SwiGLU: replay equals eager, and every link matches the oracle fed
  the GPU's own inputs;
* what the 4-bit forms do not run is still rejected."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_within, dev, empty_u8, host
from synth import workloads as W

pytestmark = pytest.mark.gpu

EPS = W.RMSNORM_EPS


@pytest.mark.parametrize("n_ff,k", [(17408, 5120), (12288, 4096), (1000, 2080), (33, 96), (1, 32), (300, 17408)])
def test_w8a16_swiglu(gpu_lib, n_ff, k):
    import torch
    wsg = gpu_lib
    seed = 0x5EEDC000 + n_ff + k
    w = synth.normal_f32(seed, 1, 2 * n_ff * k, 0.02).reshape(2 * n_ff, k)
    packed = empty_u8(wsg.q8_0_packed_bytes(2 * n_ff, k))
    wsg.quantize_q8_0_weights(dev(w), 2 * n_ff, k, packed)
    x = synth.activation(seed, 2, k, rms=True)
    xd = dev(x)
    y = torch.full((n_ff,), np.nan, dtype=torch.float32, device="cuda")
    wsg.gemv_q8_0_swiglu(packed, n_ff, k, xd, wsg.ACT_F32, y)
    full = torch.empty(2 * n_ff, dtype=torch.float32, device="cuda")
    wsg.gemv_q8_0(packed, 2 * n_ff, k, xd, wsg.ACT_F32, full)
    got, gu = host(y).astype(np.float64), host(full).astype(np.float64)
    if wsg.gemv_config(wsg.W_Q8_0, wsg.ACT_F32, 2 * n_ff, k)["split"] == 1:
        g, u = gu[:n_ff], gu[n_ff:]
        assert np.all(np.abs(got - oracle.swiglu(g, u)) <= oracle.swiglu_tolerance(g, u, 0.0, 0.0))
    dw, qw = oracle.quantize_q8_0(w)
    yr, den = oracle.gemv_q8_act_f32(dw, qw, np.ascontiguousarray(x, np.float32))
    t = oracle.q8_tolerance(den)
    tol = oracle.swiglu_tolerance(yr[:n_ff], yr[n_ff:], t[:n_ff], t[n_ff:])
    assert_within(got, oracle.swiglu(yr[:n_ff], yr[n_ff:]), tol, f"W8A16 swiglu {n_ff}x{k}")


@pytest.mark.parametrize("waves", [0, 4, 16])
@pytest.mark.parametrize("n,k", [(300, 1024), (4096, 4096), (2051, 5120), (1000, 8192), (129, 17408),
                                 (64, 36864)])
def test_rmsnorm_f32_equals_norm_then_dequant_gemv(gpu_lib, n, k, waves):
    import torch
    wsg = gpu_lib
    if waves and (n, k) not in ((2051, 5120), (129, 17408)):
        return  # workgroup sizes are swept on two shapes
    wsg.tune(wsg.TUNE_WAVES, waves)
    try:
        seed = 0x5EEDC100 + k
        w = synth.normal_f32(seed, 1, n * k, 0.02).reshape(n, k)
        packed = empty_u8(wsg.q8_0_packed_bytes(n, k))
        wsg.quantize_q8_0_weights(dev(w), n, k, packed)
        h = dev(synth.normal_f32(seed, 2, k, 1.0))
        r = dev(synth.normal_f32(seed, 3, k, 0.5))
        g = dev((np.float32(1.0) + synth.normal_f32(seed, 4, k, 0.1)).astype(np.float32))
        h_ref = torch.empty(k, dtype=torch.float32, device="cuda")
        yn = torch.empty(k, dtype=torch.float32, device="cuda")
        wsg.residual_rmsnorm_q8_0(h, r, g, k, EPS, h_out=h_ref, y=yn)
        y_ref = torch.empty(n, dtype=torch.float32, device="cuda")
        wsg.gemv_q8_0(packed, n, k, yn, wsg.ACT_F32, y_ref)
        y = torch.full((n,), np.nan, dtype=torch.float32, device="cuda")
        h_out = torch.full((k,), np.nan, dtype=torch.float32, device="cuda")
        wsg.gemv_q8_0_rmsnorm_f32(packed, n, k, h, r, g, EPS, y, h_out=h_out)
        got = host(y)
        assert np.array_equal(got.view(np.uint32), host(y_ref).view(np.uint32)), "fused differs from norm + GEMV"
        assert np.array_equal(host(h_out).view(np.uint32), host(h_ref).view(np.uint32)), "h' differs"
        dw, qw = oracle.quantize_q8_0(w)
        yo, den = oracle.gemv_q8_act_f32(dw, qw, host(yn))
        assert_within(got, yo, oracle.q8_tolerance(den), f"rmsnorm_f32 {n}x{k}")
    finally:
        wsg.tune(wsg.TUNE_WAVES, 0)


def test_deq2_rejections(gpu_lib):
    import torch
    wsg = gpu_lib
    packed = empty_u8(wsg.q4_0_packed_bytes(128, 1024))
    x = torch.zeros(1024, dtype=torch.float32, device="cuda")
    y = torch.empty(64, dtype=torch.float32, device="cuda")
    with pytest.raises(wsg.WsgError) as e:
        wsg.gemv_q4_0_swiglu(packed, 64, 1024, x, wsg.ACT_F32, y)
    assert e.value.status == wsg.ERR_MODE
    q8 = empty_u8(wsg.q8_0_packed_bytes(128, 1024))
    with pytest.raises(wsg.WsgError) as e:  # above the f32-activation staging limit
        wsg.gemv_q8_0_rmsnorm_f32(q8, 1, wsg.MAX_K_F32ACT + 32, x, None, None, EPS, y)
    assert e.value.status == wsg.ERR_SHAPE


@pytest.mark.parametrize("wl_name", ["QWEN3_8B_Q8", "DENSE27B_Q8"])
@pytest.mark.parametrize("fused", [False, True])
def test_deq2_chain_with_norms_and_swiglu(gpu_lib, wl_name, fused):
    import torch

    from weight_streaming_gemv_q8_amd.stream import TokenStream
    wsg = gpu_lib
    wl = getattr(W, wl_name)
    layers = 2
    shapes = [(m.n, m.k, m.parts) for m in wl.matrices]
    ts = TokenStream(shapes, layers, "q8_0", deq=2, norm_before=(0, 2), eps=EPS, fused_norm=fused,
                     swiglu_at=(2,))

    def fill(layer, m, part, rows, staging):
        synth.dev_normal_f32(staging.data_ptr(), wl.seed, W.weight_tensor_id(layer, m, part),
                             rows * wl.matrices[m].k, W.WEIGHT_SIGMA, stream=torch.cuda.current_stream().cuda_stream)

    ts.fill_weights(fill)
    hidden = ts.hidden
    h0 = synth.normal_f32(wl.seed, W.RESIDUAL_TENSOR_ID, hidden, 1.0)
    gains = np.stack([np.float32(1.0) + synth.normal_f32(wl.seed, W.gain_tensor_id(i), hidden, W.GAIN_SIGMA)
                      for i in range(len(ts.norms))]).astype(np.float32)
    ts.set_residual_input(torch.from_numpy(h0).cuda(), torch.from_numpy(gains).cuda())
    ops = ts.ops()
    assert not any(o.op == wsg.OP_QUANTIZE_ACT or (o.op == wsg.OP_RESIDUAL_RMSNORM and o.y_q8) for o in ops)
    ts.run_eager()
    eager = [host(y).view(np.uint32).copy() for y in ts.outputs()]
    hs = [host(n.h_out).copy() for n in ts.norms]
    for y in ts.outputs():
        y.fill_(np.nan)
    plan = ts.capture()
    for _ in range(2):
        ts.launch()
        got = [host(y).view(np.uint32).copy() for y in ts.outputs()]
        assert all(np.array_equal(a, b) for a, b in zip(eager, got)), "replay differs from eager"
    outs = [a.view(np.float32) for a in eager]
    # every link against the oracle, fed the GPU's own inputs: the norm in
    # fp64 from the GPU's residual stream, then the dequant GEMV
    rng = np.random.default_rng(0xDE92)
    nm = len(wl.matrices)
    h_in = h0
    for layer in range(layers):
        for j, m in enumerate(wl.matrices):
            i = layer * nm + j
            if j in (0, 2):
                ni = layer * 2 + (0 if j == 0 else 1)
                r = outs[i - 1] if i > 0 else None
                h_gpu, x = oracle.residual_rmsnorm(h_in, r, gains[ni], EPS)
                assert np.array_equal(h_gpu.view(np.uint32), hs[ni].view(np.uint32)), f"layer {layer} h'"
                h_in = hs[ni]
                # the GPU's normalized input is within 2^-16 of the fp64 norm;
                # the GEMV bound is taken on the fp64 one plus that slack
                x32 = x.astype(np.float32)
            else:
                x32 = outs[i - 1][:m.k]
            rows = np.array(sorted(set(int(v) for v in rng.integers(0, m.n // (2 if j == 2 else 1), 24)) | {0}))
            if j == 2:
                nff = m.n // 2
                parts = np.concatenate([rows, rows + nff])
                dw, qw = oracle.quantize_q8_0(_weight_rows(wl, layer, j, parts))
                y, den = oracle.gemv_q8_act_f32(dw, qw, x32)
                t = oracle.q8_tolerance(den) + 2.0 ** -15 * den
                hl = len(rows)
                tol = oracle.swiglu_tolerance(y[:hl], y[hl:], t[:hl], t[hl:])
                assert_within(outs[i][rows].astype(np.float64), oracle.swiglu(y[:hl], y[hl:]), tol,
                              f"layer {layer} W8A16 SwiGLU")
            else:
                dw, qw = oracle.quantize_q8_0(_weight_rows(wl, layer, j, rows))
                y, den = oracle.gemv_q8_act_f32(dw, qw, x32)
                slack = 2.0 ** -15 * den if j == 0 else 0.0
                assert_within(outs[i][rows], y, oracle.q8_tolerance(den) + slack, f"layer {layer} GEMV {m.name}")
    ts.close()


def _weight_rows(wl, layer, j, rows):
    m = wl.matrices[j]
    out = []
    for r in rows:
        part, base = 0, 0
        while r >= base + m.parts[part]:
            base += m.parts[part]
            part += 1
        out.append(synth.normal_f32(wl.seed, W.weight_tensor_id(layer, j, part), m.k, W.WEIGHT_SIGMA,
                                    first=(int(r) - base) * m.k))
    return np.stack(out)
