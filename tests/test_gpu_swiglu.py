"""The gate+up GEMV with its SwiGLU epilogue (gemv_q8_0_swiglu; GPU Kernel
Lab, "What we built", "Decode integration": the dual gate/up projection
fused with SwiGLU at batch 1).

* the fused output matches silu(g) u of the plain GEMV's own gate and up
  outputs (which the fused kernel reduces in the same order) within the
  fp32 epilogue's rounding;
* it matches the oracle (both halves in fp64, then SwiGLU) within the two
  GEMV bounds propagated through the product, on every output, for the
  27B and 8B gate+up shapes, ragged shapes, one-output and one-block
  cases, both int8 activation formats, on 4-, 8- and 16-wave workgroups;
* a 2-layer chain whose down projection reads the SwiGLU outputs replays
  bit-identically to its eager calls, and every link matches the oracle
  fed the GPU's own inputs;
* what it does not run is rejected.  (The f32-activation W8A16 form is
  tested in test_gpu_deq2.py.)"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_within, dev, empty_u8, host
from synth import workloads as W

pytestmark = pytest.mark.gpu

CASES = [(17408, 5120), (12288, 4096), (1000, 2080), (33, 96), (1, 32), (300, 12288)]


def _problem(n_ff, k, seed):
    import weight_streaming_gemv_q8_amd as wsg
    w = synth.normal_f32(seed, 1, 2 * n_ff * k, 0.02).reshape(2 * n_ff, k)
    packed = empty_u8(wsg.q8_0_packed_bytes(2 * n_ff, k))
    wsg.quantize_q8_0_weights(dev(w), 2 * n_ff, k, packed)
    x = synth.activation(seed, 2, k, rms=True)
    return w, packed, x


def _oracle(w, x, n_ff):
    dw, qw = oracle.quantize_q8_0(w)
    dx, qx = oracle.quantize_q8_0(np.ascontiguousarray(x, np.float32))
    y, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
    tol = oracle.q8_tolerance(den)
    return y[:n_ff], y[n_ff:], tol[:n_ff], tol[n_ff:]


@pytest.mark.parametrize("waves", [0, 4, 16])
@pytest.mark.parametrize("act", ["requant", "q8"])
@pytest.mark.parametrize("n_ff,k", CASES)
def test_swiglu_gemv(gpu_lib, n_ff, k, act, waves):
    import torch
    wsg = gpu_lib
    if waves and (n_ff, k) not in ((1000, 2080), (17408, 5120)):
        pytest.skip("workgroup sizes are swept on two shapes")
    wsg.tune(wsg.TUNE_WAVES, waves)
    try:
        w, packed, x = _problem(n_ff, k, 0x5EEDA000 + k + n_ff)
        xd = dev(x)
        if act == "q8":
            xq = empty_u8(wsg.act_q8_0_bytes(k))
            wsg.quantize_act_q8_0(xd, k, xq)
            xin, fmt = xq, wsg.ACT_Q8_0
        else:
            xin, fmt = xd, wsg.ACT_F32_REQUANT
        y = torch.full((n_ff,), np.nan, dtype=torch.float32, device="cuda")
        wsg.gemv_q8_0_swiglu(packed, n_ff, k, xin, fmt, y)
        full = torch.empty(2 * n_ff, dtype=torch.float32, device="cuda")
        wsg.gemv_q8_0(packed, 2 * n_ff, k, xin, fmt, full)
        got, gu = host(y).astype(np.float64), host(full).astype(np.float64)
        if wsg.gemv_config(wsg.W_Q8_0, fmt, 2 * n_ff, k)["split"] == 1:
            # same reduction of both halves: only the epilogue's rounding
            g, u = gu[:n_ff], gu[n_ff:]
            tol0 = oracle.swiglu_tolerance(g, u, 0.0, 0.0)
            assert np.all(np.abs(got - oracle.swiglu(g, u)) <= tol0), "epilogue of the plain GEMV's halves"
        g_ref, u_ref, tg, tu = _oracle(w, x, n_ff)
        tol = oracle.swiglu_tolerance(g_ref, u_ref, tg, tu)
        assert_within(got, oracle.swiglu(g_ref, u_ref), tol, f"swiglu {n_ff}x{k} {act}")
    finally:
        wsg.tune(wsg.TUNE_WAVES, 0)


def test_swiglu_rejections(gpu_lib):
    import torch
    wsg = gpu_lib
    _, packed, x = _problem(64, 1024, 0x5EEDA100)
    y = torch.empty(64, dtype=torch.float32, device="cuda")
    with pytest.raises(wsg.WsgError) as e:  # not an activation format
        wsg.gemv_q8_0_swiglu(packed, 64, 1024, dev(x), 7, y)
    assert e.value.status == wsg.ERR_MODE
    for n_ff, k in ((0, 1024), (64, 0), (64, 1000)):
        with pytest.raises(wsg.WsgError) as e:
            wsg.gemv_q8_0_swiglu(packed, n_ff, k, dev(x), wsg.ACT_F32_REQUANT, y)
        assert e.value.status == wsg.ERR_SHAPE


@pytest.mark.parametrize("wl_name", ["QWEN3_8B_Q8", "DENSE27B_Q8"])
def test_swiglu_chain(gpu_lib, wl_name):
    import torch

    from weight_streaming_gemv_q8_amd.stream import TokenStream
    wl = getattr(W, wl_name)
    layers = 2
    shapes = [(m.n, m.k, m.parts) for m in wl.matrices]
    ts = TokenStream(shapes, layers, "q8_0", deq=0, swiglu_at=(2,))

    def fill(layer, m, part, rows, staging):
        synth.dev_normal_f32(staging.data_ptr(), wl.seed, W.weight_tensor_id(layer, m, part),
                             rows * wl.matrices[m].k, W.WEIGHT_SIGMA, stream=torch.cuda.current_stream().cuda_stream)

    ts.fill_weights(fill)
    xs = np.stack([synth.activation(wl.seed, W.activation_tensor_id(l), shapes[0][1], rms=True)
                   for l in range(layers)])
    ts.set_inputs(torch.from_numpy(xs).cuda())
    assert ts.slots[2].y.numel() == shapes[2][0] // 2 == shapes[3][1]
    ts.run_eager()
    eager = [host(y).view(np.uint32).copy() for y in ts.outputs()]
    for y in ts.outputs():
        y.fill_(np.nan)
    plan = ts.capture()
    assert plan.kernel_count == len(ts.slots)
    for _ in range(2):
        ts.launch()
        got = [host(y).view(np.uint32).copy() for y in ts.outputs()]
        assert all(np.array_equal(a, b) for a, b in zip(eager, got)), "replay differs from eager"
    outs = [a.view(np.float32) for a in eager]
    rng = np.random.default_rng(0xA11)
    for layer in range(layers):
        for j, m in enumerate(wl.matrices):
            i = layer * len(wl.matrices) + j
            x = xs[layer] if j == 0 else outs[i - 1][:m.k]
            dx, qx = oracle.quantize_q8_0(np.ascontiguousarray(x, np.float32))
            if j == 2:
                nff = m.n // 2
                rows = np.array(sorted(set(int(v) for v in rng.integers(0, nff, 48)) | {0, nff - 1}))
                parts = np.concatenate([rows, rows + nff])
                wr = _weight_rows(wl, layer, j, parts)
                dw, qw = oracle.quantize_q8_0(wr)
                y, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
                t = oracle.q8_tolerance(den)
                h = len(rows)
                tol = oracle.swiglu_tolerance(y[:h], y[h:], t[:h], t[h:])
                assert_within(outs[i][rows].astype(np.float64), oracle.swiglu(y[:h], y[h:]), tol,
                              f"layer {layer} gate+up SwiGLU")
            else:
                rows = np.array(sorted(set(int(v) for v in rng.integers(0, m.n, 48)) | {0, m.n - 1}))
                dw, qw = oracle.quantize_q8_0(_weight_rows(wl, layer, j, rows))
                y, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
                assert_within(outs[i][rows], y, oracle.q8_tolerance(den), f"layer {layer} GEMV {j}")
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
