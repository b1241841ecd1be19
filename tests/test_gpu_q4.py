"""The W4 (4-bit) weight path: quantize_q4_0_weights and gemv_q4_0
(qwen3-8b-rtx4080-cutedsl, "W4A16 dequant-fused GEMM"; GPU Kernel Lab,
"Quantization experiments"; the format is reading R19).

* the device layout decodes to the oracle's scales and codes, bit for bit,
  and the scale sections' padding is zero, on ragged and full chunks;
* the GEMV matches the oracle (the int8 block-dot form over the 4-bit
  codes, or the f32-activation block dot of the W4A16 form) on every row
  within the bound of the matching Q8_0 path, for all three activation
  formats, shapes spanning several chunks and ragged tails,
  one-block and one-row cases, 4-, 8- and 16-wave workgroups and rows
  split over 1, 2 and 4 waves;
* a 2-layer 27B-shaped 4-bit chain (deq 0 and deq 2) replays
  bit-identically to its eager calls and matches the oracle link by link;
* the GEMV with the residual add + RMSNorm + re-quantization in its
  prologue (gemv_q4_0_rmsnorm) equals the norm call followed by the GEMV,
  bit for bit, and a 27B-shaped chain with the residual stream gives the
  same buffers fused and unfused;
* the gate+up GEMV with the SwiGLU epilogue (gemv_q4_0_swiglu) matches
  the plain GEMV's halves and the oracle, alone and in a chain;
* bad arguments are rejected."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_within, dev, empty_u8, host
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _row_bytes(k):
    nb = k // 32
    c = (nb + 63) // 64
    nl = nb - (c - 1) * 64
    return (c - 1) * 1152 + ((2 * nl + 15) // 16) * 16 + 16 * nl


def _decode(buf, n, k):
    """(d fp16 bits [n, k/32], q int8 [n, k], padding bytes) of the 4-bit device layout."""
    rb = _row_bytes(k)
    rows = np.asarray(buf, np.uint8)[: n * rb].reshape(n, rb)
    nb = k // 32
    c_count = (nb + 63) // 64
    d = np.empty((n, nb), np.uint16)
    q = np.empty((n, nb, 32), np.int8)
    pads = []
    for c in range(c_count):
        nbc = min(64, nb - 64 * c)
        sb = ((2 * nbc + 15) // 16) * 16
        base = c * 1152
        d[:, 64 * c:64 * c + nbc] = rows[:, base:base + 2 * nbc].copy().view("<u2")
        pads.append(rows[:, base + 2 * nbc:base + sb])
        codes = rows[:, base + sb:base + sb + 16 * nbc].reshape(n, nbc, 16)
        q[:, 64 * c:64 * c + nbc, :16] = (codes & 0xF).astype(np.int8) - 8
        q[:, 64 * c:64 * c + nbc, 16:] = (codes >> 4).astype(np.int8) - 8
    return d, q.reshape(n, k), np.concatenate([p.reshape(n, -1) for p in pads], axis=1)


@pytest.mark.parametrize("n,k", [(1, 32), (3, 96), (17, 2080), (5, 4096), (2, 17408)])
def test_quantize_q4_weights_bitexact(gpu_lib, n, k):
    wsg = gpu_lib
    assert wsg.q4_0_row_bytes(k) == _row_bytes(k) and wsg.q4_0_packed_bytes(n, k) == n * _row_bytes(k)
    rng = np.random.default_rng(n * 7 + k)
    w = (rng.normal(0, 0.02, (n, k)) * np.exp(rng.normal(0, 1, (n, 1)))).astype(np.float32)
    w[0, :32] = 0.0  # a zero block
    packed = empty_u8(wsg.q4_0_packed_bytes(n, k))
    packed.fill_(0xAB)
    wsg.quantize_q4_0_weights(dev(w), n, k, packed)
    d, q, pad = _decode(host(packed), n, k)
    d_ref, q_ref = oracle.quantize_q4_0(w)
    assert np.array_equal(d, d_ref) and np.array_equal(q, q_ref)
    assert np.all(pad == 0)


def _problem(n, k, seed):
    import weight_streaming_gemv_q8_amd as wsg
    w = synth.normal_f32(seed, 1, n * k, 0.02).reshape(n, k)
    packed = empty_u8(wsg.q4_0_packed_bytes(n, k))
    wsg.quantize_q4_0_weights(dev(w), n, k, packed)
    x = synth.activation(seed, 2, k, outlier_frac=0.01)
    return w, packed, x


@pytest.mark.parametrize("waves,split", [(0, 0), (4, 1), (16, 1), (8, 2), (16, 4)])
@pytest.mark.parametrize("act", ["requant", "q8", "f32"])
@pytest.mark.parametrize("n,k", [(1024, 1024), (1, 32), (257, 5120), (300, 2080), (100, 17408), (4096, 4096)])
def test_gemv_q4(gpu_lib, n, k, act, waves, split):
    import torch
    wsg = gpu_lib
    if (waves or split) and (n, k) not in ((300, 2080), (100, 17408)):
        pytest.skip("workgroup sizes and splits are swept on two ragged shapes")
    wsg.tune(wsg.TUNE_WAVES, waves)
    wsg.tune(wsg.TUNE_SPLITK, split)
    try:
        w, packed, x = _problem(n, k, 0x5EEDC000 + n + k)
        xd = dev(x)
        if act == "q8":
            xq = empty_u8(wsg.act_q8_0_bytes(k))
            wsg.quantize_act_q8_0(xd, k, xq)
            xin, fmt = xq, wsg.ACT_Q8_0
        else:
            xin, fmt = xd, wsg.ACT_F32 if act == "f32" else wsg.ACT_F32_REQUANT
        y = torch.full((n,), np.nan, dtype=torch.float32, device="cuda")
        wsg.gemv_q4_0(packed, n, k, xin, fmt, y)
        dw, qw = oracle.quantize_q4_0(w)
        if act == "f32":
            # the W4A16 form: the 4-bit codes against the f32 activation
            y_ref, den = oracle.gemv_q8_act_f32(dw, qw, x)
        else:
            dx, qx = oracle.quantize_q8_0(x)
            y_ref, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
        assert_within(host(y), y_ref, oracle.q8_tolerance(den), f"W4 {n}x{k} {act} waves {waves} split {split}")
    finally:
        wsg.tune(wsg.TUNE_WAVES, 0)
        wsg.tune(wsg.TUNE_SPLITK, 0)


def test_gemv_q4_rejections(gpu_lib):
    import torch
    wsg = gpu_lib
    _, packed, x = _problem(64, 1024, 0x5EEDC100)
    y = torch.empty(64, dtype=torch.float32, device="cuda")
    with pytest.raises(wsg.WsgError) as e:
        wsg.gemv_q4_0(packed, 64, 1024, dev(x), 7, y)
    assert e.value.status == wsg.ERR_MODE
    with pytest.raises(wsg.WsgError) as e:  # above the f32 path's k
        wsg.gemv_q4_0(packed, 1, 40960, dev(x), wsg.ACT_F32, y)
    assert e.value.status == wsg.ERR_SHAPE
    for n, k in ((0, 1024), (64, 0), (64, 1000)):
        with pytest.raises(wsg.WsgError) as e:
            wsg.gemv_q4_0(packed, n, k, dev(x), wsg.ACT_F32_REQUANT, y)
        assert e.value.status == wsg.ERR_SHAPE


@pytest.mark.parametrize("deq", [0, 2])
def test_q4_chain_27b_shapes(gpu_lib, deq):
    import torch

    from weight_streaming_gemv_q8_amd.stream import TokenStream
    wl = W.DENSE27B_Q8
    layers = 2
    shapes = [(m.n, m.k, m.parts) for m in wl.matrices]
    ts = TokenStream(shapes, layers, "q4_0", deq=deq)

    def fill(layer, m, part, rows, staging):
        synth.dev_normal_f32(staging.data_ptr(), wl.seed, W.weight_tensor_id(layer, m, part),
                             rows * wl.matrices[m].k, W.WEIGHT_SIGMA, stream=torch.cuda.current_stream().cuda_stream)

    ts.fill_weights(fill)
    xs = np.stack([synth.activation(wl.seed, W.activation_tensor_id(l), shapes[0][1], rms=True)
                   for l in range(layers)])
    ts.set_inputs(torch.from_numpy(xs).cuda())
    ts.run_eager()
    eager = [host(y).view(np.uint32).copy() for y in ts.outputs()]
    for y in ts.outputs():
        y.fill_(np.nan)
    plan = ts.capture()
    assert plan.kernel_count == len(ts.slots)
    ts.launch()
    got = [host(y).view(np.uint32).copy() for y in ts.outputs()]
    assert all(np.array_equal(a, b) for a, b in zip(eager, got)), "replay differs from eager"
    outs = [a.view(np.float32) for a in eager]
    rng = np.random.default_rng(0xC4)
    for layer in range(layers):
        for j, m in enumerate(wl.matrices):
            i = layer * len(wl.matrices) + j
            x = xs[layer] if j == 0 else outs[i - 1][:m.k]
            rows = np.array(sorted(set(int(v) for v in rng.integers(0, m.n, 40)) | {0, m.n - 1}))
            wr = []
            for r in rows:
                part, base = 0, 0
                while r >= base + m.parts[part]:
                    base += m.parts[part]
                    part += 1
                wr.append(synth.normal_f32(wl.seed, W.weight_tensor_id(layer, j, part), m.k, W.WEIGHT_SIGMA,
                                           first=(int(r) - base) * m.k))
            dw, qw = oracle.quantize_q4_0(np.stack(wr))
            if deq == 2:
                y_ref, den = oracle.gemv_q8_act_f32(dw, qw, np.ascontiguousarray(x, np.float32))
            else:
                dx, qx = oracle.quantize_q8_0(np.ascontiguousarray(x, np.float32))
                y_ref, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
            assert_within(outs[i][rows], y_ref, oracle.q8_tolerance(den), f"layer {layer} W4 GEMV {j}")
    ts.close()


@pytest.mark.parametrize("waves", [0, 4, 16])
@pytest.mark.parametrize("n,k", [(300, 1024), (2051, 5120), (777, 12288), (129, 17408)])
def test_q4_fused_norm_equals_norm_then_gemv(gpu_lib, n, k, waves):
    """gemv_q4_0_rmsnorm: bit for bit residual_rmsnorm_q8_0 followed by
    gemv_q4_0 on that call's codes, h_out included; the output within the
    int8 path's bound of the oracle fed those codes."""
    import torch
    from gpu_util import split_act_q8
    wsg = gpu_lib
    eps = W.RMSNORM_EPS
    wsg.tune(wsg.TUNE_WAVES, waves)
    try:
        w, packed, _ = _problem(n, k, 0x5EEDC200 + k)
        h = synth.normal_f32(0x5EEDC200 + k, 3, k, 1.0)
        r = synth.normal_f32(0x5EEDC200 + k, 4, k, 0.5)
        g = (np.float32(1.0) + synth.normal_f32(0x5EEDC200 + k, 5, k, 0.1)).astype(np.float32)
        hd, rd, gd = dev(h), dev(r), dev(g)
        h_ref = torch.empty(k, dtype=torch.float32, device="cuda")
        yq = empty_u8(wsg.act_q8_0_bytes(k))
        wsg.residual_rmsnorm_q8_0(hd, rd, gd, k, eps, h_out=h_ref, y_q8=yq)
        y_ref = torch.empty(n, dtype=torch.float32, device="cuda")
        wsg.gemv_q4_0(packed, n, k, yq, wsg.ACT_Q8_0, y_ref)
        y = torch.full((n,), np.nan, dtype=torch.float32, device="cuda")
        h_out = torch.full((k,), np.nan, dtype=torch.float32, device="cuda")
        wsg.gemv_q4_0_rmsnorm(packed, n, k, hd, rd, gd, eps, y, h_out=h_out)
        got = host(y)
        assert np.array_equal(got.view(np.uint32), host(y_ref).view(np.uint32)), "fused differs from norm + GEMV"
        assert np.array_equal(host(h_out).view(np.uint32), host(h_ref).view(np.uint32)), "h' differs"
        dx, qx = split_act_q8(host(yq), k)
        dw, qw = oracle.quantize_q4_0(w)
        y_or, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
        assert_within(got, y_or, oracle.q8_tolerance(den), f"W4 fused norm {n}x{k}")
    finally:
        wsg.tune(wsg.TUNE_WAVES, 0)


def test_q4_fused_norm_rejects_racy_buffers(gpu_lib):
    import torch
    wsg = gpu_lib
    n, k = 256, 1024
    _, packed, _ = _problem(n, k, 0x5EEDC300)
    buf = torch.zeros(4 * k, dtype=torch.float32, device="cuda")
    hd, rd, gd = buf[:k], buf[k:2 * k], buf[2 * k:3 * k]
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    for h_out, yy in ((hd, y), (rd, y), (buf[3 * k:], hd)):
        with pytest.raises(wsg.WsgError) as e:
            wsg.gemv_q4_0_rmsnorm(packed, n, k, hd, rd, gd, W.RMSNORM_EPS, yy, h_out=h_out)
        assert e.value.status == wsg.ERR_MODE


def test_q4_fused_chain_equals_unfused_chain(gpu_lib):
    """A 2-layer 27B-shaped 4-bit chain carrying the residual stream (norm
    before GEMVs 0 and 2): fused and unfused give the same buffers, and
    each graph replay equals its eager calls."""
    import torch

    from weight_streaming_gemv_q8_amd.stream import TokenStream
    wl = W.DENSE27B_Q8
    layers = 2
    shapes = [(m.n, m.k, m.parts) for m in wl.matrices]
    got = {}
    for fused in (False, True):
        ts = TokenStream(shapes, layers, "q4_0", deq=0, norm_before=(0, 2), eps=W.RMSNORM_EPS, fused_norm=fused)

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
        ts.launch()
        rep = [host(b).view(np.uint32).copy() for b in bufs]
        assert all(np.array_equal(a, b) for a, b in zip(eager, rep)), "replay differs from eager"
        got[fused] = eager
        ts.close()
        del ts
        torch.cuda.empty_cache()
    for i, (a, b) in enumerate(zip(got[False], got[True])):
        assert np.array_equal(a, b), f"buffer {i}: fused chain differs from the unfused chain"


def _w_rows(wl, layer, j, rows):
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


@pytest.mark.parametrize("waves", [0, 4])
@pytest.mark.parametrize("act", ["requant", "q8"])
@pytest.mark.parametrize("n_ff,k", [(17408, 5120), (1000, 2080), (33, 96), (1, 32)])
def test_q4_swiglu_gemv(gpu_lib, n_ff, k, act, waves):
    """gemv_q4_0_swiglu: silu(g) u of the plain 4-bit GEMV's own halves
    within the epilogue's rounding, and the oracle (both halves in fp64,
    then SwiGLU) within the two GEMV bounds carried through the product."""
    import torch
    wsg = gpu_lib
    if waves and (n_ff, k) != (1000, 2080):
        pytest.skip("workgroup sizes are swept on one ragged shape")
    wsg.tune(wsg.TUNE_WAVES, waves)
    try:
        w, packed, x = _problem(2 * n_ff, k, 0x5EEDC400 + n_ff + k)
        xd = dev(x)
        if act == "q8":
            xq = empty_u8(wsg.act_q8_0_bytes(k))
            wsg.quantize_act_q8_0(xd, k, xq)
            xin, fmt = xq, wsg.ACT_Q8_0
        else:
            xin, fmt = xd, wsg.ACT_F32_REQUANT
        y = torch.full((n_ff,), np.nan, dtype=torch.float32, device="cuda")
        wsg.gemv_q4_0_swiglu(packed, n_ff, k, xin, fmt, y)
        full = torch.empty(2 * n_ff, dtype=torch.float32, device="cuda")
        wsg.gemv_q4_0(packed, 2 * n_ff, k, xin, fmt, full)
        got, gu = host(y).astype(np.float64), host(full).astype(np.float64)
        g, u = gu[:n_ff], gu[n_ff:]
        assert np.all(np.abs(got - oracle.swiglu(g, u)) <= oracle.swiglu_tolerance(g, u, 0.0, 0.0)), \
            "epilogue of the plain GEMV's halves"
        dw, qw = oracle.quantize_q4_0(w)
        dx, qx = oracle.quantize_q8_0(x)
        yr, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
        t = oracle.q8_tolerance(den)
        tol = oracle.swiglu_tolerance(yr[:n_ff], yr[n_ff:], t[:n_ff], t[n_ff:])
        assert_within(got, oracle.swiglu(yr[:n_ff], yr[n_ff:]), tol, f"W4 swiglu {n_ff}x{k} {act}")
    finally:
        wsg.tune(wsg.TUNE_WAVES, 0)


def test_q4_swiglu_pair_paths(gpu_lib):
    """The two ways the wave pairs of gemv_q4_0_swiglu meet (halves kept in
    LDS until after the row loop, or a meeting at the end of every tile when
    a workgroup has more tiles than LDS keeps: forced here with 4-wave
    workgroups, one per CU) give the same outputs bit for bit, equal to the
    epilogue applied to the plain GEMV's halves."""
    import torch
    wsg = gpu_lib
    n_ff, k = 17408, 5120
    w, packed, x = _problem(2 * n_ff, k, 0x5EEDC600)
    xd = dev(x)
    outs = []
    try:
        for waves, wgpc in ((0, 0), (4, 1)):
            wsg.tune(wsg.TUNE_WAVES, waves)
            wsg.tune(wsg.TUNE_WG_PER_CU, wgpc)
            y = torch.full((n_ff,), np.nan, dtype=torch.float32, device="cuda")
            wsg.gemv_q4_0_swiglu(packed, n_ff, k, xd, wsg.ACT_F32_REQUANT, y)
            outs.append(host(y).view(np.uint32).copy())
        full = torch.empty(2 * n_ff, dtype=torch.float32, device="cuda")
        wsg.gemv_q4_0(packed, 2 * n_ff, k, xd, wsg.ACT_F32_REQUANT, full)
    finally:
        wsg.tune(wsg.TUNE_WAVES, 0)
        wsg.tune(wsg.TUNE_WG_PER_CU, 0)
    assert np.array_equal(outs[0], outs[1]), "kept halves vs per-tile meeting"
    gu = host(full).astype(np.float64)
    got = outs[0].view(np.float32).astype(np.float64)
    g, u = gu[:n_ff], gu[n_ff:]
    assert np.all(np.abs(got - oracle.swiglu(g, u)) <= oracle.swiglu_tolerance(g, u, 0.0, 0.0))


def test_q4_swiglu_rejections(gpu_lib):
    import torch
    wsg = gpu_lib
    _, packed, x = _problem(128, 1024, 0x5EEDC500)
    y = torch.empty(64, dtype=torch.float32, device="cuda")
    with pytest.raises(wsg.WsgError) as e:
        wsg.gemv_q4_0_swiglu(packed, 64, 1024, dev(x), wsg.ACT_F32, y)
    assert e.value.status == wsg.ERR_MODE
    for n_ff, k in ((0, 1024), (64, 1000)):
        with pytest.raises(wsg.WsgError) as e:
            wsg.gemv_q4_0_swiglu(packed, n_ff, k, dev(x), wsg.ACT_F32_REQUANT, y)
        assert e.value.status == wsg.ERR_SHAPE


def test_q4_swiglu_chain_27b_shapes(gpu_lib):
    """A 2-layer 27B-shaped 4-bit chain whose down projection reads the
    SwiGLU outputs: replays equal the eager calls; the SwiGLU link and the
    down projection match the oracle fed the GPU's own inputs."""
    import torch

    from weight_streaming_gemv_q8_amd.stream import TokenStream
    wl = W.DENSE27B_Q8
    layers = 2
    shapes = [(m.n, m.k, m.parts) for m in wl.matrices]
    ts = TokenStream(shapes, layers, "q4_0", deq=0, swiglu_at=(2,))

    def fill(layer, m, part, rows, staging):
        synth.dev_normal_f32(staging.data_ptr(), wl.seed, W.weight_tensor_id(layer, m, part),
                             rows * wl.matrices[m].k, W.WEIGHT_SIGMA, stream=torch.cuda.current_stream().cuda_stream)

    ts.fill_weights(fill)
    xs = np.stack([synth.activation(wl.seed, W.activation_tensor_id(l), shapes[0][1], rms=True)
                   for l in range(layers)])
    ts.set_inputs(torch.from_numpy(xs).cuda())
    ts.run_eager()
    eager = [host(y).view(np.uint32).copy() for y in ts.outputs()]
    for y in ts.outputs():
        y.fill_(np.nan)
    plan = ts.capture()
    assert plan.kernel_count == len(ts.slots)
    ts.launch()
    got = [host(y).view(np.uint32).copy() for y in ts.outputs()]
    assert all(np.array_equal(a, b) for a, b in zip(eager, got)), "replay differs from eager"
    outs = [a.view(np.float32) for a in eager]
    rng = np.random.default_rng(0xC5)
    for layer in range(layers):
        for j in (2, 3):
            m = wl.matrices[j]
            i = layer * len(wl.matrices) + j
            dx, qx = oracle.quantize_q8_0(np.ascontiguousarray(outs[i - 1][:m.k], np.float32))
            if j == 2:
                nff = m.n // 2
                rows = np.array(sorted(set(int(v) for v in rng.integers(0, nff, 32)) | {0, nff - 1}))
                dw, qw = oracle.quantize_q4_0(_w_rows(wl, layer, j, np.concatenate([rows, rows + nff])))
                yr, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
                t = oracle.q8_tolerance(den)
                h = len(rows)
                tol = oracle.swiglu_tolerance(yr[:h], yr[h:], t[:h], t[h:])
                assert_within(outs[i][rows].astype(np.float64), oracle.swiglu(yr[:h], yr[h:]), tol,
                              f"layer {layer} W4 gate+up SwiGLU")
            else:
                rows = np.array(sorted(set(int(v) for v in rng.integers(0, m.n, 32)) | {0, m.n - 1}))
                dw, qw = oracle.quantize_q4_0(_w_rows(wl, layer, j, rows))
                yr, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
                assert_within(outs[i][rows], yr, oracle.q8_tolerance(den), f"layer {layer} W4 down")
    ts.close()
