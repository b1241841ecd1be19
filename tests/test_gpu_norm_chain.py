"""The token chain with the residual stream between its GEMVs: before the
attention input (GEMV 0) and the MLP input (GEMV 2) of every layer, one
residual_rmsnorm_q8_0 call adds the previous GEMV's output to the residual
stream, normalizes it and re-quantizes it for the next GEMV
(emit_qwen38_generate, "Where the speed comes from", item 3; GPU Kernel Lab,
"Decode integration": residual + RMSNorm across the layer boundaries).
Layers now depend on each other through the data, not only through stream
order.

* graph replay == eager calls, bit for bit, for every buffer of the chain,
  on two consecutive replays;
* link by link against the oracle, each call fed the GPU's actual inputs
  (so no error accumulates): every norm's residual stream bit-exact, its
  normalized vector within 2^-16 relative, its Q8_0 bytes bit-exact against
  the rule applied to that vector; every GEMV within the per-row bounds."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_within, host, split_act_q8
from synth import workloads as W

pytestmark = pytest.mark.gpu

NORM_BEFORE = (0, 2)
Y_REL_TOL = 2.0 ** -16


def _chain(wl, layers, deq):
    import torch

    from weight_streaming_gemv_q8_amd.stream import TokenStream
    ts = TokenStream([(m.n, m.k, m.parts) for m in wl.matrices], layers, wl.wtype, deq=deq,
                     norm_before=NORM_BEFORE, eps=W.RMSNORM_EPS)

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
    return ts, h0, gains


def _buffers(ts):
    out = [s.y for s in ts.slots]
    for n in ts.norms:
        out += [n.h_out, n.y] + ([n.yq] if n.yq is not None else [])
    return out


def _snapshot(ts):
    return [host(b).view(np.uint8).copy() for b in _buffers(ts)]


def _weights_host(wl, layer, j):
    m = wl.matrices[j]
    parts = [synth.normal_f32(wl.seed, W.weight_tensor_id(layer, j, p), rows * m.k, W.WEIGHT_SIGMA)
             .reshape(rows, m.k) for p, rows in enumerate(m.parts)]
    return np.concatenate(parts, axis=0)


def _check_links(ts, wl, h0, gains, deq):
    k_hidden = ts.hidden
    norm_i = 0
    for i, s in enumerate(ts.slots):
        if s.norm is not None:
            n = s.norm
            h_in = h0 if norm_i == 0 else host(ts.norms[norm_i - 1].h_out)
            r = host(ts.slots[i - 1].y) if i > 0 else None
            h_ref, y_ref = oracle.residual_rmsnorm(h_in, r, gains[norm_i], W.RMSNORM_EPS)
            h_gpu, y_gpu = host(n.h_out), host(n.y)
            assert np.array_equal(h_gpu.view(np.uint32), h_ref.view(np.uint32)), f"norm {norm_i}: h'"
            err = np.abs(y_gpu.astype(np.float64) - y_ref)
            assert (err <= Y_REL_TOL * np.abs(y_ref)).all(), f"norm {norm_i}: y"
            x = y_gpu
            if n.yq is not None:
                d_gpu, q_gpu = split_act_q8(host(n.yq), k_hidden)
                d_ref, q_ref = oracle.quantize_q8_0(y_gpu)
                assert np.array_equal(d_gpu, d_ref) and np.array_equal(q_gpu, q_ref), f"norm {norm_i}: Q8_0"
            norm_i += 1
        else:
            x = host(ts.slots[i - 1].y)[:s.k]
        w = _weights_host(wl, s.layer, s.index)
        what = f"layer {s.layer} GEMV {s.index}"
        if wl.wtype == "bf16":
            y_ref, den = oracle.gemv_bf16(oracle.f32_to_bf16_rows(w), x)
            assert_within(host(s.y), y_ref, oracle.bf16_tolerance(den), what)
            continue
        dw, qw = oracle.quantize_q8_0(w)
        if deq == 2:
            y_ref, den = oracle.gemv_q8_act_f32(dw, qw, np.ascontiguousarray(x, np.float32))
        else:
            dx, qx = oracle.quantize_q8_0(np.ascontiguousarray(x, np.float32))
            y_ref, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
        assert_within(host(s.y), y_ref, oracle.q8_tolerance(den), what)


@pytest.mark.parametrize("wl_name,deq", [("QWEN3_8B_Q8", 0), ("QWEN3_8B_Q8", 2), ("QWEN3_0P6B_BF16", 0)])
def test_norm_chain_replay_and_oracle(gpu_lib, wl_name, deq):
    wl = getattr(W, wl_name)
    layers = 2
    ts, h0, gains = _chain(wl, layers, deq)
    assert len(ts.norms) == layers * len(NORM_BEFORE)
    ts.run_eager()
    eager = _snapshot(ts)
    for b in _buffers(ts):
        b.fill_(np.nan if b.dtype.is_floating_point else 0xFF)
    plan = ts.capture()
    assert plan.kernel_count == len(ts.slots) + len(ts.norms)
    for rep in range(2):
        ts.launch()
        got = _snapshot(ts)
        for j, (a, b) in enumerate(zip(eager, got)):
            assert np.array_equal(a, b), f"replay {rep}: buffer {j} differs from eager"
    _check_links(ts, wl, h0, gains, deq)
    ts.close()
