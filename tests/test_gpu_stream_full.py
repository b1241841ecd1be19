"""The 27B-scale Q8_0 token stream at full size (64 layers, 256 GEMVs,
26.7 GB of weights) in the configuration bench.py times: the persistent
token plan (emit_qwen38_generate, "Where the speed comes from", items 1-3).

* every one of the 256 outputs of a replay equals the eager calls' output
  bit for bit (same rows, same reduction order), on two consecutive replays;
* sampled rows of GEMVs spread over all 64 layers and all four matrices
  match the oracle computed one row at a time from the GPU's actual input
  of that GEMV (the chain is checked link by link, so no error
  accumulates), at deq 0 (int8 activations, requantized in the stream) and
  deq 2 (f32 activations)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_within, host
from synth import workloads as W

pytestmark = pytest.mark.gpu

WL = W.DENSE27B_Q8
ROWS_PER_GEMV = 6


def _stream(deq):
    import torch

    from weight_streaming_gemv_q8_amd.stream import TokenStream
    ts = TokenStream([(m.n, m.k, m.parts) for m in WL.matrices], WL.layers, WL.wtype, deq=deq)

    def fill(layer, m, part, rows, staging):
        synth.dev_normal_f32(staging.data_ptr(), WL.seed, W.weight_tensor_id(layer, m, part),
                             rows * WL.matrices[m].k, W.WEIGHT_SIGMA,
                             stream=torch.cuda.current_stream().cuda_stream)

    ts.fill_weights(fill)
    xs = np.stack([synth.activation(WL.seed, W.activation_tensor_id(l), WL.matrices[0].k, rms=True)
                   for l in range(WL.layers)])
    ts.set_inputs(torch.from_numpy(xs).cuda())
    return ts, xs


def _weight_rows(layer, j, rows):
    """Host copies of rows of GEMV j of a layer, generated one row at a time."""
    m = WL.matrices[j]
    out = []
    for r in rows:
        part, base = 0, 0
        while r >= base + m.parts[part]:
            base += m.parts[part]
            part += 1
        out.append(synth.normal_f32(WL.seed, W.weight_tensor_id(layer, j, part), m.k, W.WEIGHT_SIGMA,
                                    first=(r - base) * m.k))
    return np.stack(out)


def _sampled_rows(rng, n):
    rows = {0, n - 1} | set(int(v) for v in rng.integers(0, n, ROWS_PER_GEMV - 2))
    return np.array(sorted(rows))


@pytest.mark.parametrize("deq", [0, 2])
def test_full_stream_persistent(gpu_lib, deq):
    ts, xs = _stream(deq)
    ts.run_eager()
    eager = [host(y).view(np.uint32).copy() for y in ts.outputs()]
    for y in ts.outputs():
        y.fill_(np.nan)
    plan = ts.capture(persistent=True)
    assert plan.kernel_count == 1
    for rep in range(2):
        ts.launch()
        got = [host(y) for y in ts.outputs()]
        assert not plan.error()
        for i, (a, b) in enumerate(zip(eager, got)):
            assert np.array_equal(a, b.view(np.uint32)), f"replay {rep}: GEMV {i} differs from eager"

    rng = np.random.default_rng(20261202)
    nm = len(WL.matrices)
    layers = sorted({0, WL.layers - 1} | set(int(v) for v in rng.integers(1, WL.layers - 1, 4)))
    for layer in layers:
        for j, m in enumerate(WL.matrices):
            i = layer * nm + j
            x = xs[layer] if j == 0 else got[i - 1][:m.k]
            rows = _sampled_rows(rng, m.n)
            dw, qw = oracle.quantize_q8_0(_weight_rows(layer, j, rows))
            if deq == 0:
                dx, qx = oracle.quantize_q8_0(np.ascontiguousarray(x, np.float32))
                y_ref, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
            else:
                y_ref, den = oracle.gemv_q8_act_f32(dw, qw, np.ascontiguousarray(x, np.float32))
            assert_within(got[i][rows], y_ref, oracle.q8_tolerance(den), f"layer {layer} GEMV {m.name} rows {rows}")
    ts.close()
