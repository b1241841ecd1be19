"""The token streams at their full length, in the plans bench.py times
(emit_qwen38_generate, "Where the speed comes from", items 1-3; GPU Kernel
Lab, "Decode integration": fixed-address graph replay checked against eager
execution):

* the 27B-scale Q8_0 stream (64 layers, 256 GEMVs, 26.7 GB) in the graph
  plan (one node per GEMV) and the persistent plan, at deq 0 (int8
  activations requantized in each GEMV) and deq 2 (f32 activations);
* the Qwen3-8B-shaped Q8_0 stream (36 layers, 144 GEMVs) in the graph plan
  at deq 0 and deq 2;
* the Qwen3-0.6B-shaped BF16 stream (28 layers, 112 GEMVs) in the graph
  plan.

For each: two replays with different layer inputs; every output of each
replay equals the eager calls on those inputs bit for bit (same rows, same
reduction order), and sampled rows of GEMVs spread over the layers and all
four matrices match the oracle computed one row at a time from the GPU's
actual input of that GEMV (the chain is checked link by link, so no error
accumulates)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_within, host
from synth import workloads as W

pytestmark = pytest.mark.gpu

ROWS_PER_GEMV = 6
CASES = [
    ("dense27b_q8_0_64L", "graph", 0), ("dense27b_q8_0_64L", "graph", 2),
    ("dense27b_q8_0_64L", "persistent", 0), ("dense27b_q8_0_64L", "persistent", 2),
    ("qwen3_8b_q8_0_36L", "graph", 0), ("qwen3_8b_q8_0_36L", "graph", 2),
    ("qwen3_0.6b_bf16_28L", "graph", 0),
]


def _stream(wl, deq):
    import torch

    from weight_streaming_gemv_q8_amd.stream import TokenStream
    ts = TokenStream([(m.n, m.k, m.parts) for m in wl.matrices], wl.layers, wl.wtype, deq=deq)

    def fill(layer, m, part, rows, staging):
        synth.dev_normal_f32(staging.data_ptr(), wl.seed, W.weight_tensor_id(layer, m, part),
                             rows * wl.matrices[m].k, W.WEIGHT_SIGMA,
                             stream=torch.cuda.current_stream().cuda_stream)

    ts.fill_weights(fill)
    return ts


def _inputs(ts, wl, seed):
    import torch
    xs = np.stack([synth.activation(seed, W.activation_tensor_id(l), wl.matrices[0].k, rms=True)
                   for l in range(wl.layers)])
    ts.set_inputs(torch.from_numpy(xs).cuda())
    return xs


def _weight_rows(wl, layer, j, rows):
    """Host copies of rows of GEMV j of a layer, generated one row at a time."""
    m = wl.matrices[j]
    out = []
    for r in rows:
        part, base = 0, 0
        while r >= base + m.parts[part]:
            base += m.parts[part]
            part += 1
        out.append(synth.normal_f32(wl.seed, W.weight_tensor_id(layer, j, part), m.k, W.WEIGHT_SIGMA,
                                    first=(r - base) * m.k))
    return np.stack(out)


def _sampled_rows(rng, n):
    rows = {0, n - 1} | set(int(v) for v in rng.integers(0, n, ROWS_PER_GEMV - 2))
    return np.array(sorted(rows))


def _check_against_oracle(wl, deq, xs, got, rng):
    nm = len(wl.matrices)
    layers = sorted({0, wl.layers - 1} | set(int(v) for v in rng.integers(1, wl.layers - 1, 4)))
    for layer in layers:
        for j, m in enumerate(wl.matrices):
            i = layer * nm + j
            x = np.ascontiguousarray(xs[layer] if j == 0 else got[i - 1][:m.k], np.float32)
            rows = _sampled_rows(rng, m.n)
            w = _weight_rows(wl, layer, j, rows)
            if wl.wtype == "bf16":
                y_ref, den = oracle.gemv_bf16(oracle.f32_to_bf16_rows(w), x)
                tol = oracle.bf16_tolerance(den)
            else:
                dw, qw = oracle.quantize_q8_0(w)
                if deq == 0:
                    dx, qx = oracle.quantize_q8_0(x)
                    y_ref, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
                else:
                    y_ref, den = oracle.gemv_q8_act_f32(dw, qw, x)
                tol = oracle.q8_tolerance(den)
            assert_within(got[i][rows], y_ref, tol, f"{wl.name} layer {layer} GEMV {m.name} rows {rows}")


@pytest.mark.parametrize("wl_name,plan_kind,deq", CASES)
def test_full_stream(gpu_lib, wl_name, plan_kind, deq):
    wl = {w.name: w for w in W.ALL}[wl_name]
    ts = _stream(wl, deq)
    plan = ts.capture(persistent=plan_kind == "persistent")
    assert plan.kernel_count == (1 if plan_kind == "persistent" else wl.layers * len(wl.matrices))
    rng = np.random.default_rng(20261203 + deq)
    for rep, seed in enumerate((wl.seed, wl.seed + 0x100)):
        xs = _inputs(ts, wl, seed)
        ts.run_eager()
        eager = [host(y).view(np.uint32).copy() for y in ts.outputs()]
        for y in ts.outputs():
            y.fill_(np.nan)
        ts.launch()
        got = [host(y) for y in ts.outputs()]
        if plan_kind == "persistent":
            assert not plan.error()
        for i, (a, b) in enumerate(zip(eager, got)):
            assert np.array_equal(a, b.view(np.uint32)), f"replay {rep}: GEMV {i} differs from eager"
        _check_against_oracle(wl, deq, xs, got, rng)
    ts.close()
