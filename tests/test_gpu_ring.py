"""The LDS-ring whole-token plan (emit_qwen38_generate, "Where the speed
comes from", items 1-3: the weight stream must not stall between GEMVs).

* every GEMV of a replay matches the oracle fed the GPU's actual input of
  that GEMV (the chain is checked link by link), at deq 0, on sampled rows
  of the 8B- and 27B-shaped streams and on every row of small ragged
  chains (rows not a multiple of the grid, workgroups with no rows, ragged
  last chunks, one-block rows);
* GEMVs whose eager call does not split rows across waves are reduced in
  the same order, so they equal the eager calls bit for bit;
* two replays agree bit for bit (the slot handshakes leave no race), for
  every producer count, and no wait gave up;
* what the ring does not run is rejected before anything is launched."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_within, host
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _chain(shapes, layers, seed, deq=0):
    import torch

    from weight_streaming_gemv_q8_amd.stream import TokenStream
    ts = TokenStream([(n, k, parts) for n, k, parts in shapes], layers, "q8_0", deq=deq)

    def fill(layer, m, part, rows, staging):
        synth.dev_normal_f32(staging.data_ptr(), seed, W.weight_tensor_id(layer, m, part), rows * shapes[m][1],
                             W.WEIGHT_SIGMA, stream=torch.cuda.current_stream().cuda_stream)

    ts.fill_weights(fill)
    xs = np.stack([synth.activation(seed, W.activation_tensor_id(l), shapes[0][1], rms=True) for l in range(layers)])
    ts.set_inputs(torch.from_numpy(xs).cuda())
    return ts, xs


def _weight_rows(shapes, seed, layer, j, rows):
    n, k, parts = shapes[j]
    out = []
    for r in rows:
        part, base = 0, 0
        while r >= base + parts[part]:
            base += parts[part]
            part += 1
        out.append(synth.normal_f32(seed, W.weight_tensor_id(layer, j, part), k, W.WEIGHT_SIGMA,
                                    first=(r - base) * k))
    return np.stack(out)


def _snapshot(ts):
    return [host(y).view(np.uint32).copy() for y in ts.outputs()]


def _check_against_oracle(shapes, seed, xs, got, layers, rows_for):
    """Each GEMV against the oracle (int8 block-dot form) on the rows
    rows_for(n) returns, fed the GPU's own input of that GEMV."""
    nm = len(shapes)
    for layer in range(layers):
        for j, (n, k, _) in enumerate(shapes):
            i = layer * nm + j
            x = xs[layer] if j == 0 else got[i - 1][:k]
            rows = rows_for(n)
            dw, qw = oracle.quantize_q8_0(_weight_rows(shapes, seed, layer, j, rows))
            dx, qx = oracle.quantize_q8_0(np.ascontiguousarray(x, np.float32))
            y_ref, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
            assert_within(got[i][rows], y_ref, oracle.q8_tolerance(den), f"layer {layer} GEMV {j} ({n}x{k})")


def _run_ring(ts, variant):
    for y in ts.outputs():
        y.fill_(np.nan)
    plan = ts.capture(ring=variant)
    assert plan.kernel_count == 1
    ts.launch()
    first = _snapshot(ts)
    assert not plan.error(), plan.error_detail()
    for y in ts.outputs():
        y.fill_(np.nan)
    ts.launch()
    second = _snapshot(ts)
    assert not plan.error(), plan.error_detail()
    for i, (a, b) in enumerate(zip(first, second)):
        assert np.array_equal(a, b), f"slot {i}: ring replays differ"
    return [a.view(np.float32) for a in first]


def _compare_unsplit_to_eager(gpu_lib, ts, eager, got, per_layer):
    """Bit-exact where the eager call reduces rows unsplit and its input is
    bit-identical too (a layer's first GEMV, or one fed by such a GEMV)."""
    wsg = gpu_lib
    same_input = True
    for i, s in enumerate(ts.slots):
        if i % per_layer == 0:
            same_input = True
        comparable = same_input and wsg.gemv_config(wsg.W_Q8_0, ts.act_fmt(), s.n, s.k)["split"] == 1
        if comparable:
            assert np.array_equal(eager[i], got[i].view(np.uint32)), f"slot {i}: ring differs from the eager call"
        same_input = comparable


@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("wl_name,layers", [("qwen3_8b_q8_0_36L", 3), ("dense27b_q8_0_64L", 2)])
def test_ring_stream_matches_oracle_and_eager(gpu_lib, wl_name, layers, variant):
    wl = {w.name: w for w in W.ALL}[wl_name]
    shapes = [(m.n, m.k, m.parts) for m in wl.matrices]
    ts, xs = _chain(shapes, layers, wl.seed)
    ts.run_eager()
    eager = _snapshot(ts)
    got = _run_ring(ts, variant)
    _compare_unsplit_to_eager(gpu_lib, ts, eager, got, len(shapes))
    rng = np.random.default_rng(0x51A7 + variant)

    def rows_for(n):
        # first and last rows, the rows of the first and last workgroups, random rows
        return np.array(sorted({0, 1, 255, 256, n - 257, n - 1} | set(int(v) for v in rng.integers(0, n, 58))))

    _check_against_oracle(shapes, wl.seed, xs, got, layers, rows_for)
    ts.close()


RAGGED = [
    # rows not a multiple of the grid, ragged last chunks (2080: 1 block; 4128: 1 block)
    [(4100, 2048, (4100,)), (3001, 4096, (2000, 1001)), (2050, 2080, (2050,)), (2048, 2048, (2048,))],
    # fewer rows than workgroups (most workgroups idle in some GEMVs), one-block rows
    [(300, 4128, (300,)), (96, 96, (96,)), (33, 64, (33,)), (2112, 32, (2112,))],
]


@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("case", [0, 1])
def test_ring_ragged_chains_every_row(gpu_lib, case, variant):
    shapes = RAGGED[case]
    seed = 0x5EED7100 + case
    layers = 2
    ts, xs = _chain(shapes, layers, seed)
    ts.run_eager()
    eager = _snapshot(ts)
    got = _run_ring(ts, variant)
    _compare_unsplit_to_eager(gpu_lib, ts, eager, got, len(shapes))
    _check_against_oracle(shapes, seed, xs, got, layers, lambda n: np.arange(n))
    ts.close()


def test_ring_replays_many_times(gpu_lib):
    """Launch parity flips every replay: ten replays of a 2-layer 27B-shaped
    chain all equal the first."""
    wl = W.DENSE27B_Q8
    shapes = [(m.n, m.k, m.parts) for m in wl.matrices]
    ts, _ = _chain(shapes, 2, wl.seed)
    plan = ts.capture(ring=True)
    ts.launch()
    ref = _snapshot(ts)
    for rep in range(10):
        for y in ts.outputs():
            y.fill_(np.nan)
        ts.launch()
        got = _snapshot(ts)
        assert all(np.array_equal(a, b) for a, b in zip(ref, got)), f"replay {rep + 1}"
    assert not plan.error()
    ts.close()


def test_ring_plan_rejections(gpu_lib):
    wsg = gpu_lib
    wl = W.QWEN3_8B_Q8
    shapes = [(m.n, m.k, m.parts) for m in wl.matrices]
    ts, _ = _chain(shapes, 1, wl.seed, deq=2)  # f32 activations: not run by the ring
    with pytest.raises(wsg.WsgError) as e:
        ts.capture(ring=0)
    assert e.value.status == wsg.ERR_MODE
    ts.close()
    ts, _ = _chain(shapes, 1, wl.seed, deq=0)
    ops = ts.ops()
    arr = (wsg.OpDesc * len(ops))(*ops)
    plan = ctypes.c_void_p()
    for variant in (-1, wsg.RING_VARIANTS):
        assert wsg.lib().wsg_plan_create_ring(arr, len(ops), variant, None, ctypes.byref(plan)) == wsg.ERR_MODE
        assert not plan.value
    ts.close()
