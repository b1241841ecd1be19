"""The whole-token plan (one hipGraph per token; emit_qwen38_generate,
"Where the speed comes from", item 2; GPU Kernel Lab, "Decode integration":
fixed-address graph replay checked against eager execution).

* replay == eager, bit for bit, for every intermediate, and two replays
  agree (also a race check of the split-K LDS stage);
* the chain's wiring (each GEMV reads the previous output's first K
  entries) is checked end to end against an oracle chain for the f32 paths,
  with the error bound propagated through the layer;
* the first GEMV of every layer reads generator data, so it is checked
  directly against the oracle."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_within, host
from synth import workloads as W

pytestmark = pytest.mark.gpu


def _stream(wl, layers, deq=0, requant="fused"):
    import torch

    from weight_streaming_gemv_q8_amd.stream import TokenStream
    shapes = [(m.n, m.k, m.parts) for m in wl.matrices]
    ts = TokenStream(shapes, layers, wl.wtype, deq=deq, requant=requant)

    def fill(layer, m, part, rows, staging):
        synth.dev_normal_f32(staging.data_ptr(), wl.seed, W.weight_tensor_id(layer, m, part),
                             rows * wl.matrices[m].k, W.WEIGHT_SIGMA,
                             stream=torch.cuda.current_stream().cuda_stream)

    ts.fill_weights(fill)
    xs = np.stack([synth.activation(wl.seed, W.activation_tensor_id(l), wl.matrices[0].k, rms=True)
                   for l in range(layers)])
    ts.set_inputs(torch.from_numpy(xs).cuda())
    return ts, xs


def _snapshot(ts):
    return [host(y).view(np.uint32).copy() for y in ts.outputs()]


@pytest.mark.parametrize("deq,requant", [(0, "fused"), (0, "separate"), (2, "fused")])
def test_replay_equals_eager_q8(gpu_lib, deq, requant):
    ts, _ = _stream(W.QWEN3_8B_Q8, 2, deq=deq, requant=requant)
    ts.run_eager()
    eager = _snapshot(ts)
    for y in ts.outputs():
        y.fill_(np.nan)
    plan = ts.capture()
    n_gemv = len(ts.slots)
    assert plan.kernel_count == (2 * n_gemv if (deq == 0 and requant == "separate") else n_gemv)
    ts.launch()
    first = _snapshot(ts)
    ts.launch()
    second = _snapshot(ts)
    for a, b, c in zip(eager, first, second):
        assert np.array_equal(a, b) and np.array_equal(b, c)
    ts.close()


def _new_inputs(ts, wl, seed):
    """Fresh seeded layer inputs (different values on every call)."""
    import torch
    xs = np.stack([synth.activation(seed, W.activation_tensor_id(l), ts.shapes[0][1], rms=True)
                   for l in range(ts.layers)])
    ts.set_inputs(torch.from_numpy(xs).cuda())
    return xs


def _replays_follow_inputs(ts, wl, plan, seeds):
    """Before each replay the layer inputs change: every output of the
    replay must equal the eager calls on those inputs, bit for bit, and no
    wait may have timed out.  A replay that read a value left over from the
    previous replay (a plan-owned copy of an output, a stale flag) would
    differ here, since the previous replay saw other inputs."""
    for rep, seed in enumerate(seeds):
        _new_inputs(ts, wl, seed)
        ts.run_eager()
        eager = _snapshot(ts)
        for y in ts.outputs():
            y.fill_(np.nan)
        ts.launch()
        got = _snapshot(ts)
        assert not plan.error(), f"replay {rep}: a wait timed out: {plan.error_detail()}"
        for i, (a, b) in enumerate(zip(eager, got)):
            assert np.array_equal(a, b), f"replay {rep} (seed {seed:#x}): slot {i} differs from eager"


@pytest.mark.parametrize("wl_name,layers,deq", [("qwen3_8b_q8_0_36L", 3, 0), ("qwen3_8b_q8_0_36L", 2, 2),
                                                ("dense27b_q8_0_64L", 2, 0), ("dense27b_q8_0_64L", 2, 2)])
def test_persistent_replay_equals_eager(gpu_lib, wl_name, layers, deq):
    """The whole token in one resident kernel: the same rows reduced in the
    same order as the eager calls, so every output is bit-identical, on
    three consecutive replays whose inputs all differ, and no wait timed
    out."""
    wl = {w.name: w for w in W.ALL}[wl_name]
    ts, _ = _stream(wl, layers, deq=deq)
    plan = ts.capture(persistent=True)
    assert plan.kernel_count == 1
    _replays_follow_inputs(ts, wl, plan, [0x5EED7000 + i for i in range(3)])
    ts.close()


@pytest.mark.parametrize("split", [2, 4])
@pytest.mark.parametrize("deq", [0, 2])
def test_persistent_forced_split_equals_eager(gpu_lib, split, deq):
    """Forced split factors on a chain with one-chunk rows (k = 2048: some
    parts have no chunks), a ragged last chunk (k = 2080) and row counts
    that do not divide among the workgroups: the persistent kernel (whose
    waves take (row, part) units in whatever order they get to them) still
    equals the eager calls bit for bit, over three replays with changing
    inputs."""
    import torch

    from weight_streaming_gemv_q8_amd.stream import TokenStream
    wsg = gpu_lib
    shapes = [(4100, 2048, (4100,)), (3001, 4096, (3001,)), (2050, 2080, (2050,)), (2048, 2048, (2048,))]
    seed = 0x5EED5117
    wsg.tune(wsg.TUNE_SPLITK, split)
    try:
        ts = TokenStream(shapes, 2, "q8_0", deq=deq)

        def fill(layer, m, part, rows, staging):
            synth.dev_normal_f32(staging.data_ptr(), seed, W.weight_tensor_id(layer, m, part),
                                 rows * shapes[m][1], W.WEIGHT_SIGMA, stream=torch.cuda.current_stream().cuda_stream)

        ts.fill_weights(fill)
        _new_inputs(ts, None, seed)
        for slot in ts.slots:
            assert wsg.gemv_config(wsg.W_Q8_0, ts.act_fmt(), slot.n, slot.k)["split"] == split
        plan = ts.capture(persistent=True)
        _replays_follow_inputs(ts, None, plan, [seed + 1, seed + 2, seed + 3])
        ts.close()
    finally:
        wsg.tune(wsg.TUNE_SPLITK, 0)


@pytest.mark.parametrize("deq", [0, 2])
def test_persistent_small_ops_and_idle_workgroups(gpu_lib, deq):
    """Ops with fewer rows than workgroups (some workgroups own no rows),
    single-row ops and a one-block k: a workgroup's streaming waves may run
    several ops ahead of its control waves; every output still equals the
    eager calls, over three replays with changing inputs."""
    import torch

    from weight_streaming_gemv_q8_amd.stream import TokenStream
    shapes = [(96, 1024, (96,)), (300, 64, (300,)), (40, 256, (40,)), (1, 32, (1,))]
    seed = 0x5EED5119
    ts = TokenStream(shapes, 3, "q8_0", deq=deq)

    def fill(layer, m, part, rows, staging):
        synth.dev_normal_f32(staging.data_ptr(), seed, W.weight_tensor_id(layer, m, part),
                             rows * shapes[m][1], W.WEIGHT_SIGMA, stream=torch.cuda.current_stream().cuda_stream)

    ts.fill_weights(fill)
    plan = ts.capture(persistent=True)
    _replays_follow_inputs(ts, None, plan, [seed + 1, seed + 2, seed + 3])
    ts.close()


def test_persistent_plan_rejects_unsupported_ops(gpu_lib):
    wsg = gpu_lib
    ts, _ = _stream(W.QWEN3_0P6B_BF16, 1)
    with pytest.raises(wsg.WsgError) as e:
        ts.capture(persistent=True)
    assert e.value.status == wsg.ERR_MODE
    ts.close()


def test_replay_equals_eager_bf16(gpu_lib):
    ts, _ = _stream(W.QWEN3_0P6B_BF16, 3)
    ts.run_eager()
    eager = _snapshot(ts)
    ts.capture()
    for _ in range(3):
        for y in ts.outputs():
            y.fill_(np.nan)
        ts.launch()
        got = _snapshot(ts)
        assert all(np.array_equal(a, b) for a, b in zip(eager, got))
    ts.close()


def test_fused_and_separate_requant_agree(gpu_lib):
    a, _ = _stream(W.QWEN3_8B_Q8, 1, deq=0, requant="fused")
    a.launch()
    ya = _snapshot(a)
    a.close()
    del a
    b, _ = _stream(W.QWEN3_8B_Q8, 1, deq=0, requant="separate")
    b.launch()
    yb = _snapshot(b)
    b.close()
    assert all(np.array_equal(u, v) for u, v in zip(ya, yb))


def _oracle_weights(wl, layer, j):
    m = wl.matrices[j]
    w = np.concatenate([synth.normal_f32(wl.seed, W.weight_tensor_id(layer, j, p), r * m.k, W.WEIGHT_SIGMA)
                        .reshape(r, m.k) for p, r in enumerate(m.parts)])
    return w


@pytest.mark.parametrize("wl_name,deq", [("qwen3_8b_q8_0_36L", 2), ("qwen3_0.6b_bf16_28L", 0)])
def test_chain_against_oracle_with_propagated_bound(gpu_lib, wl_name, deq):
    """f32-activation chains: |y_j - y_ref_j| <= tol_j + |W_j| (B_{j-1} + ulp)
    where y_ref_j is the oracle fed its own previous output rounded to f32."""
    wl = {w.name: w for w in W.ALL}[wl_name]
    ts, xs = _stream(wl, 1, deq=deq)
    ts.launch()
    ys = [host(y) for y in ts.outputs()]
    ts.close()
    x = xs[0]
    bound_prev = None
    for j, m in enumerate(wl.matrices):
        w = _oracle_weights(wl, 0, j)
        if wl.wtype == "q8_0":
            dw, qw = oracle.quantize_q8_0(w)
            y_ref, den = oracle.gemv_q8_act_f32(dw, qw, x)
            wabs = np.abs(np.repeat(oracle.f16_bits_to_f64(dw), 32, axis=1) * qw)
            tol = oracle.q8_tolerance(den)
        else:
            wb = oracle.f32_to_bf16_rows(w)
            y_ref, den = oracle.gemv_bf16(wb, x)
            wabs = np.abs(oracle.bf16_bits_to_f64(wb))
            tol = oracle.bf16_tolerance(den)
        if bound_prev is not None:
            # the GPU's input differs from the oracle's by at most the previous
            # bound plus the rounding of the oracle's output to f32
            tol = tol * 1.01 + wabs @ bound_prev
        assert_within(ys[j], y_ref, tol, f"{wl_name} GEMV {j}")
        nxt = wl.matrices[j + 1].k if j + 1 < len(wl.matrices) else None
        if nxt is None:
            break
        bound_prev = tol[:nxt] + np.abs(y_ref[:nxt]) * 2.0 ** -24
        x = y_ref[:nxt].astype(np.float32)


def test_layer_inputs_match_oracle_int8(gpu_lib):
    """deq 0: the first GEMV of each layer reads generator data: its output
    must match the oracle (int8 block-dot form) on every row."""
    wl = W.QWEN3_8B_Q8
    ts, xs = _stream(wl, 2, deq=0)
    ts.launch()
    for layer in range(2):
        s = ts.slots[layer * len(wl.matrices)]
        y = host(s.y)
        dw, qw = oracle.quantize_q8_0(_oracle_weights(wl, layer, 0))
        dx, qx = oracle.quantize_q8_0(xs[layer])
        y_ref, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
        assert_within(y, y_ref, oracle.q8_tolerance(den), f"layer {layer} qkv")
    ts.close()


def test_persistent_plan_rejects_racy_buffers(gpu_lib):
    """Without grid barriers ops overlap in time, so the persistent plan
    refuses buffers that would race: an input straddling an earlier output,
    two outputs that overlap, and an output over an input read from outside
    the plan."""
    import torch
    wsg = gpu_lib
    n, k = 256, 256
    w = torch.zeros(n * wsg.q8_0_row_bytes(k), dtype=torch.uint8, device="cuda")
    buf = torch.zeros(4 * n, dtype=torch.float32, device="cuda")
    x0 = torch.zeros(k, dtype=torch.float32, device="cuda")
    fmt = wsg.ACT_F32_REQUANT

    def make(ops):
        arr = (wsg.OpDesc * len(ops))(*ops)
        plan = ctypes.c_void_p()
        return wsg.lib().wsg_plan_create_persistent(arr, len(ops), None, ctypes.byref(plan)), plan

    y0, y1 = buf[0:n], buf[n:2 * n]
    cases = {
        "input straddles an output": [wsg.op_gemv_q8_0(w, n, k, x0, fmt, y0),
                                      wsg.op_gemv_q8_0(w, n, k, buf[n // 2:], fmt, y1)],
        "outputs overlap": [wsg.op_gemv_q8_0(w, n, k, x0, fmt, y0),
                            wsg.op_gemv_q8_0(w, n, k, x0, fmt, buf[n // 2:])],
        "output over an outside input": [wsg.op_gemv_q8_0(w, n, k, y1, fmt, y0),
                                         wsg.op_gemv_q8_0(w, n, k, x0, fmt, y1)],
    }
    for name, ops in cases.items():
        rc, plan = make(ops)
        assert rc == wsg.ERR_MODE, name
    # the legal chain: the second op reads the first op's output
    rc, plan = make([wsg.op_gemv_q8_0(w, n, k, x0, fmt, y0), wsg.op_gemv_q8_0(w, n, k, y0, fmt, y1)])
    assert rc == wsg.OK
    assert wsg.lib().wsg_plan_destroy(plan) == wsg.OK
