"""Closing the decode loop on the device (GPU Kernel Lab, "Decode
integration": fixed token/position buffers ... LM-head GEMV + argmax +
token/position update under one graph replay; emit_qwen38_generate, "Where
the speed comes from", item 2: token and position advanced on the device).

* embed_gather returns the dequantized table row of the token it reads on
  the device, bit for bit (Q8_0: d q is exact in f32; BF16: exact), for
  first, last, interior and ragged-chunk rows, and a zero row for tokens
  outside the vocabulary;
* token_advance appends to the history while it has room and always
  counts the position;
* a whole decode step (embedding -> 2 layers of the 8B-shaped chain, in
  Q8_0 or 4-bit weights, with the residual stream, fused norms and SwiGLU
  -> final norm -> LM head + argmax -> advance) replayed from one graph
  decodes the same tokens as
  its calls run one at a time; at every step the embedding is the row of
  the token consumed, the argmax is exact on the step's own logits, and
  the logits match the oracle fed the GPU's own LM-head input."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_within, dev, empty_u8, host, split_act_q8
from synth import workloads as W

pytestmark = pytest.mark.gpu

EMB_ID, HEAD_ID = W.EMBEDDING_TENSOR_ID, W.LM_HEAD_TENSOR_ID


def _q8_rows_host(seed, tensor, hidden, rows, sigma):
    w = np.stack([synth.normal_f32(seed, tensor, hidden, sigma, first=int(r) * hidden) for r in rows])
    return oracle.quantize_q8_0(w)


@pytest.mark.parametrize("hidden", [2080, 4096])
def test_embed_gather(gpu_lib, hidden):
    import torch
    wsg = gpu_lib
    vocab, seed = 1000, 0x5EEDB000 + hidden
    table = synth.normal_f32(seed, EMB_ID, vocab * hidden, 0.5).reshape(vocab, hidden)
    packed = empty_u8(wsg.q8_0_packed_bytes(vocab, hidden))
    wsg.quantize_q8_0_weights(dev(table), vocab, hidden, packed)
    bf = torch.empty(vocab * hidden, dtype=torch.int16, device="cuda")
    wsg.convert_bf16(dev(table), vocab * hidden, bf)
    out = torch.empty(hidden, dtype=torch.float32, device="cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    for t in (0, vocab - 1, 517, -1, vocab, 2 ** 30):
        tok.fill_(t)
        wsg.embed_gather(packed, wsg.W_Q8_0, vocab, hidden, tok, out)
        got = host(out)
        if 0 <= t < vocab:
            d, q = oracle.quantize_q8_0(table[t:t + 1])
            want = (np.repeat(oracle.f16_bits_to_f64(d), 32, axis=1) * q)[0].astype(np.float32)
        else:
            want = np.zeros(hidden, np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"Q8_0 row {t}"
        wsg.embed_gather(bf, wsg.W_BF16, vocab, hidden, tok, out)
        got = host(out)
        if 0 <= t < vocab:
            want = oracle.bf16_bits_to_f64(oracle.f32_to_bf16_bits(table[t])).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"BF16 row {t}"


def test_token_advance(gpu_lib):
    import torch
    wsg = gpu_lib
    hist = torch.full((3,), -1, dtype=torch.int32, device="cuda")
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    for t in (11, 22, 33, 44, 55):
        tok.fill_(t)
        wsg.token_advance(tok, hist, 3, pos)
    assert host(hist).tolist() == [11, 22, 33] and int(host(pos)[0]) == 5
    with pytest.raises(wsg.WsgError) as e:
        wsg.token_advance(tok, hist, -1, pos)
    assert e.value.status == wsg.ERR_SHAPE


def _decode_step(vocab, layers, wtype="q8_0", deq=0):
    import torch

    from weight_streaming_gemv_q8_amd.stream import DecodeStep
    wl = W.QWEN3_8B_Q8
    shapes = [(m.n, m.k, m.parts) for m in wl.matrices]
    ds = DecodeStep(shapes, layers, vocab, capacity=16, eps=W.RMSNORM_EPS, wtype=wtype, deq=deq)
    stream = torch.cuda.current_stream().cuda_stream

    def fill(layer, m, part, rows, staging):
        synth.dev_normal_f32(staging.data_ptr(), wl.seed, W.weight_tensor_id(layer, m, part),
                             rows * wl.matrices[m].k, W.WEIGHT_SIGMA, stream=stream)

    ds.chain.fill_weights(fill)
    hidden = ds.hidden
    ds.fill_table(ds.embedding, lambda r0, st: synth.dev_normal_f32(st.data_ptr(), wl.seed, EMB_ID, st.numel(), 1.0,
                                                                     first=r0 * hidden, stream=stream))
    ds.fill_table(ds.lm_head, lambda r0, st: synth.dev_normal_f32(st.data_ptr(), wl.seed, HEAD_ID, st.numel(),
                                                                   W.WEIGHT_SIGMA, first=r0 * hidden, stream=stream))
    gains = np.stack([np.float32(1.0) + synth.normal_f32(wl.seed, W.gain_tensor_id(i), hidden, W.GAIN_SIGMA)
                      for i in range(len(ds.chain.norms))]).astype(np.float32)
    ds.chain.gains.copy_(torch.from_numpy(gains))
    return ds, wl.seed


@pytest.mark.parametrize("wtype,deq", [("q8_0", 0), ("q8_0", 1), ("q8_0", 2), ("q4_0", 0), ("q4_0", 1)])
def test_decode_step_graph_equals_eager_and_oracle(gpu_lib, wtype, deq):
    """deq (emit_qwen38_generate, the deq paragraph): 0 int8 activations
    everywhere; 1 the LM head on the f32 final norm output; 2 (Q8_0 layers)
    f32 activations in every GEMV: the fused norm GEMVs' f32 form, the
    W8A16 SwiGLU GEMV, the dequantizing down projection and LM head."""
    wsg = gpu_lib
    vocab, layers, steps, first = 32000, 2, 5, 7
    ds, seed = _decode_step(vocab, layers, wtype, deq)
    if deq == 2:
        ops = ds.ops()
        assert not any(o.op == wsg.OP_QUANTIZE_ACT for o in ops)
        assert all(o.act_fmt == wsg.ACT_F32 for o in ops
                   if o.op in (wsg.OP_GEMV_Q8_0, wsg.OP_GEMV_Q8_0_RMSNORM, wsg.OP_GEMV_Q8_0_SWIGLU,
                               wsg.OP_LM_HEAD_ARGMAX))
        assert all(o.y_q8 is None or not o.y_q8 for o in ops if o.op == wsg.OP_RESIDUAL_RMSNORM)
    hidden = ds.hidden
    rng = np.random.default_rng(0xDEC0)
    ds.reset(first)
    for step in range(steps):
        consumed = int(host(ds.token)[0])
        ds.run_eager()
        # the embedding of the token consumed
        d, q = _q8_rows_host(seed, EMB_ID, hidden, [consumed], 1.0)
        emb = (np.repeat(oracle.f16_bits_to_f64(d), 32, axis=1) * q)[0].astype(np.float32)
        assert np.array_equal(host(ds.chain.h0).view(np.uint32), emb.view(np.uint32)), f"step {step}: embedding"
        # the argmax on the step's own logits, and the logits against the oracle
        logits = host(ds.logits)
        tok = int(host(ds.token)[0])
        assert tok == oracle.argmax_f32(logits), f"step {step}: argmax"
        rows = np.array(sorted({0, vocab - 1, tok} | set(int(v) for v in rng.integers(0, vocab, 40))))
        dw, qw = _q8_rows_host(seed, HEAD_ID, hidden, rows, W.WEIGHT_SIGMA)
        if deq == 0:
            dx, qx = split_act_q8(host(ds.final_q8), hidden)
            y_ref, den = oracle.gemv_q8_act_q8(dw, qw, dx, qx)
        else:
            y_ref, den = oracle.gemv_q8_act_f32(dw, qw, host(ds.final_y))
        assert_within(logits[rows], y_ref, oracle.q8_tolerance(den), f"step {step}: LM-head logits")
    eager = host(ds.history).copy()
    assert int(host(ds.pos)[0]) == steps and np.all(eager[:steps] >= 0) and np.all(eager[steps:] == -1)

    ds.reset(first)
    plan = ds.capture()
    for _ in range(steps):
        ds.launch()
    graph = host(ds.history)
    assert plan.kernel_count == len(ds.ops()) + 1  # the LM head: GEMV with stage-1 argmax, then stage 2
    assert np.array_equal(graph, eager), f"graph decoded {graph[:steps]}, eager {eager[:steps]}"
    assert int(host(ds.pos)[0]) == steps
    ds.close()
