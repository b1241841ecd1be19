"""GPU parity of the fused LM-head argmax (emit_qwen38_generate, "Where the
speed comes from", item 2: the sampled token stays on the device; GPU
Kernel Lab, "Decode integration": LM-head GEMV + argmax).

The index must be bit-exact: ties go to the lowest index, -0 == +0.  Ties
and near-ties are planted so that they are exact in f32 under any
summation order (weights with a single nonzero code; x values 3.0 and its
f32 neighbours), plus a dense exact tie made by copying the best random
row to a lower index."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_within, check_argmax_vs_oracle, dev, empty_u8, host

pytestmark = pytest.mark.gpu

SEED = 0x5EED0003
N_VOCAB, K_HID = 151936, 4096


# ------------------------------------------------------------- argmax_f32

def _vec_cases():
    n = N_VOCAB
    rng_base = synth.normal_f32(SEED, 500, n, 1.0)
    cases = []
    v = rng_base.copy()
    v[777] = 8.0
    v[99] = 8.0
    cases.append(("exact tie", v))
    v = rng_base.copy()
    v[10] = np.nextafter(np.float32(8.0), np.float32(0))
    v[5000] = np.float32(8.0)
    v[n - 2] = np.nextafter(np.float32(8.0), np.float32(np.inf))
    cases.append(("one-ulp near ties", v))
    v = -np.abs(rng_base) - 1.0
    v[300] = -0.0
    v[200] = 0.0
    v[400] = -0.0
    cases.append(("signed zeros", v))
    v = rng_base.copy()
    v[0] = 10.0
    cases.append(("max at 0", v))
    v = rng_base.copy()
    v[n - 1] = 10.0
    cases.append(("max at n-1", v))
    cases.append(("all equal", np.full(n, 1.5, np.float32)))
    cases.append(("short", np.array([1.0, 3.0, 3.0, -1.0], np.float32)))
    cases.append(("single", np.array([-2.0], np.float32)))
    return cases


def test_argmax_f32_bitexact(gpu_lib):
    import torch
    wsg = gpu_lib
    ws = empty_u8(wsg.argmax_ws_bytes())
    idx = torch.empty(1, dtype=torch.int32, device="cuda")
    for name, v in _vec_cases():
        idx.fill_(-7)
        wsg.argmax_f32(dev(v), v.size, ws, ws.numel(), idx)
        assert int(host(idx)[0]) == oracle.argmax_f32(v), name


# ------------------------------------------------------------ LM head

C_COL = 1234  # planted column; x[c] = 3.0, x[c+1] = 3 + 2^-22, x[c+2] = 3 - 2^-22


def _hidden():
    x = synth.normal_f32(SEED, 600, K_HID, 1.0)
    x[C_COL] = np.float32(3.0)
    x[C_COL + 1] = np.nextafter(np.float32(3.0), np.float32(np.inf))
    x[C_COL + 2] = np.nextafter(np.float32(3.0), np.float32(0))
    return x


@pytest.fixture(scope="module")
def lm_weights():
    return synth.normal_f32(SEED, 601, N_VOCAB * K_HID, 0.02).reshape(N_VOCAB, K_HID)


@pytest.fixture(scope="module")
def lm_q8_ref(lm_weights):
    return oracle.quantize_q8_0(lm_weights)


# planted rows -> column they point at (col offset 0: 3.0, 1: next up, 2: next down)
PLANT_SETS = {
    "tie_lowest_wins": {1000: 0, 5000: 0, 10: 2},
    "one_ulp_above_wins": {1000: 0, 5000: 0, 10: 2, 90000: 1},
    "duplicates_lowest_wins": {1000: 0, 5000: 0, 10: 2, 90000: 1, 70000: 1, 120000: 1},
}


def _planted_q8_rows(cols):
    """Q8_0 rows that are zero except one block: d = 4.0, q = 1 at the column."""
    nb = K_HID // 32
    d = np.zeros((len(cols), nb), np.uint16)
    q = np.zeros((len(cols), K_HID), np.int8)
    for i, off in enumerate(cols):
        c = C_COL + off
        d[i, c // 32] = 0x4400  # 4.0 in binary16
        q[i, c] = 1
    return d, q


def _run_q8(wsg, packed, x, act_fmt):
    import torch
    n = N_VOCAB
    ws = empty_u8(wsg.argmax_ws_bytes())
    idx = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    logits = torch.empty(n, dtype=torch.float32, device="cuda")
    xin = dev(x)
    if act_fmt == wsg.ACT_Q8_0:
        xq = empty_u8(wsg.act_q8_0_bytes(K_HID))
        wsg.quantize_act_q8_0(xin, K_HID, xq)
        xin = xq
    wsg.lm_head_argmax(packed, wsg.W_Q8_0, n, K_HID, xin, act_fmt, ws, ws.numel(), idx, logits)
    # the same call without the logits output picks the same row
    idx2 = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    wsg.lm_head_argmax(packed, wsg.W_Q8_0, n, K_HID, xin, act_fmt, ws, ws.numel(), idx2, None)
    i1, i2 = int(host(idx)[0]), int(host(idx2)[0])
    assert i1 == i2
    return i1, host(logits)


def _oracle_q8_logits(dw, qw, x, act_fmt):
    if act_fmt == 1:  # f32 hidden (deq 1/2)
        return oracle.gemv_q8_act_f32(dw, qw, x)
    dx, qx = oracle.quantize_q8_0(x)
    return oracle.gemv_q8_act_q8(dw, qw, dx, qx)


@pytest.mark.parametrize("act_name", ["f32", "q8", "requant"])
def test_lm_head_q8_planted_ties(gpu_lib, lm_weights, lm_q8_ref, act_name):
    wsg = gpu_lib
    act_fmt = {"f32": wsg.ACT_F32, "q8": wsg.ACT_Q8_0, "requant": wsg.ACT_F32_REQUANT}[act_name]
    x = _hidden()
    n, k = N_VOCAB, K_HID
    dw, qw = lm_q8_ref
    y_rand, den_rand = _oracle_q8_logits(dw, qw, x, act_fmt)
    packed = empty_u8(wsg.q8_0_packed_bytes(n, k))
    wsg.quantize_q8_0_weights(dev(lm_weights), n, k, packed)
    rb = wsg.q8_0_row_bytes(k)

    # random rows only
    idx, logits = _run_q8(wsg, packed, x, act_fmt)
    assert_within(logits, y_rand, oracle.q8_tolerance(den_rand), "lm_head q8 random")
    assert idx == int(np.argmax(logits))          # fused index == argmax of its own logits
    check_argmax_vs_oracle(idx, y_rand, oracle.q8_tolerance(den_rand))

    for name, plant in PLANT_SETS.items():
        rows = sorted(plant)
        pd, pq = _planted_q8_rows([plant[r] for r in rows])
        aos = synth.blocks_to_aos(pd, pq)
        for i, r in enumerate(rows):
            wsg.pack_q8_0(dev(aos[i]), 1, k, packed.data_ptr() + r * rb)
        y_ref, den = y_rand.copy(), den_rand.copy()
        yp, dp = _oracle_q8_logits(pd, pq, x, act_fmt)
        y_ref[rows], den[rows] = yp, dp
        idx, logits = _run_q8(wsg, packed, x, act_fmt)
        want = oracle.argmax_f64(y_ref)
        assert idx == want, (name, idx, want)
        assert idx == int(np.argmax(logits))
        if act_fmt == wsg.ACT_F32:
            expect = {"tie_lowest_wins": 1000, "one_ulp_above_wins": 90000,
                      "duplicates_lowest_wins": 70000}[name]
            assert want == expect
    # restore the random rows that were overwritten
    for r in sorted(PLANT_SETS["duplicates_lowest_wins"]):
        wsg.quantize_q8_0_weights(dev(lm_weights[r:r + 1]), 1, k, packed.data_ptr() + r * rb)

    # dense exact tie: copy the best random row to a lower index
    best = oracle.argmax_f64(y_rand)
    low = best // 2
    pk = packed.view(n, rb)
    pk[low].copy_(pk[best])
    y_ref = y_rand.copy()
    y_ref[low] = y_rand[best]
    idx, logits = _run_q8(wsg, packed, x, act_fmt)
    assert logits[low].tobytes() == logits[best].tobytes()
    assert idx == low == oracle.argmax_f64(y_ref)


def test_lm_head_bf16_planted_ties(gpu_lib, lm_weights):
    import torch
    wsg = gpu_lib
    n, k = N_VOCAB, K_HID
    x = _hidden()
    wb_ref = oracle.f32_to_bf16_rows(lm_weights)
    y_rand, den_rand = oracle.gemv_bf16(wb_ref, x)
    wb = torch.empty(n * k, dtype=torch.int16, device="cuda")
    wsg.convert_bf16(dev(lm_weights), n * k, wb)
    ws = empty_u8(wsg.argmax_ws_bytes())

    def run():
        idx = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        logits = torch.empty(n, dtype=torch.float32, device="cuda")
        wsg.lm_head_argmax(wb, wsg.W_BF16, n, k, dev(x), wsg.ACT_F32, ws, ws.numel(), idx, logits)
        return int(host(idx)[0]), host(logits)

    idx, logits = run()
    assert_within(logits, y_rand, oracle.bf16_tolerance(den_rand), "lm_head bf16 random")
    assert idx == int(np.argmax(logits))
    check_argmax_vs_oracle(idx, y_rand, oracle.bf16_tolerance(den_rand))

    wv = wb.view(n, k)
    for name, plant in PLANT_SETS.items():
        y_ref = y_rand.copy()
        for r, off in plant.items():
            row = np.zeros(k, np.uint16)
            row[C_COL + off] = 0x4080  # 4.0 in bfloat16
            wv[r].copy_(torch.from_numpy(row.view(np.int16)).cuda())
            y_ref[r] = oracle.gemv_bf16(row.reshape(1, k), x)[0][0]
        idx, logits = run()
        expect = {"tie_lowest_wins": 1000, "one_ulp_above_wins": 90000,
                  "duplicates_lowest_wins": 70000}[name]
        assert idx == oracle.argmax_f64(y_ref) == expect, name
        assert idx == int(np.argmax(logits))
