"""lm_head_argmax_static, the LM head for callers that cannot allocate:
called through the C ABI, it must give the index and logits of
lm_head_argmax (the workspace variant) bit for bit, on two calls in a row,
the second with a smaller input (the static array keeps the first call's
keys, which the second must not read), for each weight type and
activation format."""
import ctypes

import numpy as np
import pytest

import synth
from gpu_util import dev, host

pytestmark = pytest.mark.gpu


def _head(wsg, n, k, w_type, seed):
    import torch
    w = synth.normal_f32(seed, 1, n * k, 0.02).reshape(n, k)
    wd = dev(w)
    if w_type == wsg.W_BF16:
        out = torch.empty(n * k, dtype=torch.uint16, device="cuda")
        wsg.convert_bf16(wd, n * k, out)
    else:
        out = torch.empty(wsg.q8_0_packed_bytes(n, k), dtype=torch.uint8, device="cuda")
        wsg.quantize_q8_0_weights(wd, n, k, out)
    return out


def _both(wsg, L, w, w_type, n, k, x, act):
    import torch
    ws = torch.empty(wsg.lm_head_argmax_ws_bytes(n, k, w_type), dtype=torch.uint8, device="cuda")
    idx_ref = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    log_ref = torch.full((n,), np.nan, dtype=torch.float32, device="cuda")
    wsg.lm_head_argmax(w, w_type, n, k, x, act, ws, ws.numel(), idx_ref, log_ref)
    idx = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    logits = torch.full((n,), np.nan, dtype=torch.float32, device="cuda")
    # through the C ABI directly
    rc = L.lm_head_argmax_static(ctypes.c_void_p(w.data_ptr()), w_type, n, k, ctypes.c_void_p(x.data_ptr()), act,
                                 ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(logits.data_ptr()), None)
    assert rc == wsg.OK, wsg.status_str(rc)
    a, b = host(idx_ref), host(idx)
    assert int(a[0]) == int(b[0]) and 0 <= int(b[0]) < n, (a, b)
    assert np.array_equal(host(log_ref).view(np.uint32), host(logits).view(np.uint32))
    return int(b[0])


@pytest.mark.parametrize("w_type_name,act_name", [("W_Q8_0", "ACT_F32_REQUANT"), ("W_Q8_0", "ACT_F32"),
                                                  ("W_Q8_0", "ACT_Q8_0"), ("W_BF16", "ACT_F32")])
def test_static_lm_head_equals_workspace_lm_head(gpu_lib, w_type_name, act_name):
    wsg = gpu_lib
    L = wsg.lib()
    w_type, act = getattr(wsg, w_type_name), getattr(wsg, act_name)
    # a vocabulary-sized head, then a much smaller one: the second call's
    # stage 1 has fewer workgroups than the first left keys behind
    for n, k, seed in ((151936, 4096, 0x5EED0A01), (3001, 1024, 0x5EED0A02)):
        w = _head(wsg, n, k, w_type, seed)
        x32 = dev(synth.activation(seed, 2, k))
        if act == wsg.ACT_Q8_0:
            import torch
            x = torch.empty(wsg.act_q8_0_bytes(k), dtype=torch.uint8, device="cuda")
            wsg.quantize_act_q8_0(x32, k, x)
        else:
            x = x32
        _both(wsg, L, w, w_type, n, k, x, act)
        del w


def test_static_lm_head_planted_winner_on_the_second_call(gpu_lib):
    """A first call whose winner sits in a high stage-1 workgroup, then a
    smaller call: a stale key of the first call, if read, would name a row
    the second head does not have."""
    import torch
    wsg = gpu_lib
    L = wsg.lib()
    k = 1024
    for n, best in ((100000, 99990), (5000, 17)):
        w = synth.normal_f32(0x5EED0A03, 1, n * k, 0.02).reshape(n, k)
        w[best] = 0.0
        w[best, 5] = 1.0
        x = synth.activation(0x5EED0A03, 2, k)
        x[5] = 50.0
        wq = torch.empty(wsg.q8_0_packed_bytes(n, k), dtype=torch.uint8, device="cuda")
        wsg.quantize_q8_0_weights(dev(w), n, k, wq)
        got = _both(wsg, L, wq, wsg.W_Q8_0, n, k, dev(x), wsg.ACT_F32_REQUANT)
        assert got == best
