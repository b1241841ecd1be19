"""The C-ABI library loads without a GPU, exports every function the header
declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import weight_streaming_gemv_q8_amd as wsg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wsgemv.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+char\s*\*|int64_t|int)\s+(\w+)\s*\(", text, flags=re.M)
    return names


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(wsg.LIB_PATH):
        from weight_streaming_gemv_q8_amd import build
        build.build()
    return wsg.lib()


def test_header_symbols_are_exported(L):
    names = _declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), n
    assert sorted(names) == sorted(wsg.EXPORTS)


def test_status_strings_and_sizes(L):
    for s in range(7):
        assert wsg.status_str(s)
    assert wsg.status_str(99) == "unknown status"
    assert wsg.version().count(".") == 2
    assert wsg.q8_0_row_bytes(5120) == 5440
    assert wsg.q8_0_row_bytes(17408) == 18496
    assert wsg.q8_0_row_bytes(32) == 16 + 32  # one block: scale padded to 16
    assert wsg.q8_0_row_bytes(33) == 0
    assert wsg.q8_0_packed_bytes(16384, 5120) == 16384 * 5440
    assert wsg.act_q8_0_bytes(4096) == 4096 + 256
    assert wsg.argmax_ws_bytes() >= 8 * 256
    # per-shape LM-head workspace: 8 bytes per stage-1 workgroup, never
    # more than the all-shapes maximum; -1 for a bad shape or type
    for n, k, wt in ((151936, 4096, wsg.W_Q8_0), (151936, 4096, wsg.W_BF16), (10, 32, wsg.W_Q8_0)):
        b = wsg.lm_head_argmax_ws_bytes(n, k, wt)
        assert 8 <= b <= wsg.argmax_ws_bytes() and b % 8 == 0, (n, k, wt, b)
    lib = wsg.lib()
    assert lib.lm_head_argmax_ws_bytes(0, 4096, wsg.W_Q8_0) == -1
    assert lib.lm_head_argmax_ws_bytes(10, 33, wsg.W_Q8_0) == -1
    assert lib.lm_head_argmax_ws_bytes(10, 12, wsg.W_BF16) == -1
    assert lib.lm_head_argmax_ws_bytes(10, 32, 7) == -1


# Every call below must fail validation, so nothing is launched (no GPU here).
BAD = 0x1001  # a misaligned fake address, never dereferenced


def test_gemv_q8_argument_errors(L):
    A16 = 0x10000
    cases = [
        (dict(w=A16, n=4, k=33, x=A16, act=0, y=A16), wsg.ERR_SHAPE),
        (dict(w=A16, n=-1, k=32, x=A16, act=0, y=A16), wsg.ERR_SHAPE),
        (dict(w=A16, n=4, k=wsg.MAX_K_Q8ACT + 32, x=A16, act=0, y=A16), wsg.ERR_SHAPE),
        (dict(w=A16, n=4, k=wsg.MAX_K_F32ACT + 32, x=A16, act=1, y=A16), wsg.ERR_SHAPE),
        (dict(w=A16, n=2 ** 31, k=32, x=A16, act=0, y=A16), wsg.ERR_SHAPE),
        (dict(w=None, n=4, k=32, x=A16, act=0, y=A16), wsg.ERR_NULL),
        (dict(w=A16, n=4, k=32, x=None, act=0, y=A16), wsg.ERR_NULL),
        (dict(w=A16, n=4, k=32, x=A16, act=0, y=None), wsg.ERR_NULL),
        (dict(w=BAD, n=4, k=32, x=A16, act=0, y=A16), wsg.ERR_ALIGN),
        (dict(w=A16, n=4, k=32, x=BAD, act=0, y=A16), wsg.ERR_ALIGN),
        (dict(w=A16, n=4, k=32, x=A16, act=0, y=0x10002), wsg.ERR_ALIGN),
        (dict(w=A16, n=4, k=32, x=A16, act=7, y=A16), wsg.ERR_MODE),
    ]
    for a, want in cases:
        got = L.gemv_q8_0(a["w"], a["n"], a["k"], a["x"], a["act"], a["y"], None, None)
        assert got == want, (a, got, want)
    # block dots are only defined on the int8 paths
    assert L.gemv_q8_0(A16, 4, 32, A16, wsg.ACT_F32, A16, A16, None) == wsg.ERR_MODE


def test_gemv_bf16_and_quant_argument_errors(L):
    A16 = 0x10000
    assert L.gemv_bf16(A16, 4, 12, A16, A16, None) == wsg.ERR_SHAPE
    assert L.gemv_bf16(A16, 4, wsg.MAX_K_F32ACT + 8, A16, A16, None) == wsg.ERR_SHAPE
    assert L.gemv_bf16(None, 4, 16, A16, A16, None) == wsg.ERR_NULL
    assert L.gemv_bf16(BAD, 4, 16, A16, A16, None) == wsg.ERR_ALIGN
    assert L.quantize_act_q8_0(A16, 40, A16, None) == wsg.ERR_SHAPE
    assert L.quantize_act_q8_0(None, 64, A16, None) == wsg.ERR_NULL
    assert L.quantize_act_q8_0(A16, 64, BAD, None) == wsg.ERR_ALIGN
    assert L.quantize_q8_0_weights(A16, 2, 48, A16, None) == wsg.ERR_SHAPE
    assert L.pack_q8_0(A16, 2, 64, BAD, None) == wsg.ERR_ALIGN
    assert L.convert_bf16(None, 10, A16, None) == wsg.ERR_NULL


def test_residual_rmsnorm_argument_errors(L):
    A16, BAD = 0x10000, 0x10004
    f = L.residual_rmsnorm_q8_0
    assert f(A16, A16, A16, 40, 1e-6, A16, A16, A16, None) == wsg.ERR_SHAPE
    assert f(A16, A16, A16, -32, 1e-6, A16, A16, A16, None) == wsg.ERR_SHAPE
    assert f(A16, A16, A16, wsg.MAX_K_Q8ACT + 32, 1e-6, A16, A16, A16, None) == wsg.ERR_SHAPE
    assert f(A16, A16, A16, 64, 0.0, A16, A16, A16, None) == wsg.ERR_MODE
    assert f(A16, A16, A16, 64, -1e-6, A16, A16, A16, None) == wsg.ERR_MODE
    assert f(A16, A16, A16, 64, float("inf"), A16, A16, A16, None) == wsg.ERR_MODE
    assert f(A16, A16, A16, 64, float("nan"), A16, A16, A16, None) == wsg.ERR_MODE
    assert f(None, A16, A16, 64, 1e-6, A16, A16, A16, None) == wsg.ERR_NULL
    assert f(BAD, A16, A16, 64, 1e-6, A16, A16, A16, None) == wsg.ERR_ALIGN
    assert f(A16, BAD, A16, 64, 1e-6, A16, A16, A16, None) == wsg.ERR_ALIGN
    assert f(A16, A16, BAD, 64, 1e-6, A16, A16, A16, None) == wsg.ERR_ALIGN
    assert f(A16, A16, A16, 64, 1e-6, 0x10004, A16, A16, None) == wsg.ERR_ALIGN
    assert f(A16, A16, A16, 64, 1e-6, A16, 0x10004, A16, None) == wsg.ERR_ALIGN
    assert f(A16, A16, A16, 64, 1e-6, A16, A16, 0x10008, None) == wsg.ERR_ALIGN
    # nothing to write, or an empty vector: no launch, no error
    assert f(None, None, None, 64, 1e-6, None, None, None, None) == wsg.OK
    assert f(None, None, None, 0, 1e-6, A16, A16, A16, None) == wsg.OK


def test_lm_head_and_argmax_argument_errors(L):
    A16 = 0x10000
    ws = wsg.argmax_ws_bytes()
    assert L.lm_head_argmax(A16, 5, 10, 32, A16, 0, A16, ws, A16, None, None) == wsg.ERR_MODE
    assert L.lm_head_argmax(A16, 1, 0, 32, A16, 0, A16, ws, A16, None, None) == wsg.ERR_SHAPE
    assert L.lm_head_argmax(A16, 1, 10, 32, A16, 0, A16, 4, A16, None, None) == wsg.ERR_WORKSPACE
    # a workspace of exactly the per-shape size is accepted by validation
    # (the fake addresses then fail the idx_out check, so nothing launches)
    need = wsg.lm_head_argmax_ws_bytes(151936, 4096, wsg.W_Q8_0)
    assert L.lm_head_argmax(A16, 1, 151936, 4096, A16, 0, A16, need - 8, A16, None, None) == wsg.ERR_WORKSPACE
    assert L.lm_head_argmax(A16, 1, 151936, 4096, A16, 0, A16, need, 0x10002, None, None) == wsg.ERR_ALIGN
    assert L.lm_head_argmax(A16, 1, 10, 32, A16, 0, A16, ws, None, None, None) == wsg.ERR_NULL
    assert L.lm_head_argmax(A16, 1, 10, 32, A16, 0, 0x10004, ws, A16, None, None) == wsg.ERR_ALIGN
    assert L.argmax_f32(A16, 0, A16, ws, A16, None) == wsg.ERR_SHAPE
    assert L.argmax_f32(A16, 10, A16, 16, A16, None) == wsg.ERR_WORKSPACE


def test_plan_rejects_bad_descriptors_before_capture(L):
    A16 = 0x10000
    ops = [wsg.op_gemv_q8_0(A16, 4, 33, A16, wsg.ACT_Q8_0, A16)]
    with pytest.raises(wsg.WsgError) as e:
        wsg.Plan(ops, stream=0)
    assert e.value.status == wsg.ERR_SHAPE
    ops = [wsg.OpDesc(op=wsg.OP_GEMV_Q4_0_SWIGLU + 1)]
    with pytest.raises(wsg.WsgError) as e:
        wsg.Plan(ops, stream=0)
    assert e.value.status == wsg.ERR_MODE
    h = ctypes.c_void_p()
    assert L.wsg_plan_create(None, 1, None, ctypes.byref(h)) == wsg.ERR_NULL
    assert L.wsg_plan_launch(None, None) == wsg.ERR_NULL
    assert L.wsg_plan_kernel_count(None) == -1


def test_stream_config_reports_the_kernel_shape():
    import weight_streaming_gemv_q8_amd as wsg
    cfg = wsg.stream_config()
    # 16 waves per CU, and a ring of 1-chunk items that fits 128 VGPRs
    assert cfg["waves"] == 16 and cfg["unroll"] >= 1 and cfg["sets"] >= 2


def test_deq_mode_mapping():
    # emit_qwen38_generate: deq 0 = int8 activations everywhere, 1 = f32 for
    # the LM head only, 2 = f32 for every Q8_0 GEMV
    assert wsg.act_fmt_for(0, False) == wsg.ACT_F32_REQUANT
    assert wsg.act_fmt_for(0, True, fused_requant=False) == wsg.ACT_Q8_0
    assert wsg.act_fmt_for(1, False) == wsg.ACT_F32_REQUANT
    assert wsg.act_fmt_for(1, True) == wsg.ACT_F32
    assert wsg.act_fmt_for(2, False) == wsg.ACT_F32
    assert wsg.act_fmt_for(2, True) == wsg.ACT_F32
    with pytest.raises(ValueError):
        wsg.act_fmt_for(3, False)


def test_persistent_plan_rejections_before_launch(L):
    # validation happens before any allocation or launch (no GPU needed)
    h = ctypes.c_void_p()
    A16 = 0x10000
    bf16 = (wsg.OpDesc * 1)(wsg.op_gemv_bf16(A16, 4, 32, A16, A16))
    assert L.wsg_plan_create_persistent(None, 1, None, ctypes.byref(h)) == wsg.ERR_NULL
    assert L.wsg_plan_create_persistent(bf16, 0, None, ctypes.byref(h)) == wsg.ERR_SHAPE
    assert L.wsg_plan_create_persistent(bf16, 1, None, ctypes.byref(h)) == wsg.ERR_MODE  # not a Q8_0 GEMV
    assert not h.value


def test_fused_norm_gemv_rejects_before_launch(L):
    # fake, aligned device addresses: every case fails validation, so nothing
    # is launched (no GPU needed)
    A = 0x100000
    h, r, g, h_out, y = A, A + 0x10000, A + 0x20000, A + 0x30000, A + 0x40000
    f = L.gemv_q8_0_rmsnorm
    assert f(A, 0, 1024, h, r, g, 1e-6, h_out, y, None) == wsg.ERR_SHAPE          # n = 0
    assert f(A, 8, 0, h, r, g, 1e-6, h_out, y, None) == wsg.ERR_SHAPE             # k = 0
    assert f(A, 8, 1000, h, r, g, 1e-6, h_out, y, None) == wsg.ERR_SHAPE          # k % 32
    assert f(A, 8, wsg.MAX_K_Q8ACT + 32, h, r, g, 1e-6, h_out, y, None) == wsg.ERR_SHAPE
    assert f(A, 8, 1024, h, r, g, 0.0, h_out, y, None) == wsg.ERR_MODE            # eps
    assert f(A, 8, 1024, h, r, g, 1e-6, h, y, None) == wsg.ERR_MODE               # h_out over h
    assert f(A, 8, 1024, h, r, g, 1e-6, r + 64, y, None) == wsg.ERR_MODE          # h_out over r
    assert f(A, 8, 1024, h, r, g, 1e-6, h_out, g, None) == wsg.ERR_MODE           # y over g
    assert f(A, 8, 1024, h, r, g, 1e-6, h_out, h_out + 16, None) == wsg.ERR_MODE  # y over h_out
    assert f(A, 8, 1024, h + 4, r, g, 1e-6, h_out, y, None) == wsg.ERR_ALIGN
    assert f(A, 8, 1024, None, r, g, 1e-6, h_out, y, None) == wsg.ERR_NULL
    f32 = L.gemv_q8_0_rmsnorm_f32  # the deq 2 form: the same checks, the f32 staging limit
    assert f32(A, 8, wsg.MAX_K_F32ACT + 32, h, r, g, 1e-6, h_out, y, None) == wsg.ERR_SHAPE
    assert f32(A, 8, 1024, h, r, g, 1e-6, h, y, None) == wsg.ERR_MODE
    assert f32(A, 8, 1024, h, r, g, -1.0, h_out, y, None) == wsg.ERR_MODE


def test_swiglu_gemv_rejects_before_launch(L):
    A = 0x100000
    f = L.gemv_q8_0_swiglu
    assert f(A, 64, 1024, A, 7, A + 0x10000, None) == wsg.ERR_MODE                # not a format
    assert L.gemv_q4_0_swiglu(A, 64, 1024, A, wsg.ACT_F32, A + 0x10000, None) == wsg.ERR_MODE  # 4-bit: int8 only
    assert f(A, 64, wsg.MAX_K_F32ACT + 32, A, wsg.ACT_F32, A + 0x10000, None) == wsg.ERR_SHAPE  # f32 staging limit
    assert f(A, 0, 1024, A, wsg.ACT_F32_REQUANT, A + 0x10000, None) == wsg.ERR_SHAPE
    assert f(A, 64, 1000, A, wsg.ACT_F32_REQUANT, A + 0x10000, None) == wsg.ERR_SHAPE
    assert f(A, 64, 1024, None, wsg.ACT_Q8_0, A + 0x10000, None) == wsg.ERR_NULL
    assert f(A + 8, 64, 1024, A, wsg.ACT_Q8_0, A + 0x10000, None) == wsg.ERR_ALIGN


def test_w4_entry_points_reject_before_launch(L):
    A = 0x100000
    f = L.gemv_q4_0
    assert f(A, 64, 1024, A, 7, A + 0x10000, None) == wsg.ERR_MODE
    assert f(A, 0, 1024, A, wsg.ACT_F32, A + 0x10000, None) == wsg.ERR_SHAPE
    assert f(A, 64, 1000, A, wsg.ACT_Q8_0, A + 0x10000, None) == wsg.ERR_SHAPE
    # the f32 (W4A16) form stages the activation as f32: its smaller k limit
    assert f(A, 64, 40960, A, wsg.ACT_F32, A + 0x10000, None) == wsg.ERR_SHAPE
    assert f(A, 64, 57376, A, wsg.ACT_F32_REQUANT, A + 0x10000, None) == wsg.ERR_SHAPE
    assert f(A, 64, 1024, None, wsg.ACT_F32, A + 0x10000, None) == wsg.ERR_NULL
    assert f(A + 8, 64, 1024, A, wsg.ACT_F32, A + 0x10000, None) == wsg.ERR_ALIGN
    assert L.q4_0_row_bytes(2048) == 1152 and L.q4_0_row_bytes(96) == 16 + 48
    assert L.q4_0_row_bytes(1000) == -1 and L.q4_0_packed_bytes(-1, 64) == -1
    assert L.quantize_q4_0_weights(A, 4, 1000, A, None) == wsg.ERR_SHAPE
    fn = L.gemv_q4_0_rmsnorm
    assert fn(A, 64, 1000, A, None, None, 1e-6, None, A + 0x10000, None) == wsg.ERR_SHAPE
    assert fn(A, 64, 1024, A, None, None, 0.0, None, A + 0x10000, None) == wsg.ERR_MODE
    fs = L.gemv_q4_0_swiglu
    assert fs(A, 64, 1024, A, wsg.ACT_F32, A + 0x10000, None) == wsg.ERR_MODE
    assert fs(A, 64, 1000, A, wsg.ACT_Q8_0, A + 0x10000, None) == wsg.ERR_SHAPE
    assert fs(A, 64, 1024, None, wsg.ACT_Q8_0, A + 0x10000, None) == wsg.ERR_NULL
