"""The bench's arithmetic and the workload shapes reproduce the figures the
pages print (tests/golden/pages_figures.json)."""
import json
import os

import pytest

import bench
from synth import workloads as W

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def test_tokens_per_s_closed_form():
    for key in ("tokens_per_s_w4", "tokens_per_s_fp8"):
        g = GOLD[key]
        assert round(bench.tokens_per_s(g["bandwidth_gbps"], g["bytes_per_token_gb"])) == g["printed"]


def test_dequant_op_rate_closed_form():
    g = GOLD["dequant_op_rate"]
    r = bench.dequant_op_rate_tflops(g["bandwidth_gbps"], g["bytes_per_weight"], g["ops_per_weight"])
    assert round(r) == g["printed_tflops"]
    assert r == pytest.approx(3.953, abs=1e-3)


def test_dense27b_stream_bytes():
    g = GOLD["dense27b_bytes_per_token"]
    b = W.DENSE27B_Q8.weight_bytes()
    assert b == 26_738_688_000
    assert abs(b / 1e9 - g["printed_gb"]) / g["printed_gb"] < 0.02


def test_concatenated_shapes():
    g = GOLD["concatenated_rows"]
    m = {x.name: x for x in W.DENSE27B_Q8.matrices}
    assert m["qkvz"].n == g["qkvz"] and m["gate_up"].n == g["gate_up"]
    assert sum(m["gate_up"].parts) == g["gate_up"]


def test_qwen3_8b_qkv_width():
    g = GOLD["qwen3_8b_heads"]
    qkv = W.QWEN3_8B_Q8.matrices[0]
    head_dim = 128
    assert qkv.parts == (g["q_heads"] * head_dim, g["kv_heads"] * head_dim, g["kv_heads"] * head_dim)


def test_workload_bytes_table():
    assert W.Q8_SINGLE.weight_bytes() == 1_114_112
    assert W.QWEN3_0P6B_BF16.weight_bytes() == 880_803_840
    assert W.QWEN3_8B_Q8.weight_bytes() == 7_379_877_888
    lm = W.LM_HEAD.matrices[0]
    assert lm.n * lm.k * 2 == 1_244_659_712
    assert lm.n * (lm.k // 32) * 34 == 661_225_472


def test_gbps_and_multi_gpu_refusal(capsys):
    assert bench.gbps(8e9, 1.0) == 8.0
    import sys
    argv = sys.argv
    sys.argv = ["bench.py", "--gpus", "8"]
    try:
        assert bench.main() == 2
    finally:
        sys.argv = argv
    assert "one GPU" in capsys.readouterr().err
