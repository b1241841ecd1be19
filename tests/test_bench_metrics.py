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


def _write_csv(path, header, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=header)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_kernel_labels_from_rocprof_names():
    ns = "void wsg::(anonymous namespace)::"
    cases = {
        "q8_i8_kernel<8, 1, 1, 2, true, false, false>(unsigned char const*)": "q8_i8_kernel<waves=8,split=1,unroll=1,requant>",
        "q8_i8_kernel<8, 1, 1, 0, true, false, true>(unsigned char const*)": "q8_i8_kernel<waves=8,split=1,unroll=1,q8act,argmax>",
        "q8_f32_kernel<16, 4, 1, true, false>(unsigned char const*)": "q8_f32_kernel<waves=16,split=4,unroll=1,f32act>",
        "q8_f32_norm_kernel<8, 1>(unsigned char const*)": "q8_f32_norm_kernel<waves=8,split=1>",
        "q8_i8_swiglu_kernel<8, 1>(unsigned char const*)": "q8_i8_swiglu_kernel<waves=8,f32act>",
        "q4_i8_kernel<16, 1, 2>(unsigned char const*)": "q4_i8_kernel<waves=16,split=1,requant>",
        "stream_kernel<16, 1, 3, false>(wsg::StreamOp const*, int, unsigned int*, int)": "stream_kernel<waves=16,unroll=1,sets=3,requant>",
    }
    for raw, lab in cases.items():
        assert bench.label_from_rocprof(ns + raw) == lab
        assert bench.short_kernel_name(ns + raw) == lab
    assert bench.label_from_rocprof(ns + "argmax_stage2_kernel(unsigned long const*, int, int*)") is None
    assert bench.short_kernel_name(ns + "argmax_stage2_kernel(unsigned long const*, int, int*)") == "argmax_stage2_kernel"


def test_profile_summary_groups_by_grid_and_calibrates(tmp_path, monkeypatch):
    """Per-(kernel, grid) statistics from a kernel trace, and per-launch
    bytes from counter runs scaled by the copy probe's known traffic."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    k = "void wsg::(anonymous namespace)::q8_i8_kernel<8, 1, 1, 2, true, false, false>(unsigned char const*)"
    copy = "wsg::(anonymous namespace)::copy_probe_kernel(int4v const*, int4v*, long)"
    th = ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"]
    trace = [{"Kernel_Name": k, "Grid_Size_X": 512 * 512, "Workgroup_Size_X": 512, "Start_Timestamp": 0,
              "End_Timestamp": d} for d in (16000, 17000, 15000)]
    trace += [{"Kernel_Name": k, "Grid_Size_X": 484 * 512, "Workgroup_Size_X": 512, "Start_Timestamp": 0,
               "End_Timestamp": 32000}]
    _write_csv(str(tmp_path / "s" / "run_kernel_trace.csv"), th, trace)
    ch = ["Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value"]

    def counters(d, name, vals):
        _write_csv(str(tmp_path / d / "run_counter_collection.csv"), ch,
                   [{"Kernel_Name": kn, "Grid_Size": g * 512, "Workgroup_Size": 512, "Counter_Name": name,
                     "Counter_Value": v} for kn, g, v in vals])

    counters("f", "FETCH_SIZE", [(k, 512, 1000.0), (k, 512, 1200.0), (k, 484, 3000.0)])
    counters("w", "WRITE_SIZE", [(k, 512, 10.0), (k, 512, 10.0), (k, 484, 20.0)])
    counters("cf", "FETCH_SIZE", [(copy, 2048, 512.0)])    # 1 MiB copy read, counter shows half
    counters("cw", "WRITE_SIZE", [(copy, 2048, 1024.0)])
    cmds = {"stats": "S", "fetch": "F", "write": "W", "copy_fetch": "CF", "copy_write": "CW", "probe_bytes": 1 << 20}
    out = bench.summarize_profiles(*(str(tmp_path / d) for d in ("s", "f", "w", "cf", "cw")),
                                   workload="wl", commands=cmds)
    stats = open(out[0]).read().splitlines()
    rows = [l.split() for l in stats if not l.startswith("#")]
    assert [(r[0], r[1], r[2]) for r in rows] == [("3", "512", "16.00"), ("1", "484", "32.00")]
    lab = "q8_i8_kernel<waves=8,split=1,unroll=1,requant>"
    got, refs = bench.profile_refs(lab, "wl")
    # fetch factor 2 (the counter read half the copy's bytes), write factor 1; KiB -> bytes
    assert got == round((1000 + 1200 + 3000) / 3 * 2 * 1024 + (10 + 10 + 20) / 3 * 1024)
    assert refs["stats"] == "profiles/kernel_stats_wl.txt" and refs["traffic"].endswith("_wl.txt")
    assert bench.profile_refs(lab, "other") == (None, {"stats": None, "traffic": None})


def test_config_parts_cover_every_workload_once():
    names = bench.config_part_names()
    assert names[0] == "small" and len(set(names)) == len(names)
    streams = [n for n in names if n.startswith("stream:")]
    # BF16 chains have no fused norm or SwiGLU form; Q8_0 ones have all four
    assert {n.rsplit(":", 1)[1] for n in streams if "bf16" in n} == {"plain", "norm"}
    assert {n.rsplit(":", 1)[1] for n in streams if "q8_0" in n} == {"plain", "norm", "fused_norm", "swiglu"}
    assert any(n.startswith("stream:dense27b_q8_0_64L:deq2:") for n in names)
    assert [n for n in names if n.startswith("w4:")] == ["w4:0", "w4:1", "w4:2", "w4:3"]
    assert [n for n in names if n.startswith("decode:")] == ["decode:0", "decode:1", "decode:2", "decode:3"]


def test_unknown_configs_part_is_refused_before_the_gpu():
    import subprocess
    import sys
    p = subprocess.run([sys.executable, bench.__file__, "--configs", "--configs-part", "nope"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2 and "unknown configs part" in p.stderr


def test_boundary_summary_pairs_consecutive_kernels(tmp_path, monkeypatch):
    """Graph-plan runs also get profiles/boundaries_<workload>.txt: per
    boundary (kernel, grid -> next), the traced duration, the period to the
    next start and the gap; repeated shapes (per-shape graphs) and
    dispatches far apart (host work between replays) are not boundaries."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    a = "void wsg::(anonymous namespace)::q8_i8_kernel<16, 1, 1, 2, true, false, false>(unsigned char const*)"
    b = "void wsg::(anonymous namespace)::q8_i8_kernel<16, 4, 1, 2, true, false, false>(unsigned char const*)"
    th = ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"]
    trace, t = [], 0
    for _ in range(3):  # a token of two GEMVs, three replays back to back: a 20 us then b 10 us, 1 us gaps
        trace.append({"Kernel_Name": a, "Grid_Size_X": 256 * 1024, "Workgroup_Size_X": 1024,
                      "Start_Timestamp": t, "End_Timestamp": t + 20000})
        trace.append({"Kernel_Name": b, "Grid_Size_X": 256 * 1024, "Workgroup_Size_X": 1024,
                      "Start_Timestamp": t + 21000, "End_Timestamp": t + 31000})
        t += 32000
    t += 5_000_000  # a per-shape graph later: the same kernel repeated
    for _ in range(4):
        trace.append({"Kernel_Name": a, "Grid_Size_X": 256 * 1024, "Workgroup_Size_X": 1024,
                      "Start_Timestamp": t, "End_Timestamp": t + 20000})
        t += 20000
    _write_csv(str(tmp_path / "s" / "run_kernel_trace.csv"), th, trace)
    out = bench.summarize_profiles(str(tmp_path / "s"), "-", "-", "-", "-", workload="wl_graph",
                                   commands={"stats": "S"})
    bpath = [p for p in out if "boundaries_wl_graph" in p]
    assert len(bpath) == 1
    rows = [l.split() for l in open(bpath[0]) if not l.startswith("#")]
    got = {(r[4], r[8]): (int(r[0]), float(r[1]), float(r[2]), float(r[3])) for r in rows}
    sa = "q8_i8_kernel<waves=16,split=1,unroll=1,requant>"
    sb = "q8_i8_kernel<waves=16,split=4,unroll=1,requant>"
    assert got[(sa, sb)] == (3, 20.0, 21.0, 1.0)
    assert got[(sb, sa)] == (2, 10.0, 11.0, 1.0)  # the third b is followed by the far-away graph
    assert len(got) == 2
