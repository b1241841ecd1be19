#!/usr/bin/env python3
"""Bench: the whole-token batch-1 decode GEMV weight stream on one MI355X.

One step = one replay of the captured token: every weight matrix of one
token streamed once (emit_qwen38_generate, "Where the speed comes from":
~27 GB of Q8_0 weights per token, one GEMV per concatenated projection, one
graph per token).  Default plan: one hipGraph node per GEMV, replayed
(the faster plan at deq 0 on this part); --plan persistent runs the whole
token as one resident kernel instead (captured as a one-node hipGraph).
Default workload: the 27B-scale Q8_0 stream (64 layers x
qkvz 16384x5120, out 5120x8192, gate+up 34816x5120, down 5120x17408), int8
activations (deq 0) requantized inside each GEMV.  Weights are synthetic
(seeded ~N(0, 0.02), quantized on the device) and resident in HBM before
timing starts.

Prints ONE JSON line: achieved HBM GB/s over the stream (algorithmic weight
bytes / time), microseconds per token stream, the roofline of the dominant
kernel (the token kernel itself, or per GEMV instantiation for the graph
plan, from HIP events on the launch stream), and the CPU oracle timed on a
bounded sample on the host.  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "weight_streaming_gemv_q8_amd", "csrc")


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------ arithmetic
# Closed forms used by the pages (pinned in tests/test_bench_metrics.py).

def tokens_per_s(bandwidth_gbps: float, bytes_per_token_gb: float) -> float:
    """Batch-1 decode rate when the weight stream is the whole cost."""
    return bandwidth_gbps / bytes_per_token_gb


def dequant_op_rate_tflops(bandwidth_gbps: float, bytes_per_weight: float, ops_per_weight: float) -> float:
    """Float ops per second the dequantizing GEMV form needs at a given stream rate."""
    return bandwidth_gbps / bytes_per_weight * ops_per_weight / 1000.0


def gbps(nbytes: float, seconds: float) -> float:
    return nbytes / seconds / 1e9


def source_digest() -> str:
    """Hash of every kernel source: counters taken on other sources are stale."""
    h = hashlib.sha256()
    for fn in sorted(os.listdir(CSRC)):
        if fn.endswith((".hip", ".hpp", ".cpp")):
            with open(os.path.join(CSRC, fn), "rb") as f:
                h.update(fn.encode() + b"\0" + f.read())
    return h.hexdigest()


def read_traffic(kernel_name: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters for this kernel
    in this workload (profiles/traffic_*.txt), or None if absent or taken
    on other sources."""
    if not os.path.isdir(PROFILES):
        return None
    digest = source_digest()
    for fn in sorted(os.listdir(PROFILES)):
        if not (fn.startswith("traffic_") and fn.endswith(".txt")):
            continue
        kv = {}
        with open(os.path.join(PROFILES, fn)) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    a, b = line.split(":", 1)
                    kv[a.strip()] = b.strip()
        if kv.get("kernel") == kernel_name and kv.get("workload") == workload and kv.get("source_sha256") == digest:
            try:
                return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"]), fn
            except (KeyError, ValueError):
                return None
    return None


def profile_refs(kernel_name: str, workload: str):
    """The roofline's traffic figure and the committed rocprofv3 summaries
    behind it (kernel statistics, counters) for this kernel and workload."""
    t = read_traffic(kernel_name, workload)
    stats = f"kernel_stats_{workload}.txt"
    refs = {"stats": f"profiles/{stats}" if os.path.exists(os.path.join(PROFILES, stats)) else None,
            "traffic": f"profiles/{t[1]}" if t else None}
    return (round(t[0]) if t else None), refs


# ------------------------------------------------------------ workload

def build_stream(wl, deq: int, requant: str, norm: bool = False, fused_norm: bool = False, swiglu: bool = False,
                 wtype: str = None):
    """The workload's token stream with its weights generated on the device.
    norm=True chains the layers through the residual stream: a residual add
    + RMSNorm + re-quantization call before each layer's attention input
    (GEMV 0) and MLP input (GEMV 2); fused_norm=True computes that step in
    the GEMV's prologue instead (int8 Q8_0 streams); wtype overrides the
    workload's weight format (\"q4_0\": the same shapes in 4 bits)."""
    import torch

    import synth
    from synth import workloads as W
    from weight_streaming_gemv_q8_amd.stream import TokenStream

    shapes = [(m.n, m.k, m.parts) for m in wl.matrices]
    ts = TokenStream(shapes, wl.layers, wtype or wl.wtype, deq=deq, requant=requant,
                     norm_before=(0, 2) if norm else (), eps=W.RMSNORM_EPS, fused_norm=fused_norm,
                     swiglu_at=(2,) if swiglu else ())
    log(f"allocated {ts.weight_bytes_alloc / 1e9:.3f} GB of weights; generating on the device")
    t0 = time.time()

    def fill(layer, m, part, rows, staging):
        synth.dev_normal_f32(staging.data_ptr(), wl.seed, W.weight_tensor_id(layer, m, part),
                             rows * wl.matrices[m].k, W.WEIGHT_SIGMA,
                             stream=torch.cuda.current_stream().cuda_stream)

    ts.fill_weights(fill)
    k0 = wl.matrices[0].k
    xs = [synth.activation(wl.seed, W.activation_tensor_id(l), k0, rms=True) for l in range(wl.layers)]
    import numpy as np
    ts.set_inputs(torch.from_numpy(np.stack(xs)).cuda())
    if norm:
        h0 = synth.normal_f32(wl.seed, W.RESIDUAL_TENSOR_ID, ts.hidden, 1.0)
        gains = np.stack([np.float32(1.0) + synth.normal_f32(wl.seed, W.gain_tensor_id(i), ts.hidden, W.GAIN_SIGMA)
                          for i in range(len(ts.norms))]).astype(np.float32)
        ts.set_residual_input(torch.from_numpy(h0).cuda(), torch.from_numpy(gains).cuda())
    torch.cuda.synchronize()
    log(f"weights ready in {time.time() - t0:.1f} s")
    return ts


def kernel_label(wtype: str, act_fmt: int, cfg: dict) -> str:
    import weight_streaming_gemv_q8_amd as wsg
    if wtype == "bf16":
        base = "bf16_kernel"
    elif act_fmt == wsg.ACT_F32:
        base = "q8_f32_kernel"
    else:
        base = "q8_i8_kernel"
    act = {wsg.ACT_Q8_0: "q8act", wsg.ACT_F32: "f32act", wsg.ACT_F32_REQUANT: "requant"}[act_fmt]
    return f"{base}<waves={cfg['waves']},split={cfg['split']},unroll={cfg['unroll']},{act}>"


def time_plan(ts, plan_kind, steps: int, warmup: int, stats: dict = None):
    """Capture the token ("graph": one node per call; "persistent": one
    resident kernel) and time `steps` replays with HIP events on the launch
    stream (an event between consecutive replays, so each replay's time is
    known too: stats, if given, receives their median and min in
    seconds).  Returns (mean seconds per token, kernels per token)."""
    import torch
    if plan_kind is True or plan_kind is False:  # older callers: persistent or not
        plan_kind = "persistent" if plan_kind else "graph"
    persistent = plan_kind != "graph"
    plan = ts.capture(persistent=persistent)
    kernels = plan.kernel_count
    for _ in range(warmup):
        ts.launch()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        ts.launch()
        ev[i + 1].record()
    torch.cuda.synchronize()
    if persistent and plan.error():
        raise RuntimeError(f"a wait of the {plan_kind} token kernel timed out: results invalid")
    per = sorted(ev[i].elapsed_time(ev[i + 1]) / 1e3 for i in range(steps))
    if stats is not None:
        stats["median_s"] = per[len(per) // 2]
        stats["min_s"] = per[0]
        stats["replays"] = steps
    return ev[0].elapsed_time(ev[steps]) / 1e3 / steps, kernels


def time_per_shape(ts, wtype_code: int, act_fmt: int, reps: int):
    """Every GEMV shape of the layer as it runs in the token: a graph of the
    L launches of that matrix (one per layer: that layer's weights and
    input buffers, the same kernel and launch shape as in the token),
    replayed `reps` times with HIP events on the launch stream.  Returns one
    record per shape: kernel label, n, k, algorithmic bytes and seconds per
    launch."""
    import torch

    import weight_streaming_gemv_q8_amd as wsg
    out = []
    per_layer = len(ts.slots) // ts.layers
    for j in range(per_layer):
        slots = [s for s in ts.slots if s.index == j]
        ops = []
        for s in slots:
            ops.extend(ts._slot_ops(s))
        plan = wsg.Plan(ops)
        for _ in range(2):
            plan.launch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            plan.launch()
        e1.record()
        torch.cuda.synchronize()
        plan.destroy()
        sec = e0.elapsed_time(e1) / 1e3 / (reps * len(slots))
        n, k = slots[0].n, slots[0].k
        cfg = wsg.gemv_config(wtype_code, act_fmt, n, k)
        bpl = {"q8_0": n * (k // 32) * 34, "q4_0": n * (k // 32) * 18}.get(ts.wtype, n * k * 2)
        out.append({"matrix": j, "n": n, "k": k, "label": kernel_label(ts.wtype, act_fmt, cfg), "grid": cfg["grid"],
                    "bytes": bpl, "us": sec * 1e6, "launches_per_token": len(slots), "kernels_per_launch": len(ops) // len(slots)})
    return out


def _time_calls(fn, reps: int, warmup: int = 3) -> float:
    """Seconds per call: HIP events around `reps` back-to-back calls."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps


def _stream_configs(W):
    return ((W.QWEN3_0P6B_BF16, (0,)), (W.QWEN3_8B_Q8, (0,)), (W.DENSE27B_Q8, (0, 2)))


# the 27B stream with 4-bit weights: int8 activations (deq 0) and f32 ones
# (deq 2, W4A16); at deq 0 also with the norm prologue and the SwiGLU epilogue
_W4_CONFIGS = ((0, "", {}), (2, " (W4A16)", {}),
               (0, " + residual/RMSNorm fused into the GEMVs", {"norm": True, "fused_norm": True}),
               (0, " + SwiGLU epilogue on gate+up", {"swiglu": True}))


def _decode_configs(W):
    return ((W.QWEN3_8B_Q8, "q8_0", 0), (W.DENSE27B_Q8, "q8_0", 0), (W.DENSE27B_Q8, "q8_0", 2),
            (W.DENSE27B_Q8, "q4_0", 0))


def config_part_names() -> list:
    """The parts of the configs run, in order (no GPU needed): the small
    workloads together, then each token stream, 4-bit stream and decode
    step on its own."""
    from synth import workloads as W
    names = ["small"]
    for wl, deqs in _stream_configs(W):
        for deq in deqs:
            variants = ("plain", "norm") + (("fused_norm", "swiglu") if wl.wtype == "q8_0" else ())
            names += [f"stream:{wl.name}:deq{deq}:{v}" for v in variants]
    names += [f"w4:{i}" for i in range(len(_W4_CONFIGS))]
    names += [f"decode:{i}" for i in range(len(_decode_configs(W)))]
    return names


def run_configs_in_children(steps: int, warmup: int) -> int:
    """The configs run with each part in a child process of its own, one
    after another.  A token stream's speed depends on the state its weights
    are allocated in: the first 26.7 GB allocation of a process streams ~3.5%
    faster than one made after another stream was freed (27B stream: 4783
    against 4974 us per token in one process).  A fresh process per part
    measures each the way a server allocates its weights once, at start-up.
    This process never touches the GPU."""
    import subprocess
    for name in config_part_names():
        cmd = [sys.executable, os.path.abspath(__file__), "--configs", "--configs-part", name,
               "--steps", str(steps), "--warmup", str(warmup)]
        p = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
        for line in p.stdout.splitlines():
            if line.startswith("{"):
                print(line, flush=True)
        if p.returncode != 0:
            print(f"configs part {name} failed with status {p.returncode}", file=sys.stderr)
            return p.returncode
    return 0


def measure_configs(steps: int, warmup: int, part: str = None) -> list:
    """Every workload in the way the pages run it: the single GEMV as eager
    calls (hot: one weight copy; cold: rotating over 1024 copies, more than
    L2 + MALL), the LM head as fused GEMV + argmax calls, the token streams
    as graph and persistent replays.  One record per configuration and
    mode.  part: one of config_part_names() (None: all of them, in this
    process)."""
    import numpy as np
    import torch

    import synth
    import weight_streaming_gemv_q8_amd as wsg
    from synth import workloads as W

    out = []
    want = lambda name: part is None or part == name

    def rec(wl, mode, sec, alg_bytes, **extra):
        gbps_ = gbps(alg_bytes, sec)
        r = {"workload": wl.name, "mode": mode, "us": round(sec * 1e6, 2), "GBps": round(gbps_, 1),
             "frac_of_peak": round(gbps_ / HBM_PEAK_GBPS, 4), "bytes": alg_bytes, **extra}
        log(f"{wl.name:22s} {mode:34s} {sec * 1e6:10.2f} us {gbps_:8.1f} GB/s {100 * gbps_ / HBM_PEAK_GBPS:5.1f}%")
        out.append(r)

    def small_workloads(steps, rec, s):
        # configs 0: one 1024x1024 Q8_0 GEMV
        wl = W.Q8_SINGLE
        n, k = wl.matrices[0].n, wl.matrices[0].k
        alg = n * (k // 32) * 34
        staging = torch.empty(n * k, dtype=torch.float32, device="cuda")
        copies = 1024
        wq = torch.empty((copies, wsg.q8_0_packed_bytes(n, k)), dtype=torch.uint8, device="cuda")
        for c in range(copies):
            synth.dev_normal_f32(staging.data_ptr(), wl.seed, 1 + c, n * k, W.WEIGHT_SIGMA, stream=s)
            wsg.quantize_q8_0_weights(staging, n, k, wq[c])
        x = torch.from_numpy(synth.activation(wl.seed, W.activation_tensor_id(0), k)).cuda()
        y = torch.empty(n, dtype=torch.float32, device="cuda")
        for deq, act in ((0, wsg.ACT_F32_REQUANT), (2, wsg.ACT_F32)):
            for temp, pick in (("hot", lambda i: 0), ("cold", lambda i: i % copies)):
                sec = _time_calls(lambda i: wsg.gemv_q8_0(wq[pick(i)], n, k, x, act, y), max(steps, 1) * 40)
                rec(wl, f"eager deq{deq} {temp}", sec, alg, deq=deq)
                # the same calls replayed from a graph of 256: the kernel without
                # the host's launch cost
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(256):
                        wsg.gemv_q8_0(wq[pick(i)], n, k, x, act, y)
                sec = _time_calls(lambda i: g.replay(), max(steps, 1) // 5 + 1) / 256
                rec(wl, f"graph of 256 calls deq{deq} {temp}", sec, alg, deq=deq)
                del g
        del wq, staging
        # configs 3: the LM head, fused GEMV + two-stage argmax
        wl = W.LM_HEAD
        n, k = wl.matrices[0].n, wl.matrices[0].k
        staging = torch.empty(n * k, dtype=torch.float32, device="cuda")
        synth.dev_normal_f32(staging.data_ptr(), wl.seed, 1, n * k, W.WEIGHT_SIGMA, stream=s)
        wb = torch.empty(n * k, dtype=torch.uint16, device="cuda")
        wsg.convert_bf16(staging, n * k, wb)
        wq = torch.empty(wsg.q8_0_packed_bytes(n, k), dtype=torch.uint8, device="cuda")
        wsg.quantize_q8_0_weights(staging, n, k, wq)
        del staging
        x = torch.from_numpy(synth.activation(wl.seed, W.activation_tensor_id(0), k)).cuda()
        ws = torch.empty(wsg.argmax_ws_bytes(), dtype=torch.uint8, device="cuda")
        idx = torch.empty(1, dtype=torch.int32, device="cuda")
        sec = _time_calls(lambda i: wsg.lm_head_argmax(wb, wsg.W_BF16, n, k, x, wsg.ACT_F32, ws, ws.numel(), idx),
                          max(steps, 1))
        rec(wl, "bf16 GEMV + argmax", sec, n * k * 2)
        for deq, act in ((0, wsg.ACT_F32_REQUANT), (2, wsg.ACT_F32)):
            sec = _time_calls(lambda i: wsg.lm_head_argmax(wq, wsg.W_Q8_0, n, k, x, act, ws, ws.numel(), idx),
                              max(steps, 1))
            rec(wl, f"q8_0 GEMV + argmax, deq{deq}" + (" (= deq1)" if deq == 2 else ""), sec, n * (k // 32) * 34,
                deq=deq)
        # the same matrix with 4-bit weights (18 bytes per 32 weights)
        staging = torch.empty(n * k, dtype=torch.float32, device="cuda")
        synth.dev_normal_f32(staging.data_ptr(), wl.seed, 1, n * k, W.WEIGHT_SIGMA, stream=s)
        w4 = torch.empty(wsg.q4_0_packed_bytes(n, k), dtype=torch.uint8, device="cuda")
        wsg.quantize_q4_0_weights(staging, n, k, w4)
        del staging
        y4 = torch.empty(n, dtype=torch.float32, device="cuda")
        sec = _time_calls(lambda i: wsg.gemv_q4_0(w4, n, k, x, wsg.ACT_F32_REQUANT, y4), max(steps, 1) * 4)
        rec(wl, "q4_0 GEMV (W4), deq0", sec, n * (k // 32) * 18, deq=0)
        del wb, wq, w4
        torch.cuda.empty_cache()
        # the residual add + RMSNorm + re-quantization between GEMVs, alone, at
        # the hidden sizes of the streams (bytes: h, r, g read; h', y written;
        # y_q8 written)
        for hidden in (1024, 4096, 5120):
            h = torch.from_numpy(synth.normal_f32(0x5EED0009, 0, hidden, 1.0)).cuda()
            r = torch.from_numpy(synth.normal_f32(0x5EED0009, 1, hidden, 0.5)).cuda()
            g = torch.ones(hidden, dtype=torch.float32, device="cuda")
            h_out = torch.empty_like(h)
            yv = torch.empty_like(h)
            yq = torch.empty(wsg.act_q8_0_bytes(hidden), dtype=torch.uint8, device="cuda")
            nbytes = 20 * hidden + wsg.act_q8_0_bytes(hidden)
            call = lambda i: wsg.residual_rmsnorm_q8_0(h, r, g, hidden, W.RMSNORM_EPS, h_out, yv, yq)
            sec = _time_calls(call, max(steps, 1) * 40)
            out.append({"workload": f"residual_rmsnorm_q8_0_k{hidden}", "mode": "eager", "us": round(sec * 1e6, 2),
                        "bytes": nbytes})
            log(f"residual_rmsnorm k={hidden:5d} eager {sec * 1e6:8.2f} us")
            g_ = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_):
                for i in range(256):
                    call(i)
            sec = _time_calls(lambda i: g_.replay(), max(steps, 1) // 5 + 1) / 256
            out.append({"workload": f"residual_rmsnorm_q8_0_k{hidden}", "mode": "graph of 256 calls",
                        "us": round(sec * 1e6, 2), "bytes": nbytes})
            log(f"residual_rmsnorm k={hidden:5d} graph {sec * 1e6:8.2f} us")
            del g_

    s = torch.cuda.current_stream().cuda_stream
    if want("small"):
        small_workloads(steps, rec, s)
    # configs 1, 2, 4: token streams
    for wl, deqs in _stream_configs(W):
        for deq in deqs:
            name = f"stream:{wl.name}:deq{deq}"
            alg = None
            if want(f"{name}:plain"):
                ts = build_stream(wl, deq, "fused")
                alg = ts.algorithmic_weight_bytes()
                plans = ("graph",) if wl.wtype == "bf16" else ("graph", "persistent")
                for plan in plans:
                    sec, kernels = time_plan(ts, plan, steps, warmup)
                    rec(wl, f"{plan} deq{deq}" if wl.wtype != "bf16" else plan, sec, alg, kernels_per_token=kernels,
                        deq=deq)
                ts.close()
                del ts
                torch.cuda.empty_cache()
            # the same stream with the layers chained through the residual
            # stream (a residual add + RMSNorm call before GEMVs 0 and 2)
            if want(f"{name}:norm"):
                ts = build_stream(wl, deq, "fused", norm=True)
                sec, kernels = time_plan(ts, False, steps, warmup)
                rec(wl, f"graph + residual/RMSNorm deq{deq}" if wl.wtype != "bf16" else "graph + residual/RMSNorm",
                    sec, ts.algorithmic_weight_bytes(), kernels_per_token=kernels, deq=deq)
                ts.close()
                del ts
                torch.cuda.empty_cache()
            if wl.wtype != "q8_0":
                continue
            # the same chain with the norm step in each normalized GEMV's prologue
            if want(f"{name}:fused_norm"):
                ts = build_stream(wl, deq, "fused", norm=True, fused_norm=True)
                sec, kernels = time_plan(ts, False, steps, warmup)
                rec(wl, f"graph + residual/RMSNorm fused into the GEMVs deq{deq}", sec, ts.algorithmic_weight_bytes(),
                    kernels_per_token=kernels, deq=deq)
                ts.close()
                del ts
                torch.cuda.empty_cache()
            # down reading the SwiGLU of gate+up (the epilogue fused into that GEMV)
            if want(f"{name}:swiglu"):
                ts = build_stream(wl, deq, "fused", swiglu=True)
                sec, kernels = time_plan(ts, False, steps, warmup)
                rec(wl, f"graph + SwiGLU epilogue on gate+up deq{deq}", sec, ts.algorithmic_weight_bytes(),
                    kernels_per_token=kernels, deq=deq)
                ts.close()
                del ts
                torch.cuda.empty_cache()
    for i, (deq, extra, kw) in enumerate(_W4_CONFIGS):
        if not want(f"w4:{i}"):
            continue
        ts = build_stream(W.DENSE27B_Q8, deq, "fused", wtype="q4_0", **kw)
        sec, kernels = time_plan(ts, False, steps, warmup)
        rec(W.DENSE27B_Q8, f"graph, W4 weights (q4_0){extra} deq{deq}", sec, ts.algorithmic_weight_bytes(),
            kernels_per_token=kernels, deq=deq)
        ts.close()
        del ts
        torch.cuda.empty_cache()
    # a whole decode step: embedding -> layers -> LM head + argmax -> advance
    for i, (wl, wt, deq) in enumerate(_decode_configs(W)):
        if not want(f"decode:{i}"):
            continue
        ds = build_decode(wl, wtype=wt, deq=deq)
        alg = ds.chain.algorithmic_weight_bytes() + ds.vocab * (ds.hidden // 32) * 34
        ds.capture()
        for _ in range(warmup):
            ds.launch()
        sec = _time_calls(lambda i: ds.launch(), steps, 0)
        rec(wl, "decode step graph (embedding, norms, SwiGLU, LM head + argmax, token advance), vocab 151936"
            + (", 4-bit layers" if wt == "q4_0" else "") + f", deq{deq}", sec, alg,
            kernels_per_token=ds.plan.kernel_count, deq=deq)
        ds.close()
        del ds
        torch.cuda.empty_cache()
    return out


def build_decode(wl, vocab: int = 151936, wtype: str = "q8_0", deq: int = 0):
    """A whole decode step on the workload's layer shapes (DecodeStep):
    embedding gather -> the layers with the residual stream (norms fused
    into the attention-input GEMVs, SwiGLU on gate+up) -> final norm ->
    LM head + argmax -> token/position advance, weights generated on the
    device."""
    import numpy as np
    import torch

    import synth
    from synth import workloads as W
    from weight_streaming_gemv_q8_amd.stream import DecodeStep

    shapes = [(m.n, m.k, m.parts) for m in wl.matrices]
    ds = DecodeStep(shapes, wl.layers, vocab, capacity=4096, eps=W.RMSNORM_EPS, wtype=wtype, deq=deq)
    stream = torch.cuda.current_stream().cuda_stream

    def fill(layer, m, part, rows, staging):
        synth.dev_normal_f32(staging.data_ptr(), wl.seed, W.weight_tensor_id(layer, m, part),
                             rows * wl.matrices[m].k, W.WEIGHT_SIGMA, stream=stream)

    ds.chain.fill_weights(fill)
    h = ds.hidden
    ds.fill_table(ds.embedding, lambda r0, st: synth.dev_normal_f32(st.data_ptr(), wl.seed, W.EMBEDDING_TENSOR_ID,
                                                                     st.numel(), 1.0, first=r0 * h, stream=stream))
    ds.fill_table(ds.lm_head, lambda r0, st: synth.dev_normal_f32(st.data_ptr(), wl.seed, W.LM_HEAD_TENSOR_ID,
                                                                   st.numel(), W.WEIGHT_SIGMA, first=r0 * h,
                                                                   stream=stream))
    gains = np.stack([np.float32(1.0) + synth.normal_f32(wl.seed, W.gain_tensor_id(i), h, W.GAIN_SIGMA)
                      for i in range(len(ds.chain.norms))]).astype(np.float32)
    ds.chain.gains.copy_(torch.from_numpy(gains))
    ds.reset(1)
    torch.cuda.synchronize()
    return ds


def read_ceiling(ts, reps: int = 3) -> float:
    import torch

    import weight_streaming_gemv_q8_amd as wsg
    nbytes = ts.weight_bytes_alloc // 16 * 16
    sink = torch.empty(65536, dtype=torch.float32, device="cuda")
    wsg.read_probe(ts.weights, nbytes, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        wsg.read_probe(ts.weights, nbytes, sink)
    e1.record()
    torch.cuda.synchronize()
    return gbps(nbytes * reps, e0.elapsed_time(e1) / 1e3)


# ------------------------------------------------------------ CPU baseline

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, deq: int, budget_s: float) -> dict:
    """The oracle as it stands on a bounded sample: layer 0 of the same
    stream (weights generated and quantized on the host beforehand,
    untimed, as on the GPU), its chain of GEMVs (with per-call activation
    quantization at deq 0) repeated for about budget_s / 2 seconds on one
    thread, then for as long again with the rows of every GEMV split over
    every core in sched_getaffinity (one oracle call per row range; the
    oracle's C calls release the interpreter lock).  GB/s of weight stream;
    value = the multi-threaded rate; the whole-token time is that layer's
    time x layers (extrapolated, and so labelled)."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    import synth
    from synth import workloads as W

    t_setup = time.time()
    mats = []
    for j, m in enumerate(wl.matrices):
        w = np.concatenate([synth.normal_f32(wl.seed, W.weight_tensor_id(0, j, p), r * m.k, W.WEIGHT_SIGMA)
                            .reshape(r, m.k) for p, r in enumerate(m.parts)])
        mats.append(oracle.quantize_q8_0(w) if wl.wtype == "q8_0" else oracle.f32_to_bf16_rows(w))
        del w
    x0 = synth.activation(wl.seed, W.activation_tensor_id(0), wl.matrices[0].k, rms=True)
    log(f"cpu baseline: layer 0 prepared in {time.time() - t_setup:.1f} s")
    threads = len(os.sched_getaffinity(0))

    def gemv(j, xin, rows):
        r0, r1 = rows
        if wl.wtype == "bf16":
            return oracle.gemv_bf16(mats[j][r0:r1], xin)[0]
        if deq == 2:
            return oracle.gemv_q8_act_f32(mats[j][0][r0:r1], mats[j][1][r0:r1], xin)[0]
        dx, qx = xin
        return oracle.gemv_q8_act_q8(mats[j][0][r0:r1], mats[j][1][r0:r1], dx, qx)[0]

    def layer_pass(pool, nthreads):
        x = x0
        for j, m in enumerate(wl.matrices):
            xin = np.ascontiguousarray(x[:m.k], np.float32)
            if wl.wtype == "q8_0" and deq != 2:
                xin = oracle.quantize_q8_0(xin)
            cuts = np.linspace(0, m.n, nthreads + 1).astype(int)
            ranges = [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
            if pool is None:
                x = np.concatenate([gemv(j, xin, r) for r in ranges])
            else:
                x = np.concatenate(list(pool.map(lambda r: gemv(j, xin, r), ranges)))
        return x

    def timed(pool, nthreads):
        passes = 0
        t0 = time.perf_counter()
        while True:
            layer_pass(pool, nthreads)
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget_s / 2:
                return el / passes, passes

    per_layer = wl.weight_bytes_per_layer()
    t1, p1 = timed(None, 1)
    with cf.ThreadPoolExecutor(max_workers=threads) as pool:
        tn, pn = timed(pool, threads)
    quant = ", with per-call activation quantization" if wl.wtype == "q8_0" and deq != 2 else ""
    return {
        "value": round(gbps(per_layer, tn), 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"layer 0 of {wl.name} ({per_layer / 1e6:.1f} MB of weights, {len(wl.matrices)} GEMVs{quant}); "
                   f"{pn} passes on {threads} threads (rows split over sched_getaffinity), and {p1} single-threaded; "
                   f"fp64 C oracle"),
        "cpu_model": cpu_model(),
        "single_thread": {"value": round(gbps(per_layer, t1), 4), "unit": "GB/s", "cores": 1},
        "us_per_token_extrapolated": {"threads": round(tn * wl.layers * 1e6, 1),
                                      "single_thread": round(t1 * wl.layers * 1e6, 1),
                                      "note": f"one layer's time x {wl.layers} layers (extrapolated)"},
    }


# ------------------------------------------------------------ probes

def run_probe(kind: str, nbytes: int) -> int:
    import torch

    import weight_streaming_gemv_q8_amd as wsg
    nbytes = nbytes // 16 * 16
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty(nbytes if kind == "copy" else 16, dtype=torch.uint8, device="cuda")
    sink = torch.empty(65536, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        if kind == "copy":
            wsg.copy_probe(src, dst, nbytes)
        else:
            wsg.read_probe(src, nbytes, sink)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / 3
    moved = nbytes * (2 if kind == "copy" else 1)
    print(json.dumps({"probe": kind, "bytes_read_per_launch": nbytes,
                      "bytes_written_per_launch": nbytes if kind == "copy" else 0,
                      "us_per_launch": round(sec * 1e6, 1), "GBps": round(gbps(moved, sec), 1)}), flush=True)
    return 0


# ------------------------------------------------------------ profile summaries
# rocprofv3 output (CSV) -> short text summaries under profiles/.  Runs on any
# host; the raw rocprofv3 directories stay out of the repository.

_ACT_NAMES = {"0": "q8act", "1": "f32act", "2": "requant"}


def label_from_rocprof(name: str):
    """Bench label of a kernel from its demangled rocprofv3 name (template
    arguments), or None for kernels outside the library's GEMV stream."""
    import re
    m = re.search(r"\b(q8_i8_kernel|q8_f32_kernel|bf16_kernel|stream_kernel|q8_i8_norm_kernel|q8_f32_norm_kernel|"
                  r"q8_i8_swiglu_kernel|q4_i8_kernel|q4_i8_norm_kernel|q4_i8_swiglu_kernel|q4_f32_kernel)<([^>]*)>", name)
    if not m:
        return None
    kind, args = m.group(1), [a.strip() for a in m.group(2).split(",")]
    if kind in ("q8_i8_swiglu_kernel", "q4_i8_swiglu_kernel"):
        return f"{kind}<waves={args[0]},{_ACT_NAMES[args[1]]}>"
    if kind == "q4_i8_kernel":
        return f"{kind}<waves={args[0]},split={args[1]},{_ACT_NAMES[args[2]]}>"
    if kind == "q8_i8_norm_kernel":
        return f"{kind}<waves={args[0]},split={args[1]},unroll={args[2]}>"
    if kind in ("q8_f32_norm_kernel", "q4_i8_norm_kernel", "q4_f32_kernel"):
        return f"{kind}<waves={args[0]},split={args[1]}>"
    if kind == "stream_kernel":
        sc = {"waves": int(args[0]), "unroll": int(args[1]), "sets": int(args[2])}
        return stream_label(sc, args[3] == "true")
    if kind == "q8_i8_kernel":
        extra = (",debug" if args[5] == "true" else "") + (",argmax" if args[6] == "true" else "")
        return f"q8_i8_kernel<waves={args[0]},split={args[1]},unroll={args[2]},{_ACT_NAMES[args[3]]}{extra}>"
    extra = ",argmax" if args[4] == "true" else ""
    return f"{kind}<waves={args[0]},split={args[1]},unroll={args[2]},f32act{extra}>"


def short_kernel_name(name: str) -> str:
    """A kernel's label for the summaries: the bench label for the GEMV
    kernels, else its name with template arguments and no namespaces or
    parameter list."""
    import re
    lab = label_from_rocprof(name)
    if lab:
        return lab
    s = re.sub(r"^void ", "", name)
    s = re.sub(r"\b\w+::|\(anonymous namespace\)::", "", s)
    depth, out = 0, []
    for ch in s:  # drop the parameter list (the first '(' outside template brackets)
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            break
        out.append(ch)
    return "".join(out).strip()[:90]


def stream_label(sc: dict, f32: bool) -> str:
    return f"stream_kernel<waves={sc['waves']},unroll={sc['unroll']},sets={sc['sets']},{'f32act' if f32 else 'requant'}>"


def _read_csv(path: str):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _summarize_boundaries(stats_dir: str, workload: str, commands: dict) -> str:
    """profiles/boundaries_<workload>.txt: the GEMV boundaries of the token
    replays as the rocprofv3 kernel trace sees them.  Consecutive library
    GEMV dispatches whose kernel or grid differ (a token's chain; the
    per-shape graphs repeat one shape) give, per boundary (this kernel and
    grid -> the next): the traced duration, the period to the next
    dispatch's start and the gap between this end and that start."""
    import collections
    rows = [r for r in _read_csv(os.path.join(stats_dir, "run_kernel_trace.csv"))
            if "wsg::" in r["Kernel_Name"] and "_kernel<" in short_kernel_name(r["Kernel_Name"])
            and "quantize" not in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    key = lambda r: (short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size_X"]) // max(int(r["Workgroup_Size_X"]), 1))
    agg = collections.defaultdict(lambda: ([], [], []))
    for a, b in zip(rows, rows[1:]):
        if key(a) == key(b):
            continue
        sa, ea, sb = int(a["Start_Timestamp"]), int(a["End_Timestamp"]), int(b["Start_Timestamp"])
        if sb - sa > 1_000_000:  # not back to back (host work between replays)
            continue
        d, per, gap = agg[(key(a), key(b))]
        d.append((ea - sa) / 1e3)
        per.append((sb - sa) / 1e3)
        gap.append((sb - ea) / 1e3)
    med = lambda v: sorted(v)[len(v) // 2]
    path = os.path.join(PROFILES, f"boundaries_{workload}.txt")
    with open(path, "w") as f:
        f.write(f"# GEMV boundaries of the token replays in the rocprofv3 kernel trace, {workload}\n")
        f.write(f"# command: {commands['stats']}\n")
        f.write("# medians over consecutive dispatches of different kernels or grids; us.  The trace stamps a\n"
                "# kernel's start at the previous kernel's end, so the boundary cost is inside the durations:\n"
                "# the per-workgroup timeline (python -m weight_streaming_gemv_q8_amd.timeline) splits it.\n")
        f.write(f"# {'dispatches':>10} {'duration':>9} {'period':>9} {'gap':>7}  boundary (kernel, grid -> next)\n")
        for ((la, ga), (lb, gb)), (d, per, gap) in sorted(agg.items(), key=lambda kv: -sum(kv[1][0])):
            f.write(f"  {len(d):10d} {med(d):9.2f} {med(per):9.2f} {med(gap):7.2f}  {la} grid {ga} -> {lb} grid {gb}\n")
    return path


def summarize_profiles(stats_dir: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str,
                       workload: str, commands: dict) -> list:
    """Writes profiles/kernel_stats_<workload>.txt from a --kernel-trace
    --stats run (per kernel and grid size: calls, mean, median, min, max
    and total duration) and, when counter runs are given (not "-"),
    profiles/traffic_<kernel>_<workload>.txt per library kernel from two
    --pmc runs (FETCH_SIZE, WRITE_SIZE), each scaled by what the same
    counter reads for the copy probe of known size.  Returns the files
    written."""
    import collections
    os.makedirs(PROFILES, exist_ok=True)
    written = []
    # per-dispatch durations from the trace, grouped by (kernel, grid size)
    groups = collections.defaultdict(list)
    for r in _read_csv(os.path.join(stats_dir, "run_kernel_trace.csv")):
        key = (short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size_X"]) // max(int(r["Workgroup_Size_X"]), 1))
        groups[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total_all = sum(sum(v) for v in groups.values())
    path = os.path.join(PROFILES, f"kernel_stats_{workload}.txt")
    with open(path, "w") as f:
        f.write(f"# rocprofv3 kernel statistics, {workload}, per kernel and grid (workgroups)\n")
        f.write(f"# command: {commands['stats']}\n")
        f.write(f"# {'calls':>6} {'grid':>6} {'avg_us':>10} {'median_us':>10} {'min_us':>10} {'max_us':>10} "
                f"{'total_ms':>10} {'pct':>6}  kernel\n")
        for (lab, grid), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            d = sorted(d)
            f.write(f"  {len(d):6d} {grid:6d} {sum(d) / len(d):10.2f} {d[len(d) // 2]:10.2f} {d[0]:10.2f} "
                    f"{d[-1]:10.2f} {sum(d) / 1e3:10.3f} {100 * sum(d) / total_all:6.2f}  {lab}\n")
    written.append(path)
    if workload.endswith("_graph") or workload.endswith("_graph_deq2"):
        written.append(_summarize_boundaries(stats_dir, workload, commands))
    if fetch_dir == "-" or write_dir == "-":
        return written

    def per_kernel(d, counter):
        agg = collections.defaultdict(list)
        for r in _read_csv(os.path.join(d, "run_counter_collection.csv")):
            if r["Counter_Name"] == counter:
                wg = max(int(r["Workgroup_Size"]), 1)
                agg[(r["Kernel_Name"], int(r["Grid_Size"]) // wg)].append(float(r["Counter_Value"]) * 1024.0)
        return agg

    def copy_factor(d, counter, true_bytes):
        vals = [v for (k, _), v in per_kernel(d, counter).items() if "copy_probe_kernel" in k]
        if not vals:
            raise RuntimeError(f"no copy_probe_kernel rows in {d}")
        got = sum(vals[0]) / len(vals[0])
        return true_bytes / got, got

    probe_bytes = int(commands.get("probe_bytes", 1 << 30))
    rf, rgot = copy_factor(copy_fetch_dir, "FETCH_SIZE", probe_bytes)
    wf, wgot = copy_factor(copy_write_dir, "WRITE_SIZE", probe_bytes)
    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    by_label = collections.defaultdict(list)
    for (name, grid), vals in fetch.items():
        if (name, grid) in write and ("wsg::" in name or label_from_rocprof(name)):
            by_label[short_kernel_name(name)].append((name, grid, vals, write[(name, grid)]))
    digest = source_digest()
    for lab, items in sorted(by_label.items()):
        fv = [v for it in items for v in it[2]]
        wv = [v for it in items for v in it[3]]
        fb, wb = sum(fv) / len(fv) * rf, sum(wv) / len(wv) * wf
        safe = "".join(c if c.isalnum() else "_" for c in lab).strip("_")
        path = os.path.join(PROFILES, f"traffic_{safe}_{workload}.txt")
        with open(path, "w") as f:
            f.write(f"# HBM traffic per launch from rocprofv3 counters, {workload}\n")
            f.write(f"# fetch command: {commands['fetch']}\n# write command: {commands['write']}\n")
            f.write(f"# calibration commands: {commands['copy_fetch']} ; {commands['copy_write']}\n")
            f.write(f"# calibration: copy probe of {probe_bytes} B read / {probe_bytes} B written per launch; "
                    f"FETCH_SIZE reads {rgot:.0f} B (factor {rf:.4f}), WRITE_SIZE reads {wgot:.0f} B "
                    f"(factor {wf:.4f})\n")
            f.write(f"kernel: {lab}\nworkload: {workload}\nrocprof_name: {items[0][0]}\nsource_sha256: {digest}\n")
            f.write(f"launches: {len(fv)}\nfetch_bytes_per_launch: {fb:.0f}\nwrite_bytes_per_launch: {wb:.0f}\n")
            for name, grid, fvals, wvals in sorted(items, key=lambda it: it[1]):
                f.write(f"grid {grid}: launches {len(fvals)}, fetch_bytes_per_launch {sum(fvals) / len(fvals) * rf:.0f}, "
                        f"write_bytes_per_launch {sum(wvals) / len(wvals) * wf:.0f}\n")
        written.append(path)
    return written


# ------------------------------------------------------------ main

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense27b_q8_0_64L")
    ap.add_argument("--deq", type=int, default=0, choices=(0, 1, 2))
    ap.add_argument("--requant", default="fused", choices=("fused", "separate"))
    ap.add_argument("--plan", default="graph", choices=("persistent", "graph"),
                    help="one resident kernel per token (persistent), or a graph node per GEMV")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the deq-2 line and the read ceiling")
    ap.add_argument("--probe", choices=("copy", "read"),
                    help="only run the copy (or read) probe over --probe-bytes, 3 launches: a kernel of known "
                         "traffic for calibrating hardware byte counters")
    ap.add_argument("--probe-bytes", type=int, default=1 << 30)
    ap.add_argument("--configs", action="store_true",
                    help="measure every workload (single GEMV hot/cold, LM head, the three token streams) and "
                         "print one JSON line per configuration and mode, instead of the benchmark line")
    ap.add_argument("--configs-part", default=None, metavar="NAME",
                    help="with --configs: measure one part (see config_part_names) in this process")
    ap.add_argument("--configs-one-process", action="store_true",
                    help="with --configs: measure every part in this process (for profilers; later streams "
                         "then run on re-used allocations, ~3.5%% slower)")
    ap.add_argument("--summarize", nargs=5, metavar=("STATS", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write profiles/ summaries from rocprofv3 output directories (no GPU needed); "
                         "the commands that made them are read from STATS/commands.json")
    args = ap.parse_args()
    if args.probe:
        return run_probe(args.probe, args.probe_bytes)
    if args.summarize:
        with open(os.path.join(os.path.abspath(args.summarize[0]), "commands.json")) as f:
            cmds = json.load(f)
        for p in summarize_profiles(*args.summarize, workload=cmds["workload"], commands=cmds):
            print(p)
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU step (see the design notes on "
              "sharding by output rows); run it with --gpus 1", file=sys.stderr)
        return 2

    if args.configs_part is not None:
        args.configs = True
    if args.configs and args.configs_part is None and not args.configs_one_process:
        return run_configs_in_children(args.steps, args.warmup)
    if args.configs_part is not None and args.configs_part not in config_part_names():
        print(f"unknown configs part {args.configs_part}; choose one of {config_part_names()}", file=sys.stderr)
        return 2

    import torch

    import weight_streaming_gemv_q8_amd as wsg
    from synth import workloads as W

    if args.configs:
        torch.cuda.set_device(0)
        wsg.lib()
        for r in measure_configs(args.steps, args.warmup, args.configs_part):
            print(json.dumps(r), flush=True)
        return 0

    wl = {w.name: w for w in W.ALL}.get(args.workload)
    if wl is None or wl.wtype not in ("q8_0", "bf16") or wl.layers < 2:
        print(f"unknown or non-stream workload {args.workload}; choose one of "
              f"{[w.name for w in W.ALL if w.wtype in ('q8_0', 'bf16') and w.layers > 1]}", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    wsg.lib()

    ts = build_stream(wl, args.deq, args.requant)
    alg_bytes = ts.algorithmic_weight_bytes()
    act_fmt = ts.act_fmt()
    persistent = args.plan == "persistent"
    if persistent and (wl.wtype != "q8_0" or args.requant != "fused"):
        print("the persistent plan runs Q8_0 streams with fused requantization or f32 activations", file=sys.stderr)
        return 2

    rstats = {}
    sec, kernels_per_token = time_plan(ts, args.plan, args.steps, args.warmup, rstats)
    value = gbps(alg_bytes, sec)
    log(f"{args.plan} plan, {kernels_per_token} kernel(s) per token: timed {args.steps} steps: "
        f"{sec * 1e6:.1f} us per token (median {rstats['median_s'] * 1e6:.1f}, min {rstats['min_s'] * 1e6:.1f}), "
        f"{value:.1f} GB/s")

    wtype_code = wsg.W_Q8_0 if wl.wtype == "q8_0" else wsg.W_BF16
    prof_workload = f"{wl.name}_{args.plan}" + ("_deq2" if args.deq == 2 else "")
    if persistent:
        # one launch per token: the dominant kernel is the whole stream
        label = stream_label(wsg.stream_config(), act_fmt == wsg.ACT_F32)
        traffic, refs = profile_refs(label, prof_workload)
        roofline = {
            "bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBPS, 4), "traffic": traffic, "profiles": refs,
            "kernel": label + " (the whole token in one launch)",
            "launches_per_token": 1, "bytes_per_launch": alg_bytes, "us_per_launch": round(sec * 1e6, 1),
            "timing": "HIP events around the token replays",
        }
    else:
        # each matrix of the layer as it runs in the token (its L launches in
        # one graph, HIP events around the replays), grouped by kernel
        # instantiation; the dominant one takes the most time per token
        shapes = time_per_shape(ts, wtype_code, act_fmt, reps=max(5, args.steps // 5))
        groups = {}
        for r in shapes:
            g = groups.setdefault(r["label"], {"t": 0.0, "bytes": 0, "launches": 0, "shapes": []})
            g["t"] += r["us"] * 1e-6 * r["launches_per_token"]
            g["bytes"] += r["bytes"] * r["launches_per_token"]
            g["launches"] += r["launches_per_token"]
            g["shapes"].append(r)
        dom = max(groups, key=lambda kk: groups[kk]["t"])
        g = groups[dom]
        achieved = gbps(g["bytes"] / g["launches"], g["t"] / g["launches"])
        traffic, refs = profile_refs(dom, prof_workload)
        roofline = {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "profiles": refs, "kernel": dom,
            "launches_per_token": g["launches"], "bytes_per_launch": g["bytes"] // g["launches"],
            "us_per_launch": round(g["t"] / g["launches"] * 1e6, 2),
            "timing": ("HIP events around graphs of each matrix's launches of the token (one per layer, "
                       "in token order); bytes and time summed over the kernel's shapes"),
            "shapes": [{"n": r["n"], "k": r["k"], "grid": r["grid"], "bytes_per_launch": r["bytes"],
                        "us_per_launch": round(r["us"], 2), "GBps": round(gbps(r["bytes"], r["us"] * 1e-6), 1),
                        "frac": round(gbps(r["bytes"], r["us"] * 1e-6) / HBM_PEAK_GBPS, 4)} for r in g["shapes"]],
            "other_kernels": {lab: {"launches_per_token": o["launches"],
                                    "us_per_launch": round(o["t"] / o["launches"] * 1e6, 2),
                                    "GBps": round(gbps(o["bytes"] / o["launches"], o["t"] / o["launches"]), 1)}
                              for lab, o in groups.items() if lab != dom},
        }
        for r in shapes:
            log(f"  {r['label']} n={r['n']} k={r['k']}: {r['us']:.2f} us/launch, "
                f"{gbps(r['bytes'], r['us'] * 1e-6):.1f} GB/s")
    log(f"dominant kernel {roofline['kernel']}: {roofline['us_per_launch']} us/launch, "
        f"{roofline['achieved']} GB/s")

    extras = {}
    if not args.no_extras:
        if wl.wtype == "q8_0" and args.requant == "fused":
            others = [o for o in ("graph", "persistent") if o != args.plan]
            for other in others:
                sec_o, k_o = time_plan(ts, other, args.steps, args.warmup)
                extras[f"{other}_plan"] = {"us_per_token": round(sec_o * 1e6, 1),
                                           "GBps": round(gbps(alg_bytes, sec_o), 1), "kernels_per_token": k_o}
                log(f"{other} plan: {sec_o * 1e6:.1f} us per token")
        extras["read_ceiling_GBps"] = round(read_ceiling(ts), 1)
        # the token's and the dominant kernel's rates against that ceiling
        extras["frac_of_read_ceiling"] = round(value / extras["read_ceiling_GBps"], 4)
        extras["roofline_frac_of_read_ceiling"] = round(roofline["achieved"] / extras["read_ceiling_GBps"], 4)
        log(f"read ceiling {extras['read_ceiling_GBps']} GB/s")
        if wl.wtype == "q8_0" and args.deq != 2:
            # the same stream with f32 activations (deq 2), same weights
            ts.deq = 2
            sec2, _ = time_plan(ts, args.plan, args.steps, args.warmup)
            extras["deq2"] = {"us_per_token": round(sec2 * 1e6, 1), "GBps": round(gbps(alg_bytes, sec2), 1),
                              "frac_of_peak": round(gbps(alg_bytes, sec2) / HBM_PEAK_GBPS, 4)}
            log(f"deq 2: {sec2 * 1e6:.1f} us per token")
            ts.deq = args.deq
    ts.close()

    del ts
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.deq, args.cpu_seconds)
        log(f"cpu baseline {cpu['value']} GB/s")

    dtype = "bf16xf32" if wl.wtype == "bf16" else ("int8" if act_fmt != wsg.ACT_F32 else "q8_0xf32")
    out = {
        "metric": "achieved HBM GB/s (% of peak) and us per full-token batch-1 GEMV stream",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "description": wl.description,
            "matrices": [f"{m.name} {m.n}x{m.k}" for m in wl.matrices],
            "layers": wl.layers,
            "gemvs_per_token": wl.gemvs_per_token(),
            "weight_bytes_per_token": alg_bytes,
            "deq": args.deq,
            "activation_quantization": ("fused into each GEMV" if args.requant == "fused" else "separate launch")
            if act_fmt != wsg.ACT_F32 else "none (f32 activations)",
            "kernels_per_token": kernels_per_token,
            "plan": args.plan,
        },
        "us_per_token": round(sec * 1e6, 1),
        "us_per_token_median": round(rstats["median_s"] * 1e6, 1),
        "us_per_token_min": round(rstats["min_s"] * 1e6, 1),
        "timed_replays": rstats["replays"],
        "frac_of_peak": round(value / HBM_PEAK_GBPS, 4),
        "tok_per_s_equiv": round(1.0 / sec, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    out.update(extras)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
