"""Where a GEMV boundary of the token goes: a per-workgroup timeline of the
27B-scale Q8_0 stream (deq 0, requantization fused into each GEMV).

Runs the diagnostic build (libwsgemv_timeline.so, built by
``build.build(timeline=True)``; the stamps are described in
csrc/timeline.hpp), replays the token a few times with the stamps on, and
writes a summary per matrix of the layer.

Graph plan (one launch per GEMV, the int8 GEMV kernel):

* node period: first workgroup entry of this GEMV to that of the next;
* entry spread: first to last workgroup entry of the launch;
* staging: a workgroup's entry to the end of its activation staging (median);
* body: the launch's first entry to the median workgroup end;
* tail: the median to the last workgroup end;
* gap: the last workgroup end to the next launch's first entry (the kernel
  boundary itself: completion, cache write-back, the next dispatch);
* wave spread: within a workgroup, the first to the last wave to finish its
  row loop (median over workgroups);
* the two workgroups sharing a CU (b and b + CUs): median end of each;
* the index of the wave that ends its row loop first, and last (median
  over workgroups).

Persistent plan (one resident kernel per token; per op and workgroup):

* period: median op end (results stored) to the next op's median end;
* producer tail: the previous op's median to last end (what every
  consumer of its output waits for);
* ready: the previous op's last end to this op's median input staged
  (the dependency's own latency, with the staging's round trips);
* stage: the op's first weight requests to its input staged (median);
* body: input staged to row loop end (median);
* tail: median to last row loop end;
* store: row loop end to results stored (median).

Times come from the GPU's 100 MHz constant clock.  The graph plan's stamps
cost a barrier and one workgroup store at each workgroup's end, so its
traced token is slower than the untraced one (both are reported); the
persistent kernel's stamps are a few stores per op and workgroup.  Only
the int8 form is stamped: in the stream that hands the normalized
activations over in f32 (deq 2), the GEMVs after a norm run the f32 kernel
and leave no records.

    python -m weight_streaming_gemv_q8_amd.timeline [--plan graph|persistent] [--replays 3]
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
NF, NWG = 10, 512  # fields per record, workgroups recorded per launch (timeline.hpp)
US = 0.01  # 100 MHz ticks


def _primes(lo: int, hi: int):
    for p in range(lo, hi):
        if all(p % q for q in range(2, int(p ** 0.5) + 1)):
            yield p


def _graph_records(h, outs, mod, r):
    recs = {}
    hv = h.reshape(mod, NWG, NF)
    for j, p in enumerate(outs):
        e = hv[(p >> 2) % mod]
        grid = int(e[0, 1] >> 32)
        g = min(grid, NWG)
        if grid == 0 or not (e[:g, 0] == p).all():
            raise RuntimeError(f"GEMV {j}: missing timeline records")
        recs[(r, j)] = (grid, e[:g].copy())
    return recs


def _persistent_records(h, n_ops, r):
    recs = {}
    hv = h.reshape(-1, NWG, NF)
    for j in range(n_ops):
        e = hv[j]
        grid = int(e[0, 1] >> 32)
        g = min(grid, NWG)
        if grid == 0 or not (e[:g, 0] == j).all() or (e[:g, 5] == 0).any():
            raise RuntimeError(f"op {j}: missing timeline records")
        recs[(r, j)] = (grid, e[:g].copy())
    return recs


def _graph_summary(np, by, replays, nm, n, cus):
    keys = ("period", "entry", "staging", "body", "tail", "gap", "waves", "first_wg", "second_wg", "first_w",
            "last_w")
    per = {q: {k: [] for k in keys} for q in range(nm)}
    for r in range(replays):
        for j in range(nm, n - nm):  # layers 1 .. L-2
            grid, e = by[(r, j)]
            _, e2 = by[(r, j + 1)]
            t0 = e[:, 2].min()
            ends = e[:, 6]
            d = per[j % nm]
            d["period"].append((e2[:, 2].min() - t0) * US)
            d["entry"].append((e[:, 2].max() - t0) * US)
            d["staging"].append(float(np.median(e[:, 3] - e[:, 2])) * US)
            d["body"].append((float(np.median(ends)) - t0) * US)
            d["tail"].append((ends.max() - float(np.median(ends))) * US)
            d["gap"].append((e2[:, 2].min() - ends.max()) * US)
            d["waves"].append(float(np.median(e[:, 5] - e[:, 4])) * US)
            # which wave of the workgroup ended its row loop first / last
            d["first_w"].append(float(np.median((e[:, 8] >> 32) & 0xFF)))
            d["last_w"].append(float(np.median((e[:, 8] >> 40) & 0xFF)))
            if grid > cus:
                b = np.arange(len(e))
                d["first_wg"].append(float(np.median(ends[b < cus] - t0)) * US)
                d["second_wg"].append(float(np.median(ends[(b >= cus) & (b < 2 * cus)] - t0)) * US)
    heads = ("period", "entry", "staging", "body", "tail", "gap", "waves", "1st WG", "2nd WG", "1st wave",
             "last wave")
    return per, keys, heads, ("period", "staging", "tail", "gap")


def _persistent_summary(np, by, replays, nm, n):
    keys = ("period", "prod_tail", "ready", "stage", "body", "tail", "store")
    per = {q: {k: [] for k in keys} for q in range(nm)}
    med = lambda v: float(np.median(v))
    for r in range(replays):
        for j in range(nm, n - nm):
            _, p = by[(r, j - 1)]
            _, e = by[(r, j)]
            d = per[j % nm]
            d["period"].append((med(e[:, 5]) - med(p[:, 5])) * US)
            d["prod_tail"].append((p[:, 5].max() - med(p[:, 5])) * US)
            d["ready"].append((med(e[:, 3]) - p[:, 5].max()) * US)
            d["stage"].append(med(e[:, 3] - e[:, 2]) * US)
            d["body"].append(med(e[:, 4] - e[:, 3]) * US)
            d["tail"].append((e[:, 4].max() - med(e[:, 4])) * US)
            d["store"].append(med(e[:, 5] - e[:, 4]) * US)
    return per, keys, keys, ("period", "prod_tail", "ready", "tail")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--plan", default="graph", choices=("graph", "persistent"))
    ap.add_argument("--replays", type=int, default=3)
    ap.add_argument("--out", default=None, help="summary file (default: profiles/timeline_<workload>.txt)")
    args = ap.parse_args()

    from weight_streaming_gemv_q8_amd import build as libbuild
    if not os.path.exists(libbuild.TIMELINE_LIB):
        print(f"{libbuild.TIMELINE_LIB} is missing: build it with build.build(timeline=True)", file=sys.stderr)
        return 2
    os.environ["WSG_LIBRARY"] = libbuild.TIMELINE_LIB
    sys.path.insert(0, ROOT)
    import numpy as np
    import torch

    import bench
    import weight_streaming_gemv_q8_amd as wsg
    from synth import workloads as W

    L = wsg.lib()
    L.wsg_timeline_set.argtypes = [ctypes.c_void_p, ctypes.c_uint32]
    L.wsg_timeline_set.restype = ctypes.c_int
    torch.cuda.set_device(0)
    wl = W.DENSE27B_Q8
    persistent = args.plan == "persistent"
    ts = bench.build_stream(wl, 0, "fused")
    ts.capture(persistent=persistent)
    for _ in range(5):
        ts.launch()
    torch.cuda.synchronize()

    def timed(n: int) -> float:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            ts.launch()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    untraced = min(timed(20) for _ in range(3))
    outs = [y.data_ptr() for y in ts.outputs()]
    n = len(outs)
    if persistent:
        mod = n  # one slot per op
    else:
        mod = next(p for p in _primes(8192, 1 << 17) if len({(o >> 2) % p for o in outs}) == len(outs))
    buf = torch.zeros(mod * NWG * NF, dtype=torch.int64, device="cuda")
    by, traced = {}, []
    for r in range(args.replays):
        buf.zero_()
        torch.cuda.synchronize()
        assert L.wsg_timeline_set(buf.data_ptr(), mod) == 0
        traced.append(timed(1))
        assert L.wsg_timeline_set(None, 0) == 0
        h = buf.cpu().numpy()
        by.update(_persistent_records(h, n, r) if persistent else _graph_records(h, outs, mod, r))
    ts.close()

    names = [m.name for m in wl.matrices]
    nm = len(names)
    if persistent:
        per, keys, heads, sums = _persistent_summary(np, by, args.replays, nm, n)
    else:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        per, keys, heads, sums = _graph_summary(np, by, args.replays, nm, n, cus)
    workload = f"{wl.name}_{args.plan}"
    out = args.out or os.path.join(ROOT, "profiles", f"timeline_{workload}.txt")
    med = lambda v: float(np.median(v)) if v else float("nan")
    kernel = "the persistent token kernel, per op" if persistent else "the int8 GEMV kernels"
    lines = [
        f"# per-workgroup timeline of {kernel}, {workload} (diagnostic build, s_memrealtime)",
        f"# command: python -m weight_streaming_gemv_q8_amd.timeline --plan {args.plan} --replays {args.replays}",
        f"# token: {untraced:.1f} us untraced, {med(traced):.1f} us traced (median of {args.replays} replays)",
        "# medians over layers 1..62 and the replays; us",
        "# " + f"{'matrix':8s} " + " ".join(f"{h:>9s}" for h in heads),
    ]
    tot = {k: 0.0 for k in sums}
    for q in range(nm):
        d = per[q]
        lines.append(f"  {names[q]:8s} " + " ".join(f"{med(d[k]):9.2f}" for k in keys))
        for k in tot:
            tot[k] += med(d[k])
    lines.append(f"# per layer: period {tot['period']:.2f} us (x{wl.layers} layers = {tot['period'] * wl.layers:.0f} us), "
                 "of which " + ", ".join(f"{k} {tot[k]:.2f}" for k in sums if k != "period"))
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    if not persistent:
        # how often each wave index ends the row loop first / last
        for q in range(nm):
            f8 = np.concatenate([by[(r, j)][1][:, 8] for r in range(args.replays) for j in range(nm, n - nm)
                                 if j % nm == q])
            first = np.bincount(((f8 >> 32) & 0xFF).astype(np.int64), minlength=16)
            last = np.bincount(((f8 >> 40) & 0xFF).astype(np.int64), minlength=16)
            print(f"  {names[q]:8s} first-ending wave counts {first.tolist()}")
            print(f"  {names[q]:8s} last-ending wave counts  {last.tolist()}")
    print(out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
