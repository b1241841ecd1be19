"""Where a GEMV boundary of the token goes: a per-workgroup timeline of the
int8 GEMV kernels of the 27B-scale Q8_0 stream in the graph plan.

Runs the diagnostic build (libwsgemv_timeline.so, built by
``build.build(timeline=True)``; the stamps are described in
csrc/timeline.hpp), replays the token a few times with the stamps on, and
writes a summary per matrix of the layer:

* node period: first workgroup entry of this GEMV to that of the next;
* entry spread: first to last workgroup entry of the launch;
* staging: a workgroup's entry to the end of its activation staging (median);
* body: the launch's first entry to the median workgroup end;
* tail: the median to the last workgroup end;
* gap: the last workgroup end to the next launch's first entry (the kernel
  boundary itself: completion, cache write-back, the next dispatch);
* wave spread: within a workgroup, the first to the last wave to finish its
  row loop (median over workgroups);
* the two workgroups sharing a CU (b and b + CUs): median end of each.

Times come from the GPU's 100 MHz constant clock.  The stamps cost a barrier
and one workgroup store at each workgroup's end, so the traced token is a
few per cent slower than the untraced one (both are reported).

Only the int8 form is stamped: in the stream that hands the normalized
activations over in f32 (deq 2), the GEMVs after a norm run the f32 kernel
and leave no records.

    python -m weight_streaming_gemv_q8_amd.timeline [--replays 3]
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)


def _primes(lo: int, hi: int):
    for p in range(lo, hi):
        if all(p % q for q in range(2, int(p ** 0.5) + 1)):
            yield p


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
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
    ts = bench.build_stream(wl, 0, "fused")
    ts.capture(persistent=False)
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
    mod = next(p for p in _primes(8192, 1 << 17) if len({(o >> 2) % p for o in outs}) == len(outs))
    nf, nwg = 10, 512
    buf = torch.zeros(mod * nwg * nf, dtype=torch.int64, device="cuda")
    recs, traced = [], []
    for r in range(args.replays):
        buf.zero_()
        torch.cuda.synchronize()
        assert L.wsg_timeline_set(buf.data_ptr(), mod) == 0
        traced.append(timed(1))
        assert L.wsg_timeline_set(None, 0) == 0
        h = buf.view(mod, nwg, nf).cpu().numpy()
        for j, p in enumerate(outs):
            e = h[(p >> 2) % mod]
            grid = int(e[0, 1] >> 32)
            g = min(grid, nwg)
            if grid == 0 or not (e[:g, 0] == p).all():
                raise RuntimeError(f"GEMV {j}: missing timeline records")
            recs.append((r, j, grid, e[:g].copy()))
    ts.close()

    names = [m.name for m in wl.matrices]
    nm = len(names)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    per = {q: {k: [] for k in ("period", "entry", "staging", "body", "tail", "gap", "waves", "first_wg", "second_wg")}
           for q in range(nm)}
    by = {(r, j): (grid, e) for r, j, grid, e in recs}
    us = 0.01  # 100 MHz ticks
    for r in range(args.replays):
        for j in range(nm, len(outs) - nm):  # layers 1 .. L-2
            grid, e = by[(r, j)]
            _, e2 = by[(r, j + 1)]
            t0 = e[:, 2].min()
            ends = e[:, 6]
            q = j % nm
            d = per[q]
            d["period"].append((e2[:, 2].min() - t0) * us)
            d["entry"].append((e[:, 2].max() - t0) * us)
            d["staging"].append(float(np.median(e[:, 3] - e[:, 2])) * us)
            d["body"].append((float(np.median(ends)) - t0) * us)
            d["tail"].append((ends.max() - float(np.median(ends))) * us)
            d["gap"].append((e2[:, 2].min() - ends.max()) * us)
            d["waves"].append(float(np.median(e[:, 5] - e[:, 4])) * us)
            if grid > cus:
                b = np.arange(len(e))
                d["first_wg"].append(float(np.median(ends[b < cus] - t0)) * us)
                d["second_wg"].append(float(np.median(ends[(b >= cus) & (b < 2 * cus)] - t0)) * us)
    workload = f"{wl.name}_graph"
    out = args.out or os.path.join(ROOT, "profiles", f"timeline_{workload}.txt")
    med = lambda v: float(np.median(v)) if v else float("nan")
    lines = [
        f"# per-workgroup timeline of the int8 GEMV kernels, {workload} (diagnostic build, s_memrealtime)",
        f"# command: python -m weight_streaming_gemv_q8_amd.timeline --replays {args.replays}",
        f"# token: {untraced:.1f} us untraced, {med(traced):.1f} us traced (median of {args.replays} replays)",
        "# medians over layers 1..62 and the replays; us",
        f"# {'matrix':8s} {'period':>7s} {'entry':>6s} {'staging':>8s} {'body':>7s} {'tail':>6s} {'gap':>6s} "
        f"{'waves':>6s} {'1st WG':>7s} {'2nd WG':>7s}",
    ]
    tot = {k: 0.0 for k in ("period", "staging", "tail", "gap")}
    for q in range(nm):
        d = per[q]
        lines.append(f"  {names[q]:8s} {med(d['period']):7.2f} {med(d['entry']):6.2f} {med(d['staging']):8.2f} "
                     f"{med(d['body']):7.2f} {med(d['tail']):6.2f} {med(d['gap']):6.2f} {med(d['waves']):6.2f} "
                     f"{med(d['first_wg']):7.2f} {med(d['second_wg']):7.2f}")
        for k in tot:
            tot[k] += med(d[k])
    lines.append(f"# per layer: period {tot['period']:.2f} us (x{wl.layers} layers = {tot['period'] * wl.layers:.0f} us), "
                 f"of which staging {tot['staging']:.2f}, tails {tot['tail']:.2f}, gaps {tot['gap']:.2f}")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    print(out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
