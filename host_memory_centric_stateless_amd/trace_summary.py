"""Summarise a rocprofv3 kernel + memory-copy trace of a streamed training run.

    python -m host_memory_centric_stateless_amd.trace_summary <dir>/<prefix> [--start-frac F]
        [--micro-batches N]

Reads <prefix>_kernel_trace.csv and <prefix>_memory_copy_trace.csv (rocprofv3
--kernel-trace --memory-copy-trace --output-format csv) and prints:

* per-kernel total / average duration and share of kernel time;
* busy time (union of intervals) of compute kernels, host->device copies and
  device->host traffic (DMA copies plus the gradient drain, which is a copy
  kernel writing pinned host memory and so appears in the kernel trace);
* copy/compute overlap = |copies AND kernels| / min(|copies|, |kernels|)
  (union measure), for H2D, D2H and both;
* large-copy durations (copies longer than 1 ms);
* the host-to-device link idle between weight loads, and the times the
  micro-batch losses are reduced (step and micro-batch boundaries).

--start-frac F starts the window F of the way into the trace (default: the
whole trace); --micro-batches N (micro-batches per step) adds, per step, the
link's busy and idle time between weight loads.
"""
from __future__ import annotations

import argparse
import bisect
import csv
from collections import defaultdict
from typing import List, Tuple

Interval = Tuple[int, int]
DRAIN = "copy16_kernel"  # gradient slab -> pinned host copy kernel
# link-idle gap classes, ns: [start, end), end None = open
GAP_CLASSES = ((0, 500_000), (500_000, 4_500_000), (4_500_000, 20_000_000), (20_000_000, None))


def _read(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def union(iv: List[Interval]) -> List[Interval]:
    out: List[Interval] = []
    for a, b in sorted(iv):
        if out and a <= out[-1][1]:
            if b > out[-1][1]:
                out[-1] = (out[-1][0], b)
        else:
            out.append((a, b))
    return out


def measure(iv: List[Interval]) -> int:
    return sum(b - a for a, b in iv)


def intersect(x: List[Interval], y: List[Interval]) -> List[Interval]:
    i = j = 0
    out = []
    while i < len(x) and j < len(y):
        a, b = max(x[i][0], y[j][0]), min(x[i][1], y[j][1])
        if a < b:
            out.append((a, b))
        if x[i][1] < y[j][1]:
            i += 1
        else:
            j += 1
    return out


def clip(iv, lo, hi):
    return [(max(a, lo), min(b, hi)) for a, b in iv if b > lo and a < hi]


def summarize(prefix: str, t0: int = None, t1: int = None, micro_batches: int = 0) -> str:
    kt = _read(prefix + "_kernel_trace.csv")
    mc = _read(prefix + "_memory_copy_trace.csv")
    kern = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in kt]
    drain = [(a, b) for a, b, n in kern if DRAIN in n]
    kern = [k for k in kern if DRAIN not in k[2]]
    h2d = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in mc
           if r["Direction"].endswith("HOST_TO_DEVICE")]
    d2h = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in mc
           if r["Direction"].endswith("DEVICE_TO_HOST")] + drain
    lo = t0 if t0 is not None else min([k[0] for k in kern] + [c[0] for c in h2d + d2h])
    hi = t1 if t1 is not None else max([k[1] for k in kern] + [c[1] for c in h2d + d2h])
    kern = [(max(a, lo), min(b, hi), n) for a, b, n in kern if b > lo and a < hi]
    h2d, d2h = clip(h2d, lo, hi), clip(d2h, lo, hi)

    per = defaultdict(lambda: [0, 0])
    for a, b, n in kern:
        per[n][0] += 1
        per[n][1] += b - a
    ktot = sum(v[1] for v in per.values())
    K = union([(a, b) for a, b, _ in kern])
    H, D = union(h2d), union(d2h)
    C = union(h2d + d2h)
    lines = [f"window: {(hi - lo) / 1e9:.3f} s",
             f"kernel busy (union): {measure(K) / 1e9:.3f} s  ({100 * measure(K) / (hi - lo):.1f}% of window)",
             f"H2D busy (union):    {measure(H) / 1e9:.3f} s  ({len(h2d)} copies)",
             f"D2H busy (union):    {measure(D) / 1e9:.3f} s  ({len(d2h)} copies, "
             f"{len(drain)} of them drain kernels)",
             f"any copy busy:       {measure(C) / 1e9:.3f} s"]
    for name, X in (("H2D", H), ("D2H", D), ("any copy", C)):
        if measure(X) and measure(K):
            ov = measure(intersect(X, K)) / min(measure(X), measure(K))
            lines.append(f"overlap {name:8s} with kernels: {ov:.3f}")
    for name, X in (("H2D", h2d), ("D2H", d2h)):
        big = [b - a for a, b in X if b - a > 1_000_000]
        if big:
            lines.append(f"{name} copies > 1 ms: n={len(big)} mean {sum(big) / len(big) / 1e6:.2f} ms "
                         f"min {min(big) / 1e6:.2f} max {max(big) / 1e6:.2f}")
    if drain:
        dt = sum(b - a for a, b in clip(drain, lo, hi))
        lines.append(f"drain kernels: n={len(drain)} total {dt / 1e6:.1f} ms")
    # Link idle between weight loads (host-to-device copies over 1 ms), by gap
    # length.  With two weight buffers the 4.5-20 ms gaps are the bubbles where
    # both buffers hold blocks still needed; the long ones are step boundaries
    # and the end of the run.
    loads = sorted((a, b) for a, b in h2d if b - a > 1_000_000)
    gaps = [(s1 - e0, e0) for (_, e0), (s1, _) in zip(loads, loads[1:]) if s1 > e0]

    def by_length(idle):
        parts = []
        for c0, c1 in GAP_CLASSES:
            x = [g for g in idle if g >= c0 and (c1 is None or g < c1)]
            label = f"{c0 / 1e6:g}-{c1 / 1e6:g} ms" if c1 else f">= {c0 / 1e6:g} ms"
            parts.append(f"{label}: n={len(x)} {sum(x) / 1e6:.1f} ms")
        return "; ".join(parts)

    if gaps:
        lines.append(f"H2D idle between weight loads: {sum(g for g, _ in gaps) / 1e6:.1f} ms in "
                     f"{len(gaps)} gaps; " + by_length([g for g, _ in gaps]))
        for g, t in sorted((gt for gt in gaps if gt[0] >= GAP_CLASSES[-1][0]), reverse=True)[:4]:
            lines.append(f"  gap {g / 1e6:7.1f} ms from {(t - lo) / 1e9:.3f} s")
    marks = sorted(a for a, _, n in kern if "loss_reduce_kernel" in n)
    if marks:
        lines.append("micro-batch losses reduced at (s): "
                     + " ".join(f"{(t - lo) / 1e9:.3f}" for t in marks))
    # Per step, counting micro-batches from the first loss reduction in the
    # window (taken as a step's first): from one step's last reduction to the
    # next one's, the weight loads and the link idle time between them.
    if micro_batches > 0:
        for j in range(micro_batches - 1, len(marks) - micro_batches, micro_batches):
            a, b = marks[j], marks[j + micro_batches]
            inside = [(s, e) for s, e in loads if a <= s < b]
            idle = [g for g, t in gaps if a <= t < b]
            lines.append(f"step {(a - lo) / 1e9:.3f}-{(b - lo) / 1e9:.3f} s ({(b - a) / 1e6:.0f} ms): "
                         f"{len(inside)} weight loads busy {sum(e - s for s, e in inside) / 1e6:.0f} ms, "
                         f"link idle {sum(idle) / 1e6:.0f} ms; " + by_length(idle))
    # Compute time with no copy in flight, by kernel: what keeps the overlap below 1.
    lone = defaultdict(int)
    cends = [e for _, e in C]
    for a, b, n in kern:
        i, covered = bisect.bisect_right(cends, a), 0
        while i < len(C) and C[i][0] < b:
            covered += min(b, C[i][1]) - max(a, C[i][0])
            i += 1
        lone[n] += (b - a) - covered
    lone_tot = sum(lone.values())
    if lone_tot:
        lines.append(f"kernel time with no copy in flight: {lone_tot / 1e6:.1f} ms (sum over launches)")
        for n, t in sorted(lone.items(), key=lambda kv: -kv[1])[:8]:
            short = n.replace("mt::(anonymous namespace)::", "").split("(")[0][:60]
            lines.append(f"  {short:60s} {t / 1e6:8.1f} ms")
    lines.append("")
    lines.append(f"{'kernel':70s} {'calls':>6s} {'total ms':>10s} {'avg us':>10s} {'share':>6s}")
    for n, (c, t) in sorted(per.items(), key=lambda kv: -kv[1][1]):
        short = n.replace("mt::(anonymous namespace)::", "").split("(")[0][:70]
        lines.append(f"{short:70s} {c:6d} {t / 1e6:10.1f} {t / c / 1e3:10.1f} {100 * t / ktot:5.1f}%")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("prefix")
    ap.add_argument("--start-frac", type=float, default=0.0,
                    help="start the window this fraction into the trace")
    ap.add_argument("--micro-batches", type=int, default=0,
                    help="micro-batches per step: break the link idle time down per step")
    a = ap.parse_args()
    t0 = None
    if a.start_frac > 0:
        kt = _read(a.prefix + "_kernel_trace.csv")
        lo = min(int(r["Start_Timestamp"]) for r in kt)
        hi = max(int(r["End_Timestamp"]) for r in kt)
        t0 = int(lo + a.start_frac * (hi - lo))
    print(summarize(a.prefix, t0=t0, micro_batches=a.micro_batches))


if __name__ == "__main__":
    main()
