"""The rocprofv3 trace summary on a small hand-made trace: busy and overlap
measures, the link idle time between weight loads and its per-step split."""
import csv

from host_memory_centric_stateless_amd.trace_summary import summarize

MS = 1_000_000  # ns


def _write(tmp_path, kernels, copies):
    kf = tmp_path / "t_kernel_trace.csv"
    with open(kf, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for n, a, b in kernels:
            w.writerow([n, a, b])
    cf = tmp_path / "t_memory_copy_trace.csv"
    with open(cf, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Direction", "Start_Timestamp", "End_Timestamp"])
        for d, a, b in copies:
            w.writerow([d, a, b])
    return str(tmp_path / "t")


def test_link_idle_and_per_step_split(tmp_path):
    h2d = "MEMORY_COPY_HOST_TO_DEVICE"
    # weight loads of 8 ms with gaps of 0.2, 6 and 30 ms, one of 2 ms; a drain kernel
    loads = [(0, 8), (8.2, 16.2), (22.2, 30.2), (60.2, 68.2), (70.2, 78.2)]
    copies = [(h2d, int(a * MS), int(b * MS)) for a, b in loads]
    kernels = [("gemm_kernel", int(1 * MS), int(5 * MS)),
               ("copy16_kernel", int(10 * MS), int(14 * MS)),
               ("loss_reduce_kernel", int(2 * MS), int(2.1 * MS)),
               ("loss_reduce_kernel", int(40 * MS), int(40.1 * MS)),
               ("loss_reduce_kernel", int(75 * MS), int(75.1 * MS))]
    out = summarize(_write(tmp_path, kernels, copies), micro_batches=1)
    assert ("H2D idle between weight loads: 38.2 ms in 4 gaps; 0-0.5 ms: n=1 0.2 ms; "
            "0.5-4.5 ms: n=1 2.0 ms; 4.5-20 ms: n=1 6.0 ms; >= 20 ms: n=1 30.0 ms") in out
    assert "  gap    30.0 ms from 0.030 s" in out
    # steps from one loss reduction to the next: [2, 40) ms holds the loads from
    # 8.2 and 22.2 ms and the gaps ending at 8.0 (0.2), 16.2 (6.0) and 30.2 ms
    # (30.0); [40, 75) ms the loads from 60.2 and 70.2 ms and the 2 ms gap
    lines = [l for l in out.splitlines() if l.startswith("step ")]
    assert len(lines) == 2
    assert "2 weight loads busy 16 ms, link idle 36 ms" in lines[0]
    assert "0-0.5 ms: n=1 0.2 ms" in lines[0] and "4.5-20 ms: n=1 6.0 ms" in lines[0]
    assert ">= 20 ms: n=1 30.0 ms" in lines[0]
    assert "link idle 2 ms" in lines[1] and "0.5-4.5 ms: n=1 2.0 ms" in lines[1]
    # the drain kernel counts as device-to-host traffic, not as compute; of the
    # 4.2 ms of compute (union), the 0.1 ms reduction at 40 ms has no load in flight
    assert "1 of them drain kernels" in out
    assert "overlap H2D      with kernels: 0.976" in out
