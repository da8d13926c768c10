"""Throughput of host-streamed training steps on one MI355X.

    python bench.py [--gpus 1] [--steps 3] [--warmup 1] [--config C3] [--no-cpu-baseline]

One step = every micro-batch's streamed forward and backward (weights copied
layer by layer from pinned host memory, checkpoint recompute, gradient slabs
drained into host fp32 grads), the flush, and the host AdamW -- the whole
path.  Inputs are seeded synthetic token ids; weights are N(0, 0.02) from a
seed.  Prints one JSON line.

`roofline` reports the dominant kernel of the timed steps: the library times
every kernel it launches with HIP events on the stream it runs on
(mt_kernel_timing) and sums each kind's algorithmic flop or bytes; the kind
with the most device time on the compute stream is reported against its peak.
`kernels` lists every kind.  `cpu_baseline` times the CPU oracle on one
decoder layer of the same shape.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
KERNEL_COPY_WGS = (3, 4, 8, 32)


def layer_matrix_params(cfg, layer: int) -> int:
    """Weights one token multiplies in block `layer`: the attention projections
    plus the dense SwiGLU FFN, or for a mixture-of-experts block the router and
    the top_k experts it is routed to."""
    h = cfg.hidden
    qd, kvd = cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    attn = h * qd + 2 * h * kvd + qd * h
    if getattr(cfg, "n_experts", 0) and cfg.is_moe(layer):
        return attn + h * cfg.n_experts + cfg.top_k * 3 * h * cfg.expert_ffn
    return attn + 3 * h * cfg.ffn


def model_flops_per_token(cfg) -> float:
    """6 * (block matrices + LM head) + causal attention (fwd + bwd = 3x fwd);
    recompute is not counted."""
    qd = cfg.n_heads * cfg.head_dim
    p_mm = sum(layer_matrix_params(cfg, l) for l in range(cfg.n_layers))
    return 6.0 * (p_mm + cfg.hidden * cfg.vocab) + 6.0 * cfg.n_layers * cfg.seq_len * qd


def hardware_flops_per_token(cfg) -> float:
    """Adds the recompute forwards (every layer outside the last segment) and
    the flash-backward recompute of the scores (2.5x the forward attention)."""
    qd = cfg.n_heads * cfg.head_dim
    K = cfg.ckpt_interval
    nseg = -(-cfg.n_layers // K)
    recomputed = (nseg - 1) * K
    attn_fwd = 2.0 * cfg.seq_len * qd
    return model_flops_per_token(cfg) + \
        sum(2.0 * layer_matrix_params(cfg, l) + attn_fwd for l in range(recomputed)) + \
        cfg.n_layers * 0.5 * attn_fwd


def time_dominant_gemm(sess, reps: int = 20):
    """SwiGLU gate/up GEMM of one block (T x 2F x h, bf16 MFMA), timed with
    HIP events on the library's compute stream."""
    import torch
    import host_memory_centric_stateless_amd as mt
    cfg = sess.cfg
    T, h, F = cfg.micro_batch * cfg.seq_len, cfg.hidden, cfg.ffn
    dev = sess.device
    stream = sess.streams[1]
    g = torch.Generator(device="cpu").manual_seed(5)
    A = torch.randn(T, h, generator=g).to(torch.bfloat16).to(dev)
    B = (torch.randn(2 * F, h, generator=g) * 0.02).to(torch.bfloat16).to(dev)
    m = torch.empty(T, F, dtype=torch.bfloat16, device=dev)
    gu = torch.empty(T, 2 * F, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    args = (mt.MT_GEMM_NT, mt.MT_EPI_SWIGLU, T, F, h, A, h, B, h, m, F)
    kw = dict(gu=gu, ldgu=2 * F, ffn=F, stream=stream)
    for _ in range(3):
        mt.mtk_gemm(*args, **kw)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        mt.mtk_gemm(*args, **kw)
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 2.0 * T * (2 * F) * h
    tflops = flops / (ms * 1e-3) / 1e12
    return {"kernel": "gemm_kernel<NT,SWIGLU> gate/up", "shape": [T, 2 * F, h],
            "ms": ms, "tflops": tflops, "flops": flops}


def link_roofline(nbytes: int, reps: int = 4):
    """Pinned host <-> device copy rates at layer-sized transfers: H2D alone,
    D2H alone, and both directions at once on two streams (GB/s)."""
    import torch
    dev = torch.device("cuda:0")
    h1 = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    h2 = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    d1 = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    d2 = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()

    def timed(fn_list):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True), s)
              for _, s in fn_list]
        torch.cuda.synchronize()
        for (e0, e1, s), (fn, _) in zip(ev, fn_list):
            with torch.cuda.stream(s):
                e0.record(s)
                for _ in range(reps):
                    fn()
                e1.record(s)
        torch.cuda.synchronize()
        return [nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9 for e0, e1, _ in ev]

    h2d = lambda: d1.copy_(h1, non_blocking=True)
    d2h = lambda: h2.copy_(d2, non_blocking=True)
    timed([(h2d, sa)])
    out = {"bytes_per_copy": nbytes, "h2d_GBps": timed([(h2d, sa)])[0],
           "d2h_GBps": timed([(d2h, sb)])[0]}
    a, b = timed([(h2d, sa), (d2h, sb)])
    out["duplex_h2d_GBps"], out["duplex_d2h_GBps"] = a, b
    # device -> host by a copy kernel writing host-mapped memory, alone and
    # while the copy engine runs host -> device
    import host_memory_centric_stateless_amd as mt
    for wgs in KERNEL_COPY_WGS:
        kd2h = lambda: mt.mtk_copy(h2, d2, nbytes, wgs, stream=sb)
        out[f"kernel{wgs}_d2h_GBps"] = timed([(kd2h, sb)])[0]
        a, b = timed([(h2d, sa), (kd2h, sb)])
        out[f"kernel{wgs}_duplex_h2d_GBps"], out[f"kernel{wgs}_duplex_d2h_GBps"] = a, b
    return out


def block_gemm_shapes(cfg):
    """(kind, layout, epilogue, M, N, K) of every GEMM of one block at this shape."""
    import host_memory_centric_stateless_amd as mt
    T, h, F = cfg.micro_batch * cfg.seq_len, cfg.hidden, cfg.ffn
    qd, kvd = cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    ldq = qd + 2 * kvd
    NT, NN, TN = mt.MT_GEMM_NT, mt.MT_GEMM_NN, mt.MT_GEMM_TN
    return [("gemm_nt_rope qkv", NT, mt.MT_EPI_ROPE, T, ldq, h),
            ("gemm_nt_resid o", NT, mt.MT_EPI_F32_RESID, T, h, qd),
            ("gemm_nt_swiglu gate/up", NT, mt.MT_EPI_SWIGLU, T, F, h),
            ("gemm_nt_resid down", NT, mt.MT_EPI_F32_RESID, T, h, F),
            ("gemm_nn_swiglu_bwd dm", NN, mt.MT_EPI_SWIGLU_BWD, T, F, h),
            ("gemm_tn_bf16 dWdown", TN, mt.MT_EPI_BF16, h, F, T),
            ("gemm_tn_bf16 dWgate/up", TN, mt.MT_EPI_BF16, 2 * F, h, T),
            ("gemm_nn_f32 dn2", NN, mt.MT_EPI_F32, T, h, 2 * F),
            ("gemm_nn_bf16 dO", NN, mt.MT_EPI_BF16, T, qd, h),
            ("gemm_tn_bf16 dWo", TN, mt.MT_EPI_BF16, h, qd, T),
            ("gemm_tn_bf16 dWqkv", TN, mt.MT_EPI_BF16, ldq, h, T),
            ("gemm_nn_f32 dn1", NN, mt.MT_EPI_F32, T, h, ldq)]


def head_gemm_shapes(cfg, sess_req=None):
    """The LM head's weight-gradient product of one vocabulary chunk."""
    import host_memory_centric_stateless_amd as mt
    T, h = cfg.micro_batch * cfg.seq_len, cfg.hidden
    nch = sess_req.head_chunks if sess_req else 1
    rows = min(cfg.vocab, ((cfg.vocab + nch - 1) // nch + 255) // 256 * 256)
    return [("gemm_tn_bf16 dWhead", mt.MT_GEMM_TN, mt.MT_EPI_BF16, rows, h, T)]


def mfma_ceiling(iters: int = 8000, workgroups: int = 2048):
    """The MFMA rate of a chain of register-operand MFMAs (mtk_mfma_peak),
    with its output checked: the ceiling next to the nominal peak."""
    import torch
    import host_memory_centric_stateless_amd as mt
    out = torch.zeros(workgroups * 4, dtype=torch.float32, device="cuda:0")
    mt.mtk_mfma_peak(out, workgroups, 10)  # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    mt.mtk_mfma_peak(out, workgroups, iters)
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1)
    ch = mt.mtk_mfma_peak_chains()
    ok = bool(torch.all(out == ch * 16 * iters).item())
    flop = workgroups * 4 * ch * iters * 32768.0
    return {"kernel": f"mfma_peak ({ch} v_mfma_f32_32x32x16_bf16 chains per wave, register operands)",
            "ms": ms, "TFLOPs": flop / ms / 1e9, "frac_of_nominal": flop / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS,
            "output_checked": ok, "workgroups": workgroups, "iters": iters}


def probe(cfg, reps: int = 2):
    """Run every block GEMM at this shape `reps` times, then a device copy of
    known size (the calibration reference for hardware byte counters), one
    launch per line, timed with HIP events."""
    import torch
    import host_memory_centric_stateless_amd as mt
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(7)
    out = [mfma_ceiling()]
    T = cfg.micro_batch * cfg.seq_len
    cos, sin = mt.mt_host_rope_table(cfg.seq_len, cfg.head_dim, cfg.rope_base)
    cos_d, sin_d = torch.from_numpy(cos).to(dev), torch.from_numpy(sin).to(dev)
    from host_memory_centric_stateless_amd import make_config, mt_device_requirements
    req = mt_device_requirements(make_config(cfg))
    for name, lay, epi, M, N, K in block_gemm_shapes(cfg) + head_gemm_shapes(cfg, req):
        NN_ = 2 * N if epi == mt.MT_EPI_SWIGLU else N
        A = (torch.randn(M if lay != mt.MT_GEMM_TN else K, K if lay != mt.MT_GEMM_TN else M,
                         generator=g) * 0.5).to(torch.bfloat16).to(dev)
        B = (torch.randn(NN_ if lay == mt.MT_GEMM_NT else K, K if lay == mt.MT_GEMM_NT else NN_,
                         generator=g) * 0.02).to(torch.bfloat16).to(dev)
        lda, ldb = A.shape[1], B.shape[1]
        ob = 2 if epi in (mt.MT_EPI_BF16, mt.MT_EPI_SWIGLU, mt.MT_EPI_SWIGLU_BWD,
                          mt.MT_EPI_ROPE) else 4
        ldc = 2 * N if epi == mt.MT_EPI_SWIGLU_BWD else N
        C = torch.empty(M * ldc * ob, dtype=torch.uint8, device=dev)
        R = torch.zeros(M, N, dtype=torch.float32, device=dev) if epi == mt.MT_EPI_F32_RESID else None
        gu = torch.randn(M, 2 * N, generator=g).to(torch.bfloat16).to(dev) \
            if epi in (mt.MT_EPI_SWIGLU, mt.MT_EPI_SWIGLU_BWD) else None
        kw = dict(R=R, ldr=N if R is not None else 0, gu=gu, ldgu=2 * N if gu is not None else 0,
                  ffn=N if gu is not None else 0)
        if epi == mt.MT_EPI_ROPE:
            kw.update(rope_cos=cos_d, rope_sin=sin_d, rope_seq=cfg.seq_len, rope_dim=cfg.head_dim,
                      rope_cols=(cfg.n_heads + cfg.n_kv_heads) * cfg.head_dim)
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            mt.mtk_gemm(lay, epi, M, N, K, A, lda, B, ldb, C, ldc, **kw)
            e1.record()
            e1.synchronize()
            ms = e0.elapsed_time(e1)
            flop = 2.0 * M * NN_ * K
            out.append({"kernel": name, "MNK": [M, N, K], "ms": ms, "TFLOPs": flop / ms / 1e9,
                        "algorithmic_bytes": A.numel() * 2 + B.numel() * 2 + M * NN_ * ob})
        del A, B, C, R, gu
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device=dev)
    dst = torch.empty(nb, dtype=torch.uint8, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    mt.mtk_copy(dst, src, nb, 1024)
    e1.record()
    e1.synchronize()
    out.append({"kernel": "calibration copy16 1 GiB device->device", "bytes_read": nb,
                "bytes_written": nb, "ms": e0.elapsed_time(e1),
                "GBps": 2 * nb / e0.elapsed_time(e1) / 1e6})
    return out


CPU_SAMPLE_TOKENS = 4096


def cpu_baseline(cfg, budget_s: float = 30.0):
    """The oracle (fp32 NumPy) on one decoder layer of the same width:
    forward + recompute forward + backward, on this host's cores.  The sample
    holds at most CPU_SAMPLE_TOKENS tokens (one sequence of that length when
    the configuration's sequences are longer): the oracle's attention keeps
    the whole score matrix, which at 131,072 tokens would not fit in host
    memory.  tokens/s is the sample's model TFLOP/s at the full
    configuration's model flop per token."""
    from oracle import model as OM
    from synth_inputs import make_batch, tensor_specs
    full = cfg
    if cfg.micro_batch * cfg.seq_len > CPU_SAMPLE_TOKENS:
        seq = min(cfg.seq_len, CPU_SAMPLE_TOKENS)
        cfg = cfg.replace(seq_len=seq, micro_batch=max(1, CPU_SAMPLE_TOKENS // seq))
    rng = np.random.default_rng(0)
    T = cfg.micro_batch * cfg.seq_len
    W = {}
    for name, shape, kind in tensor_specs(cfg, 0):
        W[name] = (np.ones(shape, np.float32) if kind == "gain"
                   else (rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)))
    x = rng.standard_normal((T, cfg.hidden), dtype=np.float32)
    cos, sin = OM.rope_tables(cfg.seq_len, cfg.head_dim, cfg.rope_base, np.float32)
    t0 = time.perf_counter()
    y, _ = OM.block_forward(W, x, cfg, cos, sin, cfg.micro_batch)
    _, cache = OM.block_forward(W, x, cfg, cos, sin, cfg.micro_batch)
    OM.block_backward(W, cache, np.ones_like(y) * np.float32(1e-3), cfg, cos, sin, cfg.micro_batch)
    dt = time.perf_counter() - t0
    per_layer_model = (model_flops_per_token(cfg.replace(n_layers=1, vocab=0)))
    tflops = per_layer_model * T / dt / 1e12
    blas = _blas_info()
    tok_s = tflops * 1e12 / model_flops_per_token(full)
    return {"value": tflops, "unit": "model TFLOP/s", "cores": blas["threads"], "kind": "oracle",
            "cpu_model": _cpu_model(), "blas": blas["library"], "blas_threads": blas["threads"],
            "logical_cpus": os.cpu_count(),
            "sample": f"1 decoder layer of {full.name} (hidden {cfg.hidden}) forward + recompute + "
                      f"backward on {cfg.micro_batch} x {cfg.seq_len} tokens, fp32 NumPy, {dt:.1f} s; "
                      f"tokens/s equivalent for the whole model {tok_s:.1f}"}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_info() -> dict:
    """The BLAS numpy calls and the size of its thread pool, as loaded in this
    process (the pool the oracle's matrix products actually ran on)."""
    try:
        import threadpoolctl
        for p in threadpoolctl.threadpool_info():
            if p.get("user_api") == "blas":
                return {"library": f"{p.get('internal_api')} {p.get('version')} "
                                   f"({p.get('threading_layer')}, {p.get('architecture')})",
                        "threads": int(p.get("num_threads"))}
    except Exception:
        pass
    return {"library": "unknown", "threads": int(os.environ.get("OMP_NUM_THREADS", 1))}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_tn_bf16_7b_shape_traffic.txt")


def measured_traffic(kernel: str, cfg_name: str, default_shape: bool):
    """HBM bytes per launch of the TN weight-gradient GEMM from the committed
    FETCH_SIZE / WRITE_SIZE counter runs (calibrated), or None when the
    counters do not describe this kernel, workload or kernel source."""
    import hashlib
    if kernel != "gemm_tn_bf16" or cfg_name != "llama-7B-shape" or not default_shape:
        return None
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = dict(l.split(": ", 1) for l in text.splitlines() if ": " in l and not l.startswith(" "))
    # the kernel's source and the device helpers it includes
    h = hashlib.sha256()
    for name in ("gemm.hip", "common.h"):
        with open(os.path.join(ROOT, "host_memory_centric_stateless_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if fields.get("gemm_source_sha256", "").split()[0:1] != [h.hexdigest()]:
        return None
    return float(fields["traffic_bytes_per_launch"])


def host_roofline(n: int = 1 << 28, reps: int = 5):
    """Host-memory bandwidth of a STREAM-style triad (a = b + s c, 12 bytes per
    element counted) on the library's default thread count: the roofline of
    the host AdamW and slab accumulation."""
    import host_memory_centric_stateless_amd as mt
    from host_memory_centric_stateless_amd.session import aligned_zeros
    a, b, c = aligned_zeros(n), aligned_zeros(n), aligned_zeros(n)
    b += 1.0
    c += 2.0
    t = mt.mt_host_triad(a, b, c, 3.0, reps=reps)
    del a, b, c
    return {"triad_GBps": 12.0 * n / t / 1e9, "bytes": 12 * n, "threads": "library default (<= 16)"}


def overlap(s0, s1):
    """Copy/compute overlap over the timed steps, from the library's HIP timing
    events: |copies AND kernels| / min(|copies|, |kernels|) (union measures;
    copies = weight and input loads and gradient drains on the host link)."""
    c = s1["timed_copy_ms"] - s0["timed_copy_ms"]
    k = s1["timed_kernel_ms"] - s0["timed_kernel_ms"]
    both = s1["timed_overlap_ms"] - s0["timed_overlap_ms"]
    return {"value": both / min(c, k) if min(c, k) > 0 else None, "copy_busy_ms": c,
            "kernel_busy_ms": k, "both_ms": both,
            "measured": "HIP events around every load, drain and kernel launch, timed steps"}


def mem_available_gib() -> float:
    with open("/proc/meminfo") as f:
        for line in f:
            if line.startswith("MemAvailable:"):
                return int(line.split()[1]) / 2**20
    return float("inf")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="C3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--host-threads", type=int, default=0)
    ap.add_argument("--drain-workgroups", type=int, default=None,
                    help="slab drain: 0 = DMA engine, n = copy kernel of n workgroups "
                         "(default: the library's)")
    ap.add_argument("--grad-slabs", type=int, default=0,
                    help="override the configuration's gradient slab count")
    ap.add_argument("--micro-batch", type=int, default=0,
                    help="override the configuration's sequences per micro-batch")
    ap.add_argument("--grad-accum", type=int, default=0,
                    help="override the configuration's micro-batches per step")
    ap.add_argument("--micro-batches-per-pass", type=int, default=1,
                    help="micro-batches sharing each weight residency in the headline run")
    ap.add_argument("--no-layer-major", action="store_true",
                    help="skip the second measurement with all of a step's micro-batches "
                         "in one pass")
    ap.add_argument("--host-mem-gib", type=float, default=0.0,
                    help="host memory the run may use (default: MemAvailable); the run stops "
                         "before allocating if the host state and pinned buffers exceed it")
    ap.add_argument("--no-fp32-slabs", action="store_true",
                    help="skip the second measurement of the headline step with fp32 slabs")
    ap.add_argument("--probe", action="store_true",
                    help="only run each block GEMM at this shape and a calibration copy")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the method's multi-GPU "
              "data parallelism is not implemented in this library", file=sys.stderr)
        sys.exit(2)

    import torch
    from host_memory_centric_stateless_amd import Session
    from synth_inputs import MOE_PRESETS, PRESETS, make_batch, weight_stream

    cfg = PRESETS[args.config] if args.config in PRESETS else MOE_PRESETS[args.config]
    if args.micro_batch or args.grad_accum or args.grad_slabs:
        cfg = cfg.replace(micro_batch=args.micro_batch or cfg.micro_batch,
                          grad_accum=args.grad_accum or cfg.grad_accum,
                          n_grad_slabs=args.grad_slabs or cfg.n_grad_slabs)
    if args.probe:
        for row in probe(cfg):
            print(json.dumps(row), flush=True)
        return
    from host_memory_centric_stateless_amd import make_config, mt_device_requirements
    req = mt_device_requirements(make_config(cfg, micro_batches_per_pass=args.micro_batches_per_pass))
    need_gib = (req.host_state + req.pinned_host) / 2**30 + 6.0  # + interpreter, torch, staging
    limit_gib = args.host_mem_gib or mem_available_gib()
    print(f"[bench] host memory: need ~{need_gib:.0f} GiB, limit {limit_gib:.0f} GiB",
          file=sys.stderr, flush=True)
    if need_gib > limit_gib:
        print(f"bench.py: {cfg.name} needs ~{need_gib:.0f} GiB of host memory for its fp32 state "
              f"and pinned buffers; {limit_gib:.0f} GiB are available", file=sys.stderr)
        sys.exit(3)
    t0 = time.perf_counter()
    sess = Session(cfg, host_threads=args.host_threads, drain_workgroups=args.drain_workgroups,
                   micro_batches_per_pass=args.micro_batches_per_pass)
    sess.load_weights(weight_stream(cfg, 0))
    print(f"[bench] {cfg.name}: init {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    tokens_per_step = cfg.grad_accum * cfg.micro_batch * cfg.seq_len
    losses = []
    for w in range(args.warmup):
        tok, lab = make_batch(cfg, 1 + w)
        losses.append(sess.step(tok, lab, 1 + w))
        print(f"[bench] warmup {w} loss {losses[-1]:.4f}", file=sys.stderr, flush=True)
    batches = [make_batch(cfg, 1 + args.warmup + k) for k in range(args.steps)]
    from host_memory_centric_stateless_amd import mt_get_kernel_times, mt_kernel_timing
    mt_kernel_timing(sess.ctx, True)
    s0 = sess.stats()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    # Each step returns once its loss is known; its host updates finish under
    # the next step's forward (each streamed unit's copy waits for that
    # unit's update).  The flush puts the last step's host work inside the
    # timed region.
    for k in range(args.steps):
        tok, lab = batches[k]
        losses.append(sess.step(tok, lab, 1 + args.warmup + k, flush=False))
        print(f"[bench] step {k} loss {losses[-1]:.4f} t={time.perf_counter() - t_start:.2f}s",
              file=sys.stderr, flush=True)
    sess.flush()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    s1 = sess.stats()
    ktimes = mt_get_kernel_times(sess.ctx)
    mt_kernel_timing(sess.ctx, False)

    ms_per_step = 1e3 * elapsed / args.steps
    tok_s = tokens_per_step * args.steps / elapsed
    model_tflops = model_flops_per_token(cfg) * tok_s / 1e12
    hw_tflops = hardware_flops_per_token(cfg) * tok_s / 1e12
    h2d = (s1["h2d_bytes"] - s0["h2d_bytes"]) / elapsed / 1e9
    d2h = (s1["d2h_bytes"] - s0["d2h_bytes"]) / elapsed / 1e9
    adamw_s = (s1["adamw_s"] - s0["adamw_s"]) / args.steps

    gemm = time_dominant_gemm(sess)
    ceiling = mfma_ceiling()
    link = link_roofline(sess.req.weight_buf)
    host = host_roofline()
    # host bytes per parameter and step: the last micro-batch's fused add + AdamW +
    # bf16 recast (32 B, or 36 B when it adds to an earlier micro-batch's gradient);
    # the other micro-batches' bf16 slab accumulation (6 B for the first, 10 B after)
    n_params = sum(sess.layout[g][1] for g in sess.groups)
    adamw_bpp = 36 if cfg.grad_accum > 1 else 32
    acc_bpp = (6 + 10 * (cfg.grad_accum - 2)) if cfg.grad_accum > 1 else 0
    acc_s = (s1["accumulate_s"] - s0["accumulate_s"]) / args.steps
    step_no = 1 + args.warmup + args.steps
    kernels = []
    for k in ktimes:
        row = {"kernel": k["name"], "launches_per_step": k["launches"] / args.steps,
               "ms_per_step": k["ms"] / args.steps, "avg_launch_ms": k["ms"] / max(k["launches"], 1)}
        if k["flop"] > 0:
            row["TFLOPs"] = k["flop"] / (k["ms"] * 1e-3) / 1e12
            row["frac_mfma_peak"] = row["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS
        else:
            row["GBps"] = k["bytes"] / (k["ms"] * 1e-3) / 1e9
        kernels.append(row)
    copies = ("drain_d2h", "h2d_load", "h2d_input")  # host-link copies, timed like kernels
    dom = next(k for k in ktimes if k["name"] not in copies)
    if dom["flop"] > 0:
        ach = dom["flop"] / (dom["ms"] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": ach, "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK_TFLOPS}
    else:
        ach = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": ach / HBM_PEAK_GBPS}
    traffic = measured_traffic(dom["name"], cfg.name,
                               not (args.micro_batch or args.grad_accum or args.grad_slabs))
    if roofline["bound"] == "mfma":
        roofline["frac_of_measured_ceiling"] = roofline["achieved"] / ceiling["TFLOPs"]
    roofline.update({"traffic": traffic, "kernel": dom["name"], "launches": dom["launches"],
                     "avg_launch_ms": dom["ms"] / dom["launches"],
                     "algorithmic_per_launch": (dom["flop"] or dom["bytes"]) / dom["launches"],
                     "measured": "HIP events around each launch on its stream, timed steps",
                     "traffic_unit": "HBM bytes per launch (FETCH_SIZE x 2 + WRITE_SIZE, "
                                     "calibrated on a 1 GiB copy)" if traffic else None})
    sess.close()

    # The same training step with every micro-batch of the step in one pass
    # (layer-major gradient accumulation): each layer's weights cross the
    # host link once per step instead of once per micro-batch.
    layer_major = None
    if cfg.grad_accum > 1 and args.micro_batches_per_pass == 1 and not args.no_layer_major:
        t0 = time.perf_counter()
        lm = Session(cfg, host_threads=args.host_threads, drain_workgroups=args.drain_workgroups,
                     micro_batches_per_pass=cfg.grad_accum, host_from=sess)
        lm.bind()
        print(f"[bench] layer-major pass: init {time.perf_counter() - t0:.1f} s", file=sys.stderr,
              flush=True)
        for w in range(args.warmup):
            tok, lab = make_batch(cfg, step_no)
            lm.step(tok, lab, step_no)
            step_no += 1
        lb = [make_batch(cfg, step_no + k) for k in range(args.steps)]
        mt_kernel_timing(lm.ctx, True)
        l0 = lm.stats()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        lm_losses = []
        for k in range(args.steps):
            tok, lab = lb[k]
            lm_losses.append(lm.step(tok, lab, step_no + k, flush=False))
        lm.flush()
        torch.cuda.synchronize()
        lel = time.perf_counter() - t_start
        l1 = lm.stats()
        lm.close()
        step_no += args.steps
        ltok = tokens_per_step * args.steps / lel
        layer_major = {
            "micro_batches_per_pass": cfg.grad_accum, "ms_per_step": 1e3 * lel / args.steps,
            "tokens_per_s": ltok, "model_tflops": model_flops_per_token(cfg) * ltok / 1e12,
            "hardware_tflops": hardware_flops_per_token(cfg) * ltok / 1e12,
            "h2d_GBps": (l1["h2d_bytes"] - l0["h2d_bytes"]) / lel / 1e9,
            "weight_loads_per_step": (l1["weight_loads"] - l0["weight_loads"]) / args.steps,
            "overlap": overlap(l0, l1),
            "loss_last": lm_losses[-1],
            "note": "same step (4 micro-batches of 1 x 4096, each normalised by its own "
                    "label count, gradients accumulated); the micro-batches share each "
                    "weight residency"}
        print(f"[bench] layer-major pass: {layer_major['ms_per_step']:.0f} ms/step, "
              f"{ltok:.0f} tokens/s", file=sys.stderr, flush=True)
    # The headline step again with fp32 gradient slabs (the plain reading of
    # the pages: fp32 gradients to the host) instead of the default bf16 slabs.
    fp32_slabs = None
    if not args.no_fp32_slabs:
        t0 = time.perf_counter()
        fs = Session(cfg, host_threads=args.host_threads, drain_workgroups=args.drain_workgroups,
                     micro_batches_per_pass=args.micro_batches_per_pass, slab_bf16=False,
                     host_from=sess)
        fs.bind()
        print(f"[bench] fp32 slabs: init {time.perf_counter() - t0:.1f} s", file=sys.stderr,
              flush=True)
        for w in range(args.warmup):
            tok, lab = make_batch(cfg, step_no)
            fs.step(tok, lab, step_no)
            step_no += 1
        fb = [make_batch(cfg, step_no + k) for k in range(args.steps)]
        f0 = fs.stats()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for k in range(args.steps):
            tok, lab = fb[k]
            fs.step(tok, lab, step_no + k, flush=False)
        fs.flush()
        torch.cuda.synchronize()
        fel = time.perf_counter() - t_start
        f1 = fs.stats()
        fs.close()
        step_no += args.steps
        ftok = tokens_per_step * args.steps / fel
        fp32_slabs = {
            "ms_per_step": 1e3 * fel / args.steps, "tokens_per_s": ftok,
            "model_tflops": model_flops_per_token(cfg) * ftok / 1e12,
            "d2h_GBps": (f1["d2h_bytes"] - f0["d2h_bytes"]) / fel / 1e9,
            "h2d_GBps": (f1["h2d_bytes"] - f0["h2d_bytes"]) / fel / 1e9,
            "note": "headline step with fp32 gradient slabs (4 bytes per gradient element "
                    "device -> host instead of 2)"}
        print(f"[bench] fp32 slabs: {fp32_slabs['ms_per_step']:.0f} ms/step", file=sys.stderr,
              flush=True)
    base = None if args.no_cpu_baseline else cpu_baseline(cfg)

    out = {
        "metric": "model TFLOPS & tokens/s per GPU, host-streamed layer fwd+bwd (7B/14B shapes)",
        "value": model_tflops, "unit": "model TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "layers": cfg.n_layers, "hidden": cfg.hidden,
                   "heads": cfg.n_heads, "kv_heads": cfg.n_kv_heads, "ffn": cfg.ffn,
                   "vocab": cfg.vocab, "micro_batch": cfg.micro_batch, "seq_len": cfg.seq_len,
                   "grad_accum": cfg.grad_accum, "ckpt_interval": cfg.ckpt_interval,
                   "grad_slabs": cfg.n_grad_slabs, "global_batch_tokens": tokens_per_step,
                   "micro_batches_per_pass": args.micro_batches_per_pass},
        "tokens_per_s": tok_s, "hardware_tflops": hw_tflops,
        "slab_drain": ("dma" if sess.c.drain_workgroups == 0
                       else f"copy kernel, {sess.c.drain_workgroups} workgroups"),
        "mfma_frac_end_to_end": model_tflops / MFMA_BF16_PEAK_TFLOPS,
        "h2d_GBps": h2d, "d2h_GBps": d2h, "adamw_s_per_step": adamw_s,
        "host_roofline": host,
        "host_adamw": {"GBps": n_params * adamw_bpp / adamw_s / 1e9 if adamw_s > 0 else None,
                       "bytes_per_param": adamw_bpp, "params": n_params,
                       "frac_of_triad": (n_params * adamw_bpp / adamw_s / 1e9) / host["triad_GBps"]
                       if adamw_s > 0 else None},
        "host_accumulate": {"GBps": n_params * acc_bpp / acc_s / 1e9 if acc_s > 0 else None,
                            "bytes_per_param_per_step": acc_bpp},
        "loss_last": losses[-1],
        "link_roofline": link,
        "h2d_frac_of_link": h2d / link["h2d_GBps"],
        "pipeline": {k: (s1[k] - s0[k]) / args.steps for k in
                     ("slab_waits", "slab_wait_s", "accumulate_s", "weight_loads", "layer_forwards",
                      "layer_backwards")},
        "overlap": overlap(s0, s1),
        "roofline": roofline, "kernels": kernels,
        "isolated_swiglu_gemm": {"TFLOPs": gemm["tflops"], "ms": gemm["ms"], "shape_MNK": gemm["shape"]},
        "mfma_ceiling": ceiling,
        "layer_major": layer_major,
        "fp32_slabs": fp32_slabs,
        "cpu_baseline": base,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
