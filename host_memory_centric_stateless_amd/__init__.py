"""Python binding of libmt (host-memory-centric, layer-streamed training).

Argument marshalling only: every step of the training path runs in libmt's
HIP kernels and its C++ host runtime.  PyTorch is used for device memory and
streams (the device arena and the three streams are torch allocations).

torch is imported before libmt.so is loaded so that the library binds to the
HIP runtime torch already loaded (one HIP runtime per process).  If the
library is missing this module raises ImportError: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch  # noqa: F401  (must load its HIP runtime first)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmt.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python host_memory_centric_stateless_amd/build.py`")
_lib = C.CDLL(LIB_PATH)


def _hip_runtimes():
    with open("/proc/self/maps") as f:
        return sorted({l.split()[-1] for l in f if "libamdhip64" in l})


if len(_hip_runtimes()) > 1:
    raise ImportError(f"two HIP runtimes loaded: {_hip_runtimes()}")

# --------------------------------------------------------------------- enums
MT_OK, MT_E_ARG, MT_E_STATE, MT_E_HIP, MT_E_NOMEM, MT_E_UNBOUND, MT_E_ABORTED = 0, -1, -2, -3, -4, -5, -6
MT_GROUP_EMBED, MT_GROUP_HEAD = -1, -2
MT_GEMM_NT, MT_GEMM_NN, MT_GEMM_TN = 0, 1, 2
(MT_EPI_BF16, MT_EPI_F32, MT_EPI_F32_RESID, MT_EPI_F32_ACCUM, MT_EPI_SWIGLU, MT_EPI_SWIGLU_BWD,
 MT_EPI_ROPE) = range(7)
_STATUS = {0: "MT_OK", -1: "MT_E_ARG", -2: "MT_E_STATE", -3: "MT_E_HIP", -4: "MT_E_NOMEM",
           -5: "MT_E_UNBOUND", -6: "MT_E_ABORTED"}


class MtError(RuntimeError):
    def __init__(self, status, what, detail=""):
        self.status = status
        super().__init__(f"{what} -> {_STATUS.get(status, status)} {detail}".strip())


# ----------------------------------------------------------------- structs
class mt_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("rms_eps", C.c_float), ("rope_base", C.c_float),
                ("micro_batch", C.c_int32), ("seq_len", C.c_int32), ("ckpt_interval", C.c_int32),
                ("n_grad_slabs", C.c_int32), ("host_threads", C.c_int32),
                ("slab_bf16", C.c_int32), ("drain_workgroups", C.c_int32),
                ("micro_batches_per_pass", C.c_int32), ("head_token_chunk", C.c_int32),
                ("n_experts", C.c_int32), ("top_k", C.c_int32), ("expert_ffn", C.c_int32),
                ("moe_every", C.c_int32)]


class mt_tensor_desc(C.Structure):
    _fields_ = [("name", C.c_char * 16), ("offset", C.c_int64), ("numel", C.c_int64),
                ("rows", C.c_int32), ("cols", C.c_int32)]


class mt_device_req(C.Structure):
    _fields_ = [("weight_buf", C.c_size_t), ("grad_slab", C.c_size_t), ("window", C.c_size_t),
                ("checkpoints", C.c_size_t), ("workspace", C.c_size_t),
                ("device_total", C.c_size_t), ("pinned_host", C.c_size_t),
                ("host_state", C.c_size_t), ("unit_elems", C.c_int64),
                ("head_chunks", C.c_int32), ("reserved", C.c_int32)]


class mt_device_arena(C.Structure):
    _fields_ = [("weight_buf", C.c_void_p * 2), ("grad_slab", C.c_void_p * 64),
                ("window", C.c_void_p), ("checkpoints", C.c_void_p), ("workspace", C.c_void_p),
                ("stream_prefetch", C.c_void_p), ("stream_compute", C.c_void_p),
                ("stream_offload", C.c_void_p), ("weight_buf_bytes", C.c_size_t),
                ("grad_slab_bytes", C.c_size_t), ("window_bytes", C.c_size_t),
                ("checkpoints_bytes", C.c_size_t), ("workspace_bytes", C.c_size_t)]


class mt_adamw_hparams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double)]


class mt_stats(C.Structure):
    _fields_ = [("h2d_bytes", C.c_int64), ("d2h_bytes", C.c_int64), ("weight_loads", C.c_int64),
                ("layer_forwards", C.c_int64), ("layer_backwards", C.c_int64),
                ("slab_waits", C.c_int64), ("slab_wait_s", C.c_double),
                ("accumulate_s", C.c_double), ("adamw_s", C.c_double),
                ("microbatches", C.c_int64), ("timed_copy_ms", C.c_double),
                ("timed_kernel_ms", C.c_double), ("timed_overlap_ms", C.c_double)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class mt_kernel_time(C.Structure):
    _fields_ = [("name", C.c_char * 32), ("launches", C.c_int64), ("ms", C.c_double),
                ("flop", C.c_double), ("bytes", C.c_double)]


class mt_gemm_args(C.Structure):
    _fields_ = [("layout", C.c_int32), ("epilogue", C.c_int32), ("M", C.c_int64),
                ("N", C.c_int64), ("K", C.c_int64), ("A", C.c_void_p), ("lda", C.c_int64),
                ("B", C.c_void_p), ("ldb", C.c_int64), ("C", C.c_void_p), ("ldc", C.c_int64),
                ("R", C.c_void_p), ("ldr", C.c_int64), ("gu", C.c_void_p), ("ldgu", C.c_int64),
                ("ffn", C.c_int64), ("rope_cos", C.c_void_p), ("rope_sin", C.c_void_p),
                ("rope_cols", C.c_int64), ("rope_seq", C.c_int32), ("rope_dim", C.c_int32),
                ("group_off", C.c_void_p), ("groups", C.c_int32), ("group_reserved", C.c_int32),
                ("group_stride_b", C.c_int64), ("group_stride_c", C.c_int64)]


_P = C.c_void_p
_I32, _I64, _F = C.c_int32, C.c_int64, C.c_float
_SIGS = {
    "mt_layout": ([C.POINTER(mt_config), _I32, C.POINTER(mt_tensor_desc), _I32,
                   C.POINTER(_I32), C.POINTER(_I64)], C.c_int),
    "mt_device_requirements": ([C.POINTER(mt_config), C.POINTER(mt_device_req)], C.c_int),
    "mt_create": ([C.POINTER(mt_config), C.POINTER(mt_device_arena), C.POINTER(_P)], C.c_int),
    "mt_bind_layer": ([_P, _I32, _P, _P, _P, _P, _I64], C.c_int),
    "mt_forward": ([_P, _P, _P, _F, _P], C.c_int),
    "mt_backward": ([_P, _I32], C.c_int),
    "mt_backward_step": ([_P, _I32, C.POINTER(mt_adamw_hparams), _I64], C.c_int),
    "mt_flush_grads": ([_P], C.c_int),
    "mt_sync_loss": ([_P], C.c_int),
    "mt_step_loss": ([_P, C.POINTER(C.c_float)], C.c_int),
    "mt_moe_routing": ([_P, _I32, _P], C.c_int),
    "mt_adamw_step": ([_P, C.POINTER(mt_adamw_hparams), _I64], C.c_int),
    "mt_get_stats": ([_P, C.POINTER(mt_stats)], C.c_int),
    "mt_last_error": ([_P], C.c_char_p),
    "mt_kernel_timing": ([_P, _I32], C.c_int),
    "mt_get_kernel_times": ([_P, C.POINTER(mt_kernel_time), _I32, C.POINTER(_I32)], C.c_int),
    "mt_destroy": ([_P], None),
    "mt_host_cast_bf16": ([_P, _P, _I64, _I32], C.c_int),
    "mt_host_adamw": ([_P, _P, _P, _P, _P, _I64, C.POINTER(mt_adamw_hparams), _I64, _I32], C.c_int),
    "mt_host_accumulate": ([_P, _P, _I64, _I32, _I32], C.c_int),
    "mt_host_adamw_slab": ([_P, _P, _P, _P, _P, _P, _I32, _I32, _I64, C.POINTER(mt_adamw_hparams),
                            _I64, _I32], C.c_int),
    "mt_host_rope_table": ([_I32, _I32, _F, _P, _P], C.c_int),
    "mt_host_triad": ([_P, _P, _P, _F, _I64, _I32, _I32, C.POINTER(C.c_double)], C.c_int),
    "mtk_gemm": ([C.POINTER(mt_gemm_args), _P], C.c_int),
    "mtk_rmsnorm_fwd": ([_P, _P, _P, _P, _I64, _I32, _F, _P], C.c_int),
    "mtk_rmsnorm_bwd_workspace": ([_I64, _I32], C.c_size_t),
    "mtk_rmsnorm_bwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _P], C.c_int),
    "mtk_rmsnorm_bwd_noalloc": ([_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _P], C.c_int),
    "mtk_noalloc_scratch_bytes": ([], C.c_size_t),
    "mtk_rope": ([_P, _I64, _I32, _I32, _I32, _I32, _P, _P, _I32, _P], C.c_int),
    "mtk_attention_fwd": ([_P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P], C.c_int),
    "mtk_attention_bwd_workspace": ([_I32, _I32, _I32, _I32, _I32], C.c_size_t),
    "mtk_attention_bwd": ([_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P], C.c_int),
    "mtk_attention_bwd_rope": ([_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P],
                               C.c_int),
    "mtk_cross_entropy": ([_P, _I64, _P, _I64, _I32, _F, _I64, _P, _I64, _P, _P, _P], C.c_int),
    "mtk_copy": ([_P, _P, C.c_size_t, _I32, _P], C.c_int),
    "mtk_mfma_peak": ([_P, _I32, _I32, _P], C.c_int),
    "mtk_mfma_peak_chains": ([], C.c_int32),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTED = sorted(_SIGS)


def lib():
    return _lib


def _check(status, what, ctx=None):
    if status != MT_OK:
        detail = _lib.mt_last_error(ctx).decode() if ctx else ""
        raise MtError(status, what, detail)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    return s.cuda_stream if hasattr(s, "cuda_stream") else int(s)


# ------------------------------------------------------------ config helpers
DEFAULT_DRAIN_WORKGROUPS = 4  # slabs leave through a 4-workgroup copy kernel


def default_drain_workgroups(cfg, slab_bf16: bool = True, micro_batches_per_pass: int = 1) -> int:
    """Copy-kernel workgroups for the slab drain.  A drain of three
    workgroups leaves the weight loads more of the link and trails into the
    next micro-batch's forward pass, whose device-to-host direction is
    otherwise idle: that needs a next micro-batch in the step (more passes per
    step than one) and bf16 slabs (fp32 slabs carry twice the bytes).
    Otherwise the tail of the drain would hold up the step's end, and four
    workgroups keep up."""
    passes = max(1, int(getattr(cfg, "grad_accum", 1)) // max(1, int(micro_batches_per_pass)))
    return 3 if (slab_bf16 and passes > 1) else DEFAULT_DRAIN_WORKGROUPS


def make_config(cfg, host_threads: int = 0, slab_bf16: bool = True,
                drain_workgroups: int = DEFAULT_DRAIN_WORKGROUPS,
                micro_batches_per_pass: int = 1, head_token_chunk: int = 0) -> mt_config:
    """mt_config from any object with the ModelConfig attribute names."""
    return mt_config(cfg.n_layers, cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn,
                     cfg.vocab, cfg.rms_eps, cfg.rope_base, cfg.micro_batch, cfg.seq_len,
                     cfg.ckpt_interval, cfg.n_grad_slabs, host_threads, int(bool(slab_bf16)),
                     int(drain_workgroups), int(micro_batches_per_pass), int(head_token_chunk),
                     int(getattr(cfg, "n_experts", 0)), int(getattr(cfg, "top_k", 2)),
                     int(getattr(cfg, "expert_ffn", 0)), int(getattr(cfg, "moe_every", 1)))


# ------------------------------------------------------------- C-ABI calls
def mt_layout(cfg: mt_config, group: int):
    n = _I32()
    total = _I64()
    descs = (mt_tensor_desc * 16)()
    _check(_lib.mt_layout(C.byref(cfg), group, descs, 16, C.byref(n), C.byref(total)), "mt_layout")
    return [(d.name.decode(), d.offset, d.numel, d.rows, d.cols) for d in descs[:n.value]], total.value


def mt_device_requirements(cfg: mt_config) -> mt_device_req:
    r = mt_device_req()
    _check(_lib.mt_device_requirements(C.byref(cfg), C.byref(r)), "mt_device_requirements")
    return r


def mt_create(cfg: mt_config, arena: mt_device_arena):
    ctx = _P()
    _check(_lib.mt_create(C.byref(cfg), C.byref(arena), C.byref(ctx)), "mt_create")
    return ctx


def mt_bind_layer(ctx, group, master, grad, m, v):
    for a in (master, grad, m, v):
        assert a.dtype == np.float32 and a.flags.c_contiguous
    _check(_lib.mt_bind_layer(ctx, group, _ptr(master), _ptr(grad), _ptr(m), _ptr(v),
                              master.size), f"mt_bind_layer({group})", ctx)


def mt_forward(ctx, tokens: np.ndarray, labels: np.ndarray, grad_scale: float, loss_out=None):
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    _check(_lib.mt_forward(ctx, _ptr(tokens), _ptr(labels), grad_scale, _ptr(loss_out)),
           "mt_forward", ctx)


def mt_backward(ctx, accumulate: int):
    _check(_lib.mt_backward(ctx, int(accumulate)), "mt_backward", ctx)


def mt_backward_step(ctx, accumulate: int, hp: mt_adamw_hparams, step: int):
    _check(_lib.mt_backward_step(ctx, int(accumulate), C.byref(hp), step), "mt_backward_step", ctx)


def mt_flush_grads(ctx):
    _check(_lib.mt_flush_grads(ctx), "mt_flush_grads", ctx)


def mt_sync_loss(ctx):
    _check(_lib.mt_sync_loss(ctx), "mt_sync_loss", ctx)


def mt_step_loss(ctx) -> float:
    out = C.c_float()
    _check(_lib.mt_step_loss(ctx, C.byref(out)), "mt_step_loss", ctx)
    return out.value


def mt_moe_routing(ctx, layer: int, tokens: int, top_k: int) -> np.ndarray:
    out = np.empty((tokens, top_k), np.int32)
    _check(_lib.mt_moe_routing(ctx, layer, _ptr(out)), "mt_moe_routing", ctx)
    return out


def mt_adamw_step(ctx, hp: mt_adamw_hparams, step: int):
    _check(_lib.mt_adamw_step(ctx, C.byref(hp), step), "mt_adamw_step", ctx)


def mt_get_stats(ctx) -> dict:
    s = mt_stats()
    _check(_lib.mt_get_stats(ctx, C.byref(s)), "mt_get_stats", ctx)
    return s.as_dict()


def mt_kernel_timing(ctx, enable: bool):
    _check(_lib.mt_kernel_timing(ctx, int(bool(enable))), "mt_kernel_timing", ctx)


def mt_get_kernel_times(ctx) -> list:
    """[{name, launches, ms, flop, bytes}] by descending device time."""
    n = _I32()
    buf = (mt_kernel_time * 64)()
    _check(_lib.mt_get_kernel_times(ctx, buf, 64, C.byref(n)), "mt_get_kernel_times", ctx)
    return [{"name": k.name.decode(), "launches": k.launches, "ms": k.ms, "flop": k.flop,
             "bytes": k.bytes} for k in buf[:min(n.value, 64)]]


def mt_last_error(ctx) -> str:
    return _lib.mt_last_error(ctx).decode()


def mt_destroy(ctx):
    _lib.mt_destroy(ctx)


def mt_host_cast_bf16(src: np.ndarray, dst: np.ndarray, threads: int = 0):
    _check(_lib.mt_host_cast_bf16(_ptr(src), _ptr(dst), src.size, threads), "mt_host_cast_bf16")


def mt_host_adamw(master, grad, m, v, bf16_out, hp: mt_adamw_hparams, step: int, threads: int = 0):
    _check(_lib.mt_host_adamw(_ptr(master), _ptr(grad), _ptr(m), _ptr(v), _ptr(bf16_out),
                              master.size, C.byref(hp), step, threads), "mt_host_adamw")


def mt_host_adamw_slab(master, grad, m, v, bf16_out, slab, accumulate: int,
                       hp: mt_adamw_hparams, step: int, threads: int = 0):
    """slab: uint16 (bf16 bits) or float32 array of master.size elements."""
    sb = 1 if slab.dtype == np.uint16 else 0
    _check(_lib.mt_host_adamw_slab(_ptr(master), _ptr(grad), _ptr(m), _ptr(v), _ptr(bf16_out),
                                   _ptr(slab), sb, int(accumulate), master.size, C.byref(hp), step,
                                   threads), "mt_host_adamw_slab")


def mt_host_accumulate(grad, src, accumulate: int, threads: int = 0):
    _check(_lib.mt_host_accumulate(_ptr(grad), _ptr(src), grad.size, accumulate, threads),
           "mt_host_accumulate")


def mt_host_triad(a, b, c, s: float, reps: int = 5, threads: int = 0) -> float:
    """Fastest of `reps` passes of a = b + s c (host float32 arrays), seconds."""
    t = C.c_double()
    _check(_lib.mt_host_triad(_ptr(a), _ptr(b), _ptr(c), s, a.size, reps, threads, C.byref(t)),
           "mt_host_triad")
    return t.value


def mt_host_rope_table(seq_len: int, head_dim: int, base: float):
    c = np.empty((seq_len, head_dim // 2), np.float32)
    s = np.empty_like(c)
    _check(_lib.mt_host_rope_table(seq_len, head_dim, base, _ptr(c), _ptr(s)), "mt_host_rope_table")
    return c, s


# -------------------------------------------------------- kernel entry points
def mtk_gemm(layout, epilogue, M, N, K, A, lda, B, ldb, Cm, ldc, R=None, ldr=0, gu=None, ldgu=0,
             ffn=0, stream=None, rope_cos=None, rope_sin=None, rope_cols=0, rope_seq=0,
             rope_dim=0, group_off=None, groups=0, group_stride_b=0, group_stride_c=0):
    a = mt_gemm_args(layout, epilogue, M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(Cm), ldc,
                     _ptr(R), ldr, _ptr(gu), ldgu, ffn, _ptr(rope_cos), _ptr(rope_sin), rope_cols,
                     rope_seq, rope_dim, _ptr(group_off), groups, 0, group_stride_b,
                     group_stride_c)
    _check(_lib.mtk_gemm(C.byref(a), _stream(stream)), "mtk_gemm")


def mtk_rmsnorm_fwd(x, g, out, rstd, T, h, eps, stream=None):
    _check(_lib.mtk_rmsnorm_fwd(_ptr(x), _ptr(g), _ptr(out), _ptr(rstd), T, h, eps,
                                _stream(stream)), "mtk_rmsnorm_fwd")


def mtk_rmsnorm_bwd_workspace(T, h) -> int:
    return _lib.mtk_rmsnorm_bwd_workspace(T, h)


def mtk_rmsnorm_bwd(dn, x, rstd, g, resid, dx, dx_bf16, dg, workspace, T, h, stream=None):
    _check(_lib.mtk_rmsnorm_bwd(_ptr(dn), _ptr(x), _ptr(rstd), _ptr(g), _ptr(resid), _ptr(dx),
                                _ptr(dx_bf16), _ptr(dg), _ptr(workspace), T, h, _stream(stream)),
           "mtk_rmsnorm_bwd")


def mtk_rmsnorm_bwd_noalloc(dn, x, rstd, g, resid, dx, dx_bf16, dg, T, h, stream=None):
    """mtk_rmsnorm_bwd on the library's fixed per-GPU scratch (no allocation)."""
    _check(_lib.mtk_rmsnorm_bwd_noalloc(_ptr(dn), _ptr(x), _ptr(rstd), _ptr(g), _ptr(resid),
                                        _ptr(dx), _ptr(dx_bf16), _ptr(dg), T, h, _stream(stream)),
           "mtk_rmsnorm_bwd_noalloc")


def mtk_noalloc_scratch_bytes() -> int:
    return _lib.mtk_noalloc_scratch_bytes()


def mtk_rope(qkv, T, seq_len, n_heads, n_kv_heads, head_dim, cos_t, sin_t, inverse, stream=None):
    _check(_lib.mtk_rope(_ptr(qkv), T, seq_len, n_heads, n_kv_heads, head_dim, _ptr(cos_t),
                         _ptr(sin_t), inverse, _stream(stream)), "mtk_rope")


def mtk_attention_fwd(qkv, o, lse, batch, seq_len, n_heads, n_kv_heads, head_dim, stream=None):
    _check(_lib.mtk_attention_fwd(_ptr(qkv), _ptr(o), _ptr(lse), batch, seq_len, n_heads,
                                  n_kv_heads, head_dim, _stream(stream)), "mtk_attention_fwd")


def mtk_attention_bwd_workspace(batch, seq_len, n_heads, n_kv_heads, head_dim) -> int:
    return _lib.mtk_attention_bwd_workspace(batch, seq_len, n_heads, n_kv_heads, head_dim)


def mtk_attention_bwd(qkv, o, dout, lse, workspace, dqkv, batch, seq_len, n_heads, n_kv_heads,
                      head_dim, stream=None):
    _check(_lib.mtk_attention_bwd(_ptr(qkv), _ptr(o), _ptr(dout), _ptr(lse), _ptr(workspace),
                                  _ptr(dqkv), batch, seq_len, n_heads, n_kv_heads, head_dim,
                                  _stream(stream)), "mtk_attention_bwd")


def mtk_attention_bwd_rope(qkv, o, dout, lse, workspace, dqkv, batch, seq_len, n_heads,
                           n_kv_heads, head_dim, cos_t, sin_t, stream=None):
    _check(_lib.mtk_attention_bwd_rope(_ptr(qkv), _ptr(o), _ptr(dout), _ptr(lse), _ptr(workspace),
                                       _ptr(dqkv), batch, seq_len, n_heads, n_kv_heads, head_dim,
                                       _ptr(cos_t), _ptr(sin_t), _stream(stream)),
           "mtk_attention_bwd_rope")


def mtk_cross_entropy(logits, ld, labels, T, V, grad_scale, n_valid, dlogits, ld_d, loss_rows,
                      loss_out, stream=None):
    _check(_lib.mtk_cross_entropy(_ptr(logits), ld, _ptr(labels), T, V, grad_scale, n_valid,
                                  _ptr(dlogits), ld_d, _ptr(loss_rows), _ptr(loss_out),
                                  _stream(stream)), "mtk_cross_entropy")


def mtk_mfma_peak(out, workgroups, iters, stream=None):
    _check(_lib.mtk_mfma_peak(_ptr(out), workgroups, iters, _stream(stream)), "mtk_mfma_peak")


def mtk_mfma_peak_chains() -> int:
    return _lib.mtk_mfma_peak_chains()


def mtk_copy(dst, src, nbytes, workgroups, stream=None):
    _check(_lib.mtk_copy(_ptr(dst), _ptr(src), nbytes, workgroups, _stream(stream)), "mtk_copy")


from .session import Session, aligned_zeros  # noqa: E402,F401
