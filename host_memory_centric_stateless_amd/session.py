"""A training session: host state, device arena and one libmt context.

Plumbing only.  Host state (fp32 master / grad / Adam m / v per group) is
plain numpy memory owned here; the device arena and the three streams are
torch allocations handed to libmt; every step runs inside libmt.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, Iterable, Optional, Tuple

import numpy as np
import torch

from . import (MT_GROUP_EMBED, MT_GROUP_HEAD, default_drain_workgroups, make_config, mt_adamw_hparams, mt_adamw_step,
               mt_backward, mt_backward_step, mt_bind_layer, mt_create, mt_destroy, mt_device_arena,
               mt_device_requirements, mt_flush_grads, mt_forward, mt_get_stats, mt_layout,
               mt_step_loss, mt_sync_loss)


def aligned_zeros(n: int, align: int = 64) -> np.ndarray:
    """fp32 zeros whose data pointer is `align`-byte aligned."""
    raw = np.zeros(n + align // 4, dtype=np.float32)
    off = (-raw.ctypes.data % align) // 4
    return raw[off:off + n]


class Session:
    def __init__(self, cfg, host_threads: int = 0, device: str = "cuda:0",
                 ckpt_interval: Optional[int] = None, n_grad_slabs: Optional[int] = None,
                 slab_bf16: bool = True, drain_workgroups: Optional[int] = None,
                 micro_batches_per_pass: int = 1, host_from: Optional["Session"] = None,
                 head_token_chunk: int = 0):
        """host_from: use that session's host fp32 state (same model shape)
        instead of allocating a new one; call bind() before the first step."""
        if ckpt_interval is not None:
            cfg = cfg.replace(ckpt_interval=ckpt_interval)
        if n_grad_slabs is not None:
            cfg = cfg.replace(n_grad_slabs=n_grad_slabs)
        self.cfg = cfg
        self.c = make_config(cfg, host_threads, slab_bf16,
                             default_drain_workgroups(cfg, slab_bf16, micro_batches_per_pass)
                             if drain_workgroups is None
                             else drain_workgroups, micro_batches_per_pass, head_token_chunk)
        self.mb_per_pass = micro_batches_per_pass
        self.req = mt_device_requirements(self.c)
        self.groups = [MT_GROUP_EMBED] + list(range(cfg.n_layers)) + [MT_GROUP_HEAD]
        self.layout: Dict[int, Tuple[list, int]] = {g: mt_layout(self.c, g) for g in self.groups}
        if host_from is not None:
            if {g: host_from.layout[g][1] for g in self.groups} != \
                    {g: self.layout[g][1] for g in self.groups}:
                raise ValueError("host_from has a different model shape")
            self.master, self.grad = host_from.master, host_from.grad
            self.m, self.v = host_from.m, host_from.v
        else:
            self.master, self.grad, self.m, self.v = {}, {}, {}, {}
            for g in self.groups:
                n = self.layout[g][1]
                self.master[g] = aligned_zeros(n)
                self.grad[g] = aligned_zeros(n)
                self.m[g] = aligned_zeros(n)
                self.v[g] = aligned_zeros(n)

        self.device = torch.device(device)
        r = self.req

        def dev(nbytes):
            return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=self.device)

        self.wbuf = [dev(r.weight_buf) for _ in range(2)]
        self.slabs = [dev(r.grad_slab) for _ in range(cfg.n_grad_slabs)]
        self.window = dev(r.window)
        self.ckpt = dev(r.checkpoints)
        self.ws = dev(r.workspace)
        self.streams = [torch.cuda.Stream(device=self.device) for _ in range(3)]
        a = mt_device_arena()
        a.weight_buf[0] = self.wbuf[0].data_ptr()
        a.weight_buf[1] = self.wbuf[1].data_ptr()
        for i, s in enumerate(self.slabs):
            a.grad_slab[i] = s.data_ptr()
        a.window = self.window.data_ptr()
        a.checkpoints = self.ckpt.data_ptr()
        a.workspace = self.ws.data_ptr()
        a.stream_prefetch = self.streams[0].cuda_stream
        a.stream_compute = self.streams[1].cuda_stream
        a.stream_offload = self.streams[2].cuda_stream
        a.weight_buf_bytes = self.wbuf[0].numel()
        a.grad_slab_bytes = self.slabs[0].numel()
        a.window_bytes = self.window.numel()
        a.checkpoints_bytes = self.ckpt.numel()
        a.workspace_bytes = self.ws.numel()
        self.arena = a
        with torch.cuda.device(self.device):
            self.ctx = mt_create(self.c, a)
        self.bound = False

    # ------------------------------------------------------------ weights
    def views(self, group: int, which: str = "master") -> Dict[str, np.ndarray]:
        flat = getattr(self, which)[group]
        return {name: flat[off:off + n].reshape(rows, cols) if rows > 1 else flat[off:off + n]
                for name, off, n, rows, cols in self.layout[group][0]}

    def load_weights(self, stream: Iterable) -> None:
        """Copy (group, name, array) tuples into the fp32 masters, then bind."""
        vs = {g: self.views(g) for g in self.groups}
        for g, name, arr in stream:
            vs[g][name][...] = np.asarray(arr, dtype=np.float32).reshape(vs[g][name].shape)
        self.bind()

    def bind(self) -> None:
        with torch.cuda.device(self.device):
            for g in self.groups:
                mt_bind_layer(self.ctx, g, self.master[g], self.grad[g], self.m[g], self.v[g])
        self.bound = True

    # --------------------------------------------------------------- steps
    def forward_backward(self, tokens: np.ndarray, labels: np.ndarray) -> float:
        """All micro-batches of one step (tokens/labels [acc, b, s]); grads
        land in self.grad.  Returns the mean micro-batch loss."""
        acc = tokens.shape[0]
        npass, tok, lab = self._passes(tokens, labels)
        losses = np.zeros(npass, dtype=np.float32)
        with torch.cuda.device(self.device):
            for k in range(npass):
                out = losses[k:k + 1]
                mt_forward(self.ctx, tok[k], lab[k], 1.0 / acc, out)
                mt_backward(self.ctx, 1 if k > 0 else 0)
            mt_flush_grads(self.ctx)
            loss = mt_step_loss(self.ctx)
        self._losses = losses  # keep the output buffer alive until flush wrote it
        return loss

    def _passes(self, tokens: np.ndarray, labels: np.ndarray):
        """[acc, b, s] micro-batches -> passes of mb_per_pass micro-batches,
        each a contiguous int32 array (micro-batch-major)."""
        acc, n = tokens.shape[0], self.mb_per_pass
        if acc % n:
            raise ValueError(f"{acc} micro-batches do not split into passes of {n}")
        tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(acc // n, -1)
        lab = np.ascontiguousarray(labels, dtype=np.int32).reshape(acc // n, -1)
        return acc // n, tok, lab

    def step(self, tokens: np.ndarray, labels: np.ndarray, step: int, lr: Optional[float] = None,
             weight_decay: float = 0.01, overlap_optimizer: bool = True, flush: bool = True) -> float:
        """One optimizer step.  overlap_optimizer: run each group's AdamW on
        the CPU worker as soon as its gradient of the last micro-batch is in
        (mt_backward_step) instead of after the flush (mt_adamw_step).
        flush=False (overlapped optimizer only): return once the step's loss
        is known, leaving the host updates of this step to finish under the
        next step's forward; call flush() before reading grads or weights."""
        hp = mt_adamw_hparams(lr if lr is not None else self.cfg.lr, 0.9, 0.999, 1e-8, weight_decay)
        if not overlap_optimizer:
            loss = self.forward_backward(tokens, labels)
            mt_adamw_step(self.ctx, hp, step)
            return loss
        acc = tokens.shape[0]
        npass, tok, lab = self._passes(tokens, labels)
        losses = np.zeros(npass, dtype=np.float32)
        with torch.cuda.device(self.device):
            for k in range(npass):
                mt_forward(self.ctx, tok[k], lab[k], 1.0 / acc, losses[k:k + 1])
                if k + 1 < npass:
                    mt_backward(self.ctx, 1 if k > 0 else 0)
                else:
                    mt_backward_step(self.ctx, 1 if k > 0 else 0, hp, step)
            if flush:
                mt_flush_grads(self.ctx)
            else:
                mt_sync_loss(self.ctx)
            loss = mt_step_loss(self.ctx)
        self._losses = losses
        return loss

    def flush(self) -> None:
        """Wait for every gradient drain, host accumulation and update."""
        with torch.cuda.device(self.device):
            mt_flush_grads(self.ctx)

    def stats(self) -> dict:
        return mt_get_stats(self.ctx)

    def close(self) -> None:
        if getattr(self, "ctx", None):
            mt_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
