"""One optimizer step of the streamed method (oracle driver).

Per step: for each of the ``grad_accum`` micro-batches run the streamed
forward/backward (gradient written on the first micro-batch, added after it),
then AdamW on every group (lqnn 二, 三.3; travelaiplan 核心功能 1-2).  The
loss gradient of each micro-batch is scaled by 1/grad_accum (reading O5), so
the host gradient is the mean over micro-batches.  The reported step loss is
the mean of the micro-batch losses.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from . import layout as L
from .adamw import AdamWHparams, adamw_step
from .model import forward_backward_streamed, forward_backward_whole


class HostState:
    """fp32 (or fp64) master / grad / m / v flat arrays per group."""

    def __init__(self, cfg, dtype=np.float32):
        self.cfg = cfg
        self.dtype = dtype
        self.groups: List[int] = [L.EMBED] + list(range(cfg.n_layers)) + [L.HEAD]
        self.master: Dict[int, np.ndarray] = {}
        self.grad: Dict[int, np.ndarray] = {}
        self.m: Dict[int, np.ndarray] = {}
        self.v: Dict[int, np.ndarray] = {}
        for g in self.groups:
            n = L.group_layout(cfg, g)[1]
            self.master[g] = np.zeros(n, dtype)
            self.grad[g] = np.zeros(n, dtype)
            self.m[g] = np.zeros(n, dtype)
            self.v[g] = np.zeros(n, dtype)

    def load_weights(self, stream) -> None:
        """Fill masters from an iterator of (group, name, array)."""
        views = {g: L.unpack(self.cfg, g, self.master[g]) for g in self.groups}
        for g, name, arr in stream:
            views[g][name][...] = arr

    def params(self) -> Dict[int, Dict[str, np.ndarray]]:
        return {g: L.unpack(self.cfg, g, self.master[g]) for g in self.groups}


def train_step(st: HostState, tokens: np.ndarray, labels: np.ndarray, step: int,
               hp: Optional[AdamWHparams] = None, K: Optional[int] = None,
               mode: str = "streamed", routing=None) -> float:
    """tokens/labels [acc, b, s].  Updates st in place; returns the step loss.
    routing: optional [acc] list of {layer: expert selection} for
    mixture-of-experts blocks (see oracle.moe.route)."""
    cfg = st.cfg
    hp = hp or AdamWHparams(lr=cfg.lr)
    K = K or cfg.ckpt_interval
    acc = tokens.shape[0]
    scale = 1.0 / acc
    losses = []
    for mb in range(acc):
        if mode == "streamed":
            loss = forward_backward_streamed(st.master, tokens[mb], labels[mb], cfg, scale, K,
                                             st.grad, accumulate=mb > 0,
                                             routing=routing[mb] if routing else None)
        elif mode == "whole":
            loss, grads = forward_backward_whole(st.params(), tokens[mb], labels[mb], cfg, scale,
                                                 routing=routing[mb] if routing else None)
            for g in st.groups:
                gf = L.pack(cfg, g, grads[g], dtype=st.dtype)
                if mb == 0:
                    st.grad[g][...] = gf
                else:
                    st.grad[g] += gf
        else:
            raise ValueError(mode)
        losses.append(float(loss))
    for g in st.groups:
        adamw_step(st.master[g], st.grad[g], st.m[g], st.v[g], step, hp)
    return float(np.mean(losses))
