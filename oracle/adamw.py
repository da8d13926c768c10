"""Host AdamW on fp32 master/grad/m/v (oracle).

Method: parameters, gradients and Adam moments live in host memory and the
optimizer step runs on the CPU where they are (zhichai D1; travelaiplan
核心功能 1; lqnn 二: ParameterState holds fp32 master, grad, m, v and the
step updates the in-memory master).  The pages name PyTorch AdamW semantics
(lqnn 二), so the step is decoupled-weight-decay Adam (reading O7):

  p <- p * (1 - lr*wd)
  m <- b1*m + (1-b1)*g
  v <- b2*v + (1-b2)*g^2
  p <- p - lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)

with t the 1-based step, defaults b1=0.9, b2=0.999, eps=1e-8, wd=0.01.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class AdamWHparams:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01


def adamw_step(p: np.ndarray, g: np.ndarray, m: np.ndarray, v: np.ndarray, step: int,
               hp: AdamWHparams) -> None:
    """In-place update of p, m, v (same dtype)."""
    assert step >= 1
    p *= 1.0 - hp.lr * hp.weight_decay
    m *= hp.beta1
    m += (1.0 - hp.beta1) * g
    v *= hp.beta2
    v += (1.0 - hp.beta2) * (g * g)
    mhat = m / (1.0 - hp.beta1 ** step)
    vhat = v / (1.0 - hp.beta2 ** step)
    p -= hp.lr * mhat / (np.sqrt(vhat) + hp.eps)
