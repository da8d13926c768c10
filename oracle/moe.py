"""Mixture-of-experts feed-forward: the second parameter-structure group.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Method: the layers of a model are grouped by parameter structure and each
group gets its own stateless template and flat buffers; hybrid-attention and
mixture-of-experts layers form their own groups (m.lqnn.cn MegaTrain article,
四).  The pages give no formula for the MoE layer; the oracle takes the plain
sparse-MoE reading (readings M1-M4 below) and writes it out.

A block whose FFN is a mixture of experts replaces

    y = h1 + SwiGLU(n2)        by        y = h1 + sum_j g_j(t) E_{e_j(t)}(n2_t)

with, per token t:

* M1 router: r = n2 W_router^T (no bias), one logit per expert;
* M2 selection: e_1..e_k = the k experts with the largest router logits, ties
  to the lower expert index.  The choice is an integer decided by floating
  point, so it is taken in the precision of the kernels (bf16 operands,
  accumulated exactly here): the logits used for the decision are computed
  from the bf16-rounded n2 and W_router;
* M3 gates: g = softmax over the k selected logits (of the exact r); the
  selection itself has zero derivative;
* M4 experts: E_e(x) = (silu(x Wg_e^T) * (x Wu_e^T)) Wd_e^T, each a SwiGLU of
  width F_e; no capacity limit, no dropped tokens, no auxiliary loss.

Backward (chain rule): with o_j = E_{e_j}(n2_t) and dy the block-output
gradient, dg_j = <dy, o_j>; the expert sees dy * g_j; the softmax gives
dr_{e_j} = g_j (dg_j - sum_i g_i dg_i) (0 for experts not selected); then
dW_router = dr^T n2 and dn2 = sum_j dE_{e_j}/dx + dr W_router.
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np
import torch

from .model import swiglu, swiglu_bwd


def _bf16(a: np.ndarray) -> np.ndarray:
    """Round to bf16 (round to nearest even), returned in a's dtype."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy().astype(a.dtype)


def expert_weights(W: Dict[str, np.ndarray], e: int, h: int, Fe: int):
    """Views of expert e's gate [Fe, h], up [Fe, h] and down [h, Fe] matrices."""
    gu = W["w_gu"][e * 2 * Fe:(e + 1) * 2 * Fe]
    return gu[:Fe], gu[Fe:], W["w_down"][e * h:(e + 1) * h]


def route(n2: np.ndarray, w_router: np.ndarray, k: int, sel=None):
    """Router logits r [T, E], selected experts sel [T, k] (M2) and gates g [T, k] (M3).
    sel: a selection taken elsewhere (a parity run hands in the one the
    kernels took, which may differ from this one only at near-ties: the
    selection is a discontinuous function of the logits)."""
    r = n2 @ w_router.T
    if sel is None:
        sel = decide(n2, w_router, k)
    sel = np.asarray(sel)
    sl = np.take_along_axis(r, sel, axis=1)
    z = np.exp(sl - sl.max(axis=1, keepdims=True))
    g = z / z.sum(axis=1, keepdims=True)
    return r, sel, g


def decide(n2: np.ndarray, w_router: np.ndarray, k: int) -> np.ndarray:
    """The k largest router logits per token, ties to the lower index, decided
    on bf16-rounded operands (M2)."""
    dec = _bf16(n2).astype(np.float64) @ _bf16(w_router).astype(np.float64).T
    return np.argsort(-dec, axis=1, kind="stable")[:, :k]


def ffn_forward(W: Dict[str, np.ndarray], n2: np.ndarray, cfg, sel=None) -> Tuple[np.ndarray, dict]:
    """sum_j g_j E_{e_j}(n2) for every token (sel: see :func:`route`).
    Returns (f [T, h], cache)."""
    T, h = n2.shape
    E, k, Fe = cfg.n_experts, cfg.top_k, cfg.expert_ffn
    r, sel, g = route(n2, W["w_router"], k, sel)
    f = np.zeros_like(n2)
    per = []
    for e in range(E):
        tok, slot = np.nonzero(sel == e)      # tokens routed to e, in token order
        wg, wu, wd = expert_weights(W, e, h, Fe)
        x = n2[tok]
        a = x @ wg.T
        u = x @ wu.T
        m = swiglu(a, u)
        o = m @ wd.T
        f[tok] += g[tok, slot][:, None] * o
        per.append(dict(tok=tok, slot=slot, x=x, a=a, u=u, m=m, o=o))
    return f, dict(n2=n2, r=r, sel=sel, g=g, per=per)


def ffn_backward(W: Dict[str, np.ndarray], c: dict, df: np.ndarray, cfg):
    """Backward of :func:`ffn_forward` for df = dL/df.  Returns (dn2, grads)."""
    T, h = df.shape
    E, Fe = cfg.n_experts, cfg.expert_ffn
    n2, sel, g = c["n2"], c["sel"], c["g"]
    dn2 = np.zeros_like(n2)
    dg = np.zeros_like(g)
    g_gu = np.zeros_like(W["w_gu"])
    g_down = np.zeros_like(W["w_down"])
    for e in range(E):
        p = c["per"][e]
        tok, slot = p["tok"], p["slot"]
        wg, wu, wd = expert_weights(W, e, h, Fe)
        dg[tok, slot] = np.sum(df[tok] * p["o"], axis=1)
        do = g[tok, slot][:, None] * df[tok]
        g_down[e * h:(e + 1) * h] = do.T @ p["m"]
        dm = do @ wd
        da, du = swiglu_bwd(dm, p["a"], p["u"])
        g_gu[e * 2 * Fe:e * 2 * Fe + Fe] = da.T @ p["x"]
        g_gu[e * 2 * Fe + Fe:(e + 1) * 2 * Fe] = du.T @ p["x"]
        dn2[tok] += da @ wg + du @ wu
    dsl = g * (dg - np.sum(g * dg, axis=1, keepdims=True))
    dr = np.zeros((T, E), dtype=n2.dtype)
    np.put_along_axis(dr, sel, dsl, axis=1)
    grads = {"w_router": dr.T @ n2, "w_gu": g_gu, "w_down": g_down}
    dn2 += dr @ W["w_router"]
    return dn2, grads
