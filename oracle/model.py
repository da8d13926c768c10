"""Decoder block, head and embedding: forward, analytic backward, and the
whole-model and streamed-with-recompute drivers.

Method being checked:
  * zhichai D2 / travelaiplan 核心功能 2: layers run one at a time on weights
    streamed in; each layer's gradients go back to host memory per layer.
  * zhichai D3 / lqnn 三.4: an activation checkpoint every K layers; backward
    re-runs the forward of each K-layer segment from its checkpoint.
  * zhichai D4 / travelaiplan 核心功能 3: a stateless layer template bound to
    host-supplied flat weights (here: views unpacked from a flat array).
Streaming and recompute move data, not math, so the streamed driver must give
the same numbers as the plain whole-model driver (bit-for-bit in this module).

Block (reading O1 -- pages call the layers "Llama Transformer layers", lqnn 四):
  n1 = RMSNorm(x) * g1                      r = 1/sqrt(mean_h(x^2) + eps)
  q, k, v = n1 Wq^T, n1 Wk^T, n1 Wv^T
  q, k <- RoPE (rotate-half pairs (i, i+d/2), theta_i = base^(-2i/d),
          angle = pos * theta_i in float64, pos restarting at every sequence)
  o_j = softmax(q_j k_g^T / sqrt(d) + causal mask) v_g,  g = j // (n_q / n_kv)
  h1 = x + concat(o) Wo^T
  n2 = RMSNorm(h1) * g2
  y  = h1 + (silu(n2 Wg^T) * (n2 Wu^T)) Wd^T,  silu(a) = a * sigmoid(a)
Head: xf = RMSNorm(x_L) * gf, logits = xf Wh^T,
  loss = mean over labelled positions of (logsumexp(logits_t) - logits_t[label_t]).
Embedding: x0 = E[token].

All functions take arrays of one floating dtype (float64 for self-checks,
float32 for parity runs) and keep it.  Activations are [T, features] with
T = batch * seq tokens in sequence-major order.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Tuple

import numpy as np

from . import layout as L


# ----------------------------------------------------------------- RMSNorm
def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float):
    """n = x * r * g with r = 1 / sqrt(mean(x^2) + eps) per row.  Returns (n, r[T,1])."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * g, r


def rmsnorm_bwd(dn: np.ndarray, x: np.ndarray, r: np.ndarray, g: np.ndarray):
    """Chain rule of rmsnorm.  xhat = x r;  dg = sum_t dn*xhat;
    dx = r * (dn*g - xhat * mean_h(dn*g*xhat))."""
    xhat = x * r
    dxhat = dn * g
    dg = np.sum(dn * xhat, axis=0)
    dx = r * (dxhat - xhat * np.mean(dxhat * xhat, axis=-1, keepdims=True))
    return dx, dg


# -------------------------------------------------------------------- RoPE
def rope_tables(seq_len: int, head_dim: int, base: float, dtype):
    """cos/sin [seq_len, head_dim/2]: angles pos*base^(-2i/d) formed in float64,
    then rounded to ``dtype`` (reading O3)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / head_dim)
    ang = np.arange(seq_len, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, inverse: bool = False):
    """Rotate pairs (i, i + d/2) of x [b, s, heads, d] by +angle (or -angle).
    (a, b) -> (a cos - b sin, b cos + a sin)."""
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    if inverse:
        s = -s
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# --------------------------------------------------------------- attention
def _scores(qh: np.ndarray, kh: np.ndarray, scale: float) -> np.ndarray:
    """Causal softmax probabilities P [s, s] for one head of one sequence."""
    s = qh.shape[0]
    S = (qh @ kh.T) * scale
    S = np.where(np.tril(np.ones((s, s), dtype=bool)), S, -np.inf)
    S = S - S.max(axis=1, keepdims=True)
    E = np.exp(S)
    return E / E.sum(axis=1, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Causal grouped-query softmax attention.  q [b,s,nq,d], k/v [b,s,nkv,d].
    Query head j reads KV head j // (nq/nkv) (reading O4)."""
    b, s, nq, d = q.shape
    nkv = k.shape[2]
    grp = nq // nkv
    scale = 1.0 / math.sqrt(d)
    o = np.empty_like(q)
    for bi in range(b):
        for j in range(nq):
            gk = j // grp
            P = _scores(q[bi, :, j], k[bi, :, gk], scale)
            o[bi, :, j] = P @ v[bi, :, gk]
    return o


def attention_rows(q, k, v, rows) -> np.ndarray:
    """Outputs of :func:`attention` for selected query positions only (each
    query row depends on keys 0..row).  q/k/v as in :func:`attention`;
    rows: 1-D positions.  Returns [b, len(rows), nq, d]."""
    b, s, nq, d = q.shape
    grp = nq // k.shape[2]
    scale = 1.0 / math.sqrt(d)
    out = np.empty((b, len(rows), nq, d), dtype=q.dtype)
    for bi in range(b):
        for j in range(nq):
            gk = j // grp
            for ri, t in enumerate(rows):
                sc = (k[bi, :t + 1, gk] @ q[bi, t, j]) * scale
                sc = sc - sc.max()
                e = np.exp(sc)
                out[bi, ri, j] = (e / e.sum()) @ v[bi, :t + 1, gk]
    return out


def attention_bwd(q, k, v, do):
    """Analytic backward of :func:`attention` (P recomputed from q, k).
    dP = dO v^T; dS = P * (dP - rowsum(P*dP)); dq = dS k/sqrt(d);
    dk = dS^T q/sqrt(d); dv = P^T dO.  dk, dv sum over the query heads of a group."""
    b, s, nq, d = q.shape
    nkv = k.shape[2]
    grp = nq // nkv
    scale = 1.0 / math.sqrt(d)
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for bi in range(b):
        for j in range(nq):
            gk = j // grp
            P = _scores(q[bi, :, j], k[bi, :, gk], scale)
            dP = do[bi, :, j] @ v[bi, :, gk].T
            dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
            dq[bi, :, j] = (dS @ k[bi, :, gk]) * scale
            dk[bi, :, gk] += (dS.T @ q[bi, :, j]) * scale
            dv[bi, :, gk] += P.T @ do[bi, :, j]
    return dq, dk, dv


def attention_lse(q, k) -> np.ndarray:
    """log-sum-exp of the scaled causal scores, [b, s, nq] (used to check the
    statistic a flash kernel saves for its backward)."""
    b, s, nq, d = q.shape
    grp = nq // k.shape[2]
    scale = 1.0 / math.sqrt(d)
    out = np.empty((b, s, nq), dtype=q.dtype)
    mask = np.tril(np.ones((s, s), dtype=bool))
    for bi in range(b):
        for j in range(nq):
            S = (q[bi, :, j] @ k[bi, :, j // grp].T) * scale
            S = np.where(mask, S, -np.inf)
            mx = S.max(axis=1, keepdims=True)
            out[bi, :, j] = (mx + np.log(np.exp(S - mx).sum(axis=1, keepdims=True)))[:, 0]
    return out


# ------------------------------------------------------------------ SwiGLU
def sigmoid(a):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def swiglu(a, u):
    return a * sigmoid(a) * u


def swiglu_bwd(dm, a, u):
    """da = dm*u*s*(1 + a*(1-s)), du = dm*a*s with s = sigmoid(a)."""
    s = sigmoid(a)
    return dm * u * s * (1.0 + a * (1.0 - s)), dm * a * s


# ------------------------------------------------------------------- block
def block_forward(W: Dict[str, np.ndarray], x: np.ndarray, cfg, cos, sin, batch: int,
                  sel=None):
    """One decoder block.  x [T, h] with T = batch * seq.  sel: an expert
    selection handed to a mixture-of-experts block (oracle.moe.route).
    Returns (y, cache)."""
    T, h = x.shape
    s = T // batch
    nq, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    n1, r1 = rmsnorm(x, W["attn_norm"], cfg.rms_eps)
    q = (n1 @ W["wq"].T).reshape(batch, s, nq, d)
    k = (n1 @ W["wk"].T).reshape(batch, s, nkv, d)
    v = (n1 @ W["wv"].T).reshape(batch, s, nkv, d)
    qr = rope(q, cos, sin)
    kr = rope(k, cos, sin)
    o = attention(qr, kr, v).reshape(T, nq * d)
    h1 = x + o @ W["wo"].T
    n2, r2 = rmsnorm(h1, W["mlp_norm"], cfg.rms_eps)
    cache = dict(x=x, n1=n1, r1=r1, qr=qr, kr=kr, v=v, o=o, h1=h1, n2=n2, r2=r2)
    if "w_router" in W:  # a mixture-of-experts block (oracle.moe)
        from . import moe
        f, cache["moe"] = moe.ffn_forward(W, n2, cfg, sel)
        return h1 + f, cache
    a = n2 @ W["w_gate"].T
    u = n2 @ W["w_up"].T
    m = swiglu(a, u)
    y = h1 + m @ W["w_down"].T
    cache.update(a=a, u=u, m=m)
    return y, cache


def block_backward(W: Dict[str, np.ndarray], c: Dict[str, np.ndarray], dy: np.ndarray,
                   cfg, cos, sin, batch: int):
    """Analytic backward of :func:`block_forward`.  Returns (dx, grads by name)."""
    T, h = dy.shape
    s = T // batch
    nq, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    g: Dict[str, np.ndarray] = {}
    if "w_router" in W:
        from . import moe
        dn2, gm = moe.ffn_backward(W, c["moe"], dy, cfg)
        g.update(gm)
    else:
        g["w_down"] = dy.T @ c["m"]
        dm = dy @ W["w_down"]
        da, du = swiglu_bwd(dm, c["a"], c["u"])
        g["w_gate"] = da.T @ c["n2"]
        g["w_up"] = du.T @ c["n2"]
        dn2 = da @ W["w_gate"] + du @ W["w_up"]
    dh1n, g["mlp_norm"] = rmsnorm_bwd(dn2, c["h1"], c["r2"], W["mlp_norm"])
    dh1 = dy + dh1n
    g["wo"] = dh1.T @ c["o"]
    do = (dh1 @ W["wo"]).reshape(batch, s, nq, d)
    dqr, dkr, dv = attention_bwd(c["qr"], c["kr"], c["v"], do)
    dq = rope(dqr, cos, sin, inverse=True).reshape(T, nq * d)
    dk = rope(dkr, cos, sin, inverse=True).reshape(T, nkv * d)
    dv = dv.reshape(T, nkv * d)
    g["wq"] = dq.T @ c["n1"]
    g["wk"] = dk.T @ c["n1"]
    g["wv"] = dv.T @ c["n1"]
    dn1 = dq @ W["wq"] + dk @ W["wk"] + dv @ W["wv"]
    dxn, g["attn_norm"] = rmsnorm_bwd(dn1, c["x"], c["r1"], W["attn_norm"])
    return dh1 + dxn, g


# -------------------------------------------------------------------- head
def cross_entropy(logits: np.ndarray, labels: np.ndarray, grad_scale: float):
    """Mean next-token cross-entropy over labelled rows (label < 0 ignored) and
    its gradient (softmax - onehot) * grad_scale / n_labelled (reading O5).
    With no labelled row the loss and gradient are 0."""
    T, V = logits.shape
    valid = labels >= 0
    n = int(valid.sum())
    mx = logits.max(axis=1, keepdims=True)
    lse = mx + np.log(np.exp(logits - mx).sum(axis=1, keepdims=True))
    idx = np.nonzero(valid)[0]
    if n == 0:
        return logits.dtype.type(0.0), np.zeros_like(logits), lse[:, 0]
    per = lse[idx, 0] - logits[idx, labels[idx]]
    loss = per.sum() / n
    dl = np.exp(logits - lse)
    dl[idx, labels[idx]] -= 1.0
    dl[~valid] = 0.0
    dl *= grad_scale / n
    return loss, dl, lse[:, 0]


def head_forward_backward(Wh: Dict[str, np.ndarray], xL: np.ndarray, labels: np.ndarray,
                          grad_scale: float, eps: float):
    """Final RMSNorm, LM head, loss and their backward.  Returns (loss, dxL, grads)."""
    xf, rf = rmsnorm(xL, Wh["final_norm"], eps)
    logits = xf @ Wh["w_head"].T
    loss, dl, _ = cross_entropy(logits, labels, grad_scale)
    g = {"w_head": dl.T @ xf}
    dxf = dl @ Wh["w_head"]
    dxL, g["final_norm"] = rmsnorm_bwd(dxf, xL, rf, Wh["final_norm"])
    return loss, dxL, g


# --------------------------------------------------------------- embedding
def embed(E: np.ndarray, tokens: np.ndarray) -> np.ndarray:
    return E[tokens.reshape(-1)]


def embed_bwd(dx0: np.ndarray, tokens: np.ndarray, vocab: int) -> np.ndarray:
    """dE[tok[t]] += dx0[t] in token order; rows never seen stay exactly 0 (O12)."""
    dE = np.zeros((vocab, dx0.shape[1]), dtype=dx0.dtype)
    np.add.at(dE, tokens.reshape(-1), dx0)
    return dE


# ------------------------------------------------------------------ drivers
def _tables(cfg, dtype):
    return rope_tables(cfg.seq_len, cfg.head_dim, cfg.rope_base, dtype)


def forward_backward_whole(params: Dict[int, Dict[str, np.ndarray]], tokens: np.ndarray,
                           labels: np.ndarray, cfg, grad_scale: float, routing=None):
    """Plain model: keep every layer's activations, then backward.
    params {group: {name: array}}; tokens/labels [b, s]; routing: optional
    {layer: expert selection} for mixture-of-experts blocks.  Returns (loss,
    grads {group: {name: array}})."""
    routing = routing or {}
    dtype = params[L.EMBED]["emb"].dtype
    cos, sin = _tables(cfg, dtype)
    b = tokens.shape[0]
    x = embed(params[L.EMBED]["emb"], tokens)
    caches = []
    for l in range(cfg.n_layers):
        x, c = block_forward(params[l], x, cfg, cos, sin, b, routing.get(l))
        caches.append(c)
    loss, dy, gh = head_forward_backward(params[L.HEAD], x, labels.reshape(-1), grad_scale,
                                         cfg.rms_eps)
    grads = {L.HEAD: gh}
    for l in reversed(range(cfg.n_layers)):
        dy, grads[l] = block_backward(params[l], caches[l], dy, cfg, cos, sin, b)
    grads[L.EMBED] = {"emb": embed_bwd(dy, tokens, cfg.vocab)}
    return loss, grads


def forward_backward_streamed(flats: Dict[int, np.ndarray], tokens: np.ndarray,
                              labels: np.ndarray, cfg, grad_scale: float, K: int,
                              grad_flats: Dict[int, np.ndarray], accumulate: bool,
                              stats: Optional[dict] = None, routing=None, progress=None):
    """Streamed execution with segment recompute.

    flats: {group: flat array} holding the weights (lqnn 三.1).  Forward keeps
    only the input of every K-th layer (lqnn 三.4).  Backward walks segments
    last-to-first, re-runs the segment's forwards from its checkpoint, then
    runs the segment's layers backwards; each layer's gradient is packed into a
    flat array and written (accumulate=False) or added (accumulate=True) into
    ``grad_flats[group]`` -- the host gradient of lqnn 二 / 三.3.
    routing: optional {layer: expert selection} for mixture-of-experts blocks.
    progress: optional callable taking a short message after each layer (for
    long runs; it sees no values).
    Returns the micro-batch loss.
    """
    routing = routing or {}
    say = progress or (lambda msg: None)
    dtype = flats[L.EMBED].dtype
    cos, sin = _tables(cfg, dtype)
    b = tokens.shape[0]
    nL = cfg.n_layers
    ckpt: List[np.ndarray] = []
    x = embed(L.unpack(cfg, L.EMBED, flats[L.EMBED])["emb"], tokens)
    for l in range(nL):
        if l % K == 0:
            ckpt.append(x)
        x, _ = block_forward(L.unpack(cfg, l, flats[l]), x, cfg, cos, sin, b, routing.get(l))
        say(f"forward layer {l}")
    loss, dy, gh = head_forward_backward(L.unpack(cfg, L.HEAD, flats[L.HEAD]), x,
                                         labels.reshape(-1), grad_scale, cfg.rms_eps)
    say("head")

    def land(group, gdict):
        gf = L.pack(cfg, group, gdict, dtype=dtype)
        if accumulate:
            grad_flats[group] += gf
        else:
            grad_flats[group][...] = gf

    land(L.HEAD, gh)
    recomputed = 0
    for seg in reversed(range(len(ckpt))):
        lo, hi = seg * K, min(nL, seg * K + K)
        x = ckpt[seg]
        window = []
        for l in range(lo, hi):
            x, c = block_forward(L.unpack(cfg, l, flats[l]), x, cfg, cos, sin, b, routing.get(l))
            window.append(c)
            recomputed += 1
            say(f"recompute layer {l}")
        for l in reversed(range(lo, hi)):
            dy, gl = block_backward(L.unpack(cfg, l, flats[l]), window[l - lo], dy, cfg, cos,
                                    sin, b)
            land(l, gl)
            say(f"backward layer {l}")
    land(L.EMBED, {"emb": embed_bwd(dy, tokens, cfg.vocab)})
    if stats is not None:
        stats["recomputed_layers"] = recomputed
        stats["checkpoints"] = len(ckpt)
    return loss
