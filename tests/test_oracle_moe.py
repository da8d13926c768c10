"""Pins of the oracle's mixture-of-experts block (oracle/moe.py) against
things other than itself:

* finite differences in float64: a directional derivative over every
  parameter of a tiny model whose second block is an MoE, and per element for
  every MoE tensor;
* torch.autograd in float64 on the same definition, written with torch ops;
* closed forms: with all experts equal the MoE equals the dense SwiGLU of that
  expert (gates sum to one) and the router gradient vanishes; with top_k = E
  it is the softmax-gated mixture of all experts; a per-token brute force of
  the routing and combine on tiny inputs;
* the streamed driver with recompute equals the whole-model driver bit for
  bit on a model with both structure groups.
"""
import math

import numpy as np
import pytest
import torch

from oracle import layout as L
from oracle import model as M
from oracle import moe as MOE
from oracle.train import HostState
from synth_inputs import FD_TINY_MOE, MOE_PRESETS, make_batch, tensor_specs, weight_stream


def _params(cfg, seed, std=0.5):
    rng = np.random.default_rng(seed)
    P = {}
    for g in [L.EMBED] + list(range(cfg.n_layers)) + [L.HEAD]:
        P[g] = {}
        for name, shape, kind in tensor_specs(cfg, g):
            P[g][name] = (1.0 + 0.3 * rng.standard_normal(shape)) if kind == "gain" \
                else std * rng.standard_normal(shape)
    return P


def _batch(cfg, seed):
    rng = np.random.default_rng(seed)
    tok = rng.integers(0, cfg.vocab, size=(cfg.micro_batch, cfg.seq_len)).astype(np.int64)
    lab = np.full_like(tok, -1)
    lab[:, :-1] = tok[:, 1:]
    return tok, lab


def _loss(P, tok, lab, cfg):
    return float(M.forward_backward_whole(P, tok, lab, cfg, 1.0)[0])


def test_moe_block_present():
    cfg = FD_TINY_MOE
    assert not cfg.is_moe(0) and cfg.is_moe(1)
    names = [n for n, _ in L.group_shapes(cfg, 1)]
    assert "w_router" in names and "w_gate" not in names


def test_fd_directional_all_params_with_moe():
    cfg = FD_TINY_MOE
    P = _params(cfg, 21)
    tok, lab = _batch(cfg, 22)
    _, G = M.forward_backward_whole(P, tok, lab, cfg, 1.0)
    rng = np.random.default_rng(23)
    U = {g: {n: rng.standard_normal(a.shape) for n, a in d.items()} for g, d in P.items()}
    analytic = sum(float(np.sum(G[g][n] * U[g][n])) for g in P for n in P[g])
    h = 1e-6
    shift = lambda s: {g: {n: P[g][n] + s * h * U[g][n] for n in P[g]} for g in P}
    fd = (_loss(shift(+1), tok, lab, cfg) - _loss(shift(-1), tok, lab, cfg)) / (2 * h)
    assert abs(fd - analytic) <= 1e-6 * abs(analytic), (fd, analytic)


@pytest.mark.parametrize("name", ["w_router", "w_gu", "w_down", "mlp_norm", "wq"])
def test_fd_per_element_moe_tensors(name):
    cfg = FD_TINY_MOE
    P = _params(cfg, 24)
    tok, lab = _batch(cfg, 25)
    _, G = M.forward_backward_whole(P, tok, lab, cfg, 1.0)
    rng = np.random.default_rng(26)
    a = P[1][name]
    idx = [tuple(rng.integers(0, s) for s in a.shape) for _ in range(6)]
    h = 1e-6
    for i in idx:
        old = a[i]
        a[i] = old + h
        lp = _loss(P, tok, lab, cfg)
        a[i] = old - h
        lm = _loss(P, tok, lab, cfg)
        a[i] = old
        fd = (lp - lm) / (2 * h)
        an = G[1][name][i]
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3), (name, i, fd, an)


def _torch_moe_loss(P, tok, lab, cfg):
    """The model written with torch ops (float64), MoE blocks included, with
    the expert choice taken on bf16-rounded operands as the oracle reads it."""
    T = {g: {n: torch.tensor(a, dtype=torch.float64, requires_grad=True) for n, a in d.items()}
         for g, d in P.items()}
    b, s = tok.shape
    nq, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    h, E, k, Fe = cfg.hidden, cfg.n_experts, cfg.top_k, cfg.expert_ffn
    rms = lambda x, w: x * torch.rsqrt((x * x).mean(-1, keepdim=True) + cfg.rms_eps) * w
    i = torch.arange(d // 2, dtype=torch.float64)
    ang = torch.arange(s, dtype=torch.float64)[:, None] * (cfg.rope_base ** (-2 * i / d))[None]
    cos, sin = torch.cos(ang)[None, :, None, :], torch.sin(ang)[None, :, None, :]

    def rot(x):
        x1, x2 = x[..., : d // 2], x[..., d // 2:]
        return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], -1)

    x = T[L.EMBED]["emb"][torch.tensor(tok.reshape(-1))]
    mask = torch.tril(torch.ones(s, s, dtype=torch.bool))
    for l in range(cfg.n_layers):
        W = T[l]
        n1 = rms(x, W["attn_norm"])
        q = rot((n1 @ W["wq"].T).view(b, s, nq, d)).permute(0, 2, 1, 3)
        kk = rot((n1 @ W["wk"].T).view(b, s, nkv, d)).permute(0, 2, 1, 3)
        v = (n1 @ W["wv"].T).view(b, s, nkv, d).permute(0, 2, 1, 3)
        kk = kk.repeat_interleave(nq // nkv, dim=1)
        v = v.repeat_interleave(nq // nkv, dim=1)
        S = ((q @ kk.transpose(-1, -2)) / math.sqrt(d)).masked_fill(~mask, float("-inf"))
        o = (torch.softmax(S, -1) @ v).permute(0, 2, 1, 3).reshape(b * s, nq * d)
        h1 = x + o @ W["wo"].T
        n2 = rms(h1, W["mlp_norm"])
        if cfg.is_moe(l):
            r = n2 @ W["w_router"].T
            with torch.no_grad():
                rb = n2.to(torch.bfloat16).double() @ W["w_router"].to(torch.bfloat16).double().T
                order = torch.tensor(np.argsort(-rb.numpy(), axis=1, kind="stable")[:, :k])
            gate = torch.softmax(torch.gather(r, 1, order), dim=1)
            f = torch.zeros_like(n2)
            for e in range(E):
                wg = W["w_gu"][e * 2 * Fe:e * 2 * Fe + Fe]
                wu = W["w_gu"][e * 2 * Fe + Fe:(e + 1) * 2 * Fe]
                wd = W["w_down"][e * h:(e + 1) * h]
                out = (torch.nn.functional.silu(n2 @ wg.T) * (n2 @ wu.T)) @ wd.T
                ge = (gate * (order == e)).sum(1, keepdim=True)
                f = f + ge * out
            x = h1 + f
        else:
            x = h1 + (torch.nn.functional.silu(n2 @ W["w_gate"].T) * (n2 @ W["w_up"].T)) @ W["w_down"].T
    logits = rms(x, T[L.HEAD]["final_norm"]) @ T[L.HEAD]["w_head"].T
    loss = torch.nn.functional.cross_entropy(logits, torch.tensor(lab.reshape(-1)), ignore_index=-1)
    loss.backward()
    return float(loss.detach()), {g: {n: t.grad.numpy() for n, t in d.items()} for g, d in T.items()}


def test_moe_matches_torch_autograd_float64():
    cfg = FD_TINY_MOE
    P = _params(cfg, 27)
    tok, lab = _batch(cfg, 28)
    loss, G = M.forward_backward_whole(P, tok, lab, cfg, 1.0)
    tl, TG = _torch_moe_loss(P, tok, lab, cfg)
    assert abs(loss - tl) <= 1e-12 * abs(tl)
    for g in P:
        for n in P[g]:
            err = np.max(np.abs(G[g][n] - TG[g][n]))
            assert err <= 1e-10 * max(1.0, np.max(np.abs(TG[g][n]))), (g, n, err)


def _moe_weights(cfg, rng, equal=False):
    h, E, Fe = cfg.hidden, cfg.n_experts, cfg.expert_ffn
    one = [rng.standard_normal((2 * Fe, h)) * 0.3, rng.standard_normal((h, Fe)) * 0.3]
    gu = np.concatenate([one[0] if equal else rng.standard_normal((2 * Fe, h)) * 0.3
                         for _ in range(E)])
    down = np.concatenate([one[1] if equal else rng.standard_normal((h, Fe)) * 0.3
                           for _ in range(E)])
    return {"w_router": rng.standard_normal((E, h)), "w_gu": gu, "w_down": down}


def test_equal_experts_reduce_to_dense_swiglu():
    cfg = FD_TINY_MOE
    rng = np.random.default_rng(30)
    W = _moe_weights(cfg, rng, equal=True)
    n2 = rng.standard_normal((20, cfg.hidden))
    f, c = MOE.ffn_forward(W, n2, cfg)
    Fe, h = cfg.expert_ffn, cfg.hidden
    wg, wu, wd = W["w_gu"][:Fe], W["w_gu"][Fe:2 * Fe], W["w_down"][:h]
    dense = M.swiglu(n2 @ wg.T, n2 @ wu.T) @ wd.T
    np.testing.assert_allclose(f, dense, rtol=1e-12, atol=1e-12)
    df = rng.standard_normal(f.shape)
    dn2, g = MOE.ffn_backward(W, c, df, cfg)
    assert np.max(np.abs(g["w_router"])) <= 1e-12 * np.max(np.abs(df)) * 100
    # the experts' gradients add up to the dense block's
    dm = df @ wd
    da, du = M.swiglu_bwd(dm, n2 @ wg.T, n2 @ wu.T)
    np.testing.assert_allclose(dn2, da @ wg + du @ wu, rtol=1e-10, atol=1e-12)
    gsum = sum(g["w_down"][e * h:(e + 1) * h] for e in range(cfg.n_experts))
    np.testing.assert_allclose(gsum, df.T @ M.swiglu(n2 @ wg.T, n2 @ wu.T), rtol=1e-10,
                               atol=1e-12)


def test_top_k_equal_to_e_is_the_softmax_mixture():
    cfg = FD_TINY_MOE.replace(top_k=FD_TINY_MOE.n_experts)
    rng = np.random.default_rng(31)
    W = _moe_weights(cfg, rng)
    n2 = rng.standard_normal((12, cfg.hidden))
    f, _ = MOE.ffn_forward(W, n2, cfg)
    r = n2 @ W["w_router"].T
    p = np.exp(r - r.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    Fe, h = cfg.expert_ffn, cfg.hidden
    ref = np.zeros_like(n2)
    for e in range(cfg.n_experts):
        wg, wu = W["w_gu"][e * 2 * Fe:e * 2 * Fe + Fe], W["w_gu"][e * 2 * Fe + Fe:(e + 1) * 2 * Fe]
        ref += p[:, e:e + 1] * (M.swiglu(n2 @ wg.T, n2 @ wu.T) @ W["w_down"][e * h:(e + 1) * h].T)
    np.testing.assert_allclose(f, ref, rtol=1e-12, atol=1e-12)


def test_routing_and_combine_brute_force():
    cfg = FD_TINY_MOE
    rng = np.random.default_rng(32)
    W = _moe_weights(cfg, rng)
    n2 = rng.standard_normal((9, cfg.hidden))
    f, c = MOE.ffn_forward(W, n2, cfg)
    Fe, h, k = cfg.expert_ffn, cfg.hidden, cfg.top_k
    for t in range(n2.shape[0]):
        r = [float(n2[t] @ W["w_router"][e]) for e in range(cfg.n_experts)]
        # the k largest logits (the decision is taken on bf16-rounded operands; far from ties
        # here, so it picks the same experts as the exact logits)
        top = sorted(range(cfg.n_experts), key=lambda e: (-r[e], e))[:k]
        assert list(c["sel"][t]) == top
        z = [math.exp(r[e] - max(r[i] for i in top)) for e in top]
        out = np.zeros(h)
        for j, e in enumerate(top):
            wg, wu = W["w_gu"][e * 2 * Fe:e * 2 * Fe + Fe], W["w_gu"][e * 2 * Fe + Fe:(e + 1) * 2 * Fe]
            a, u = wg @ n2[t], wu @ n2[t]
            m = a / (1 + np.exp(-a)) * u
            out += z[j] / sum(z) * (W["w_down"][e * h:(e + 1) * h] @ m)
        np.testing.assert_allclose(f[t], out, rtol=1e-12, atol=1e-12)


def test_streamed_equals_whole_bit_exact_with_moe():
    cfg = MOE_PRESETS["M1"].replace(n_layers=4, ckpt_interval=2, seq_len=64)
    tok, lab = make_batch(cfg, 1)
    st = HostState(cfg, np.float32)
    st.load_weights(weight_stream(cfg, 0))
    loss_w, G = M.forward_backward_whole(st.params(), tok[0], lab[0], cfg, 1.0)
    for K in (1, 2, 4):
        gf = {g: np.zeros_like(st.master[g]) for g in st.groups}
        loss_s = M.forward_backward_streamed(st.master, tok[0], lab[0], cfg, 1.0, K, gf, False)
        assert loss_s == loss_w
        for g in st.groups:
            np.testing.assert_array_equal(gf[g], L.pack(cfg, g, G[g]), err_msg=f"K={K} g={g}")
