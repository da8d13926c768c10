"""Pins of the CPU oracle against things other than itself.

Each check is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a wrong mask or head mapping)
fails at least one of them:

* finite differences in float64 pin every analytic backward against its forward;
* torch.autograd (float64, CPU) is a second, independent derivative;
* closed forms pin the forwards: constant-row RMSNorm, RoPE of a unit vector,
  attention with zero queries (uniform causal average), grouped-head mapping,
  uniform-logit cross-entropy, AdamW's first step;
* invariants: RMS of the normalised row, RoPE norm and relative-position
  invariance, probability rows summing to one, dlogits rows summing to zero;
* the streamed-with-recompute driver equals the whole-model driver bit for bit;
* the initial loss of N(0, 0.02) weights sits at ln V + 0.0002 h.
"""
import math

import numpy as np
import pytest
import torch

from oracle import layout as L
from oracle import model as M
from oracle.adamw import AdamWHparams, adamw_step
from oracle.train import HostState, train_step
from synth_inputs import FD_TINY, PRESETS, make_batch, tensor_specs, weight_stream


# ------------------------------------------------------------ helpers
def _fd_params(cfg, seed=7, std=0.5):
    """float64 params with large weights and non-unit gains so that every
    nonlinearity and every gain participates in the gradient."""
    rng = np.random.default_rng(seed)
    P = {}
    for g in [L.EMBED] + list(range(cfg.n_layers)) + [L.HEAD]:
        P[g] = {}
        for name, shape, kind in tensor_specs(cfg, g):
            if kind == "gain":
                P[g][name] = 1.0 + 0.3 * rng.standard_normal(shape)
            else:
                P[g][name] = std * rng.standard_normal(shape)
    return P


def _tiny_batch(cfg, seed=3):
    rng = np.random.default_rng(seed)
    tok = rng.integers(0, cfg.vocab, size=(cfg.micro_batch, cfg.seq_len)).astype(np.int64)
    lab = np.full_like(tok, -1)
    lab[:, :-1] = tok[:, 1:]
    return tok, lab


def _loss(P, tok, lab, cfg):
    loss, _ = M.forward_backward_whole(P, tok, lab, cfg, 1.0)
    return float(loss)


# --------------------------------------------------- finite differences
def test_fd_directional_all_params():
    cfg = FD_TINY
    P = _fd_params(cfg)
    tok, lab = _tiny_batch(cfg)
    _, G = M.forward_backward_whole(P, tok, lab, cfg, 1.0)
    rng = np.random.default_rng(11)
    U = {g: {n: rng.standard_normal(a.shape) for n, a in d.items()} for g, d in P.items()}
    analytic = sum(float(np.sum(G[g][n] * U[g][n])) for g in P for n in P[g])
    h = 1e-6

    def shifted(sign):
        return {g: {n: P[g][n] + sign * h * U[g][n] for n in P[g]} for g in P}

    fd = (_loss(shifted(+1), tok, lab, cfg) - _loss(shifted(-1), tok, lab, cfg)) / (2 * h)
    assert abs(fd - analytic) <= 1e-6 * abs(analytic), (fd, analytic)


def test_fd_per_element_every_tensor():
    cfg = FD_TINY
    P = _fd_params(cfg, seed=8)
    tok, lab = _tiny_batch(cfg, seed=4)
    _, G = M.forward_backward_whole(P, tok, lab, cfg, 1.0)
    rng = np.random.default_rng(12)
    h = 1e-6
    scale = max(float(np.max(np.abs(G[g][n]))) for g in P for n in P[g])
    for g in P:
        for name in P[g]:
            arr = P[g][name]
            for _ in range(4):
                idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
                if g == L.EMBED:          # pick a row that the batch reads
                    idx = (int(tok.reshape(-1)[rng.integers(0, tok.size)]), idx[1])
                old = arr[idx]
                arr[idx] = old + h
                fp = _loss(P, tok, lab, cfg)
                arr[idx] = old - h
                fm = _loss(P, tok, lab, cfg)
                arr[idx] = old
                fd = (fp - fm) / (2 * h)
                assert abs(fd - G[g][name][idx]) <= 1e-6 * scale + 1e-6 * abs(fd), (g, name, idx)


# ------------------------------------------------ torch.autograd, float64
def _torch_loss(P, tok, lab, cfg):
    """Same model written with torch ops; gradients from autograd."""
    T = {g: {n: torch.tensor(a, dtype=torch.float64, requires_grad=True) for n, a in d.items()}
         for g, d in P.items()}
    b, s = tok.shape
    nq, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    eps = cfg.rms_eps

    def rms(x, w):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps) * w

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
        k = rot((n1 @ W["wk"].T).view(b, s, nkv, d)).permute(0, 2, 1, 3)
        v = (n1 @ W["wv"].T).view(b, s, nkv, d).permute(0, 2, 1, 3)
        k = k.repeat_interleave(nq // nkv, dim=1)
        v = v.repeat_interleave(nq // nkv, dim=1)
        S = (q @ k.transpose(-1, -2)) / math.sqrt(d)
        S = S.masked_fill(~mask, float("-inf"))
        o = (torch.softmax(S, -1) @ v).permute(0, 2, 1, 3).reshape(b * s, nq * d)
        h1 = x + o @ W["wo"].T
        n2 = rms(h1, W["mlp_norm"])
        x = h1 + (torch.nn.functional.silu(n2 @ W["w_gate"].T) * (n2 @ W["w_up"].T)) @ W["w_down"].T
    xf = rms(x, T[L.HEAD]["final_norm"])
    logits = xf @ T[L.HEAD]["w_head"].T
    loss = torch.nn.functional.cross_entropy(logits, torch.tensor(lab.reshape(-1)), ignore_index=-1)
    loss.backward()
    return float(loss), {g: {n: t.grad.numpy() for n, t in d.items()} for g, d in T.items()}


def test_matches_torch_autograd_float64():
    cfg = FD_TINY
    P = _fd_params(cfg, seed=9)
    tok, lab = _tiny_batch(cfg, seed=5)
    loss, G = M.forward_backward_whole(P, tok, lab, cfg, 1.0)
    tl, TG = _torch_loss(P, tok, lab, cfg)
    assert abs(loss - tl) <= 1e-12 * abs(tl)
    for g in P:
        for n in P[g]:
            err = np.max(np.abs(G[g][n] - TG[g][n]))
            assert err <= 1e-10 * max(1.0, np.max(np.abs(TG[g][n]))), (g, n, err)


# ----------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_forms():
    h, eps = 64, 1e-5
    x = np.full((3, h), 0.37)
    n, r = M.rmsnorm(x, np.ones(h), eps)
    np.testing.assert_allclose(n, 0.37 / math.sqrt(0.37 ** 2 + eps), rtol=1e-15)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, h)) * 3.0
    n, r = M.rmsnorm(x, np.ones(h), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(n * n, axis=1)), 1.0, rtol=1e-13)
    g = rng.standard_normal(h)
    n2, _ = M.rmsnorm(x, g, 0.0)
    np.testing.assert_allclose(n2, n * g, rtol=1e-13)


def test_rmsnorm_bwd_orthogonal_to_input_when_eps_zero():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 32))
    g = rng.standard_normal(32)
    _, r = M.rmsnorm(x, g, 0.0)
    dx, _ = M.rmsnorm_bwd(rng.standard_normal((6, 32)), x, r, g)
    np.testing.assert_allclose(np.sum(dx * x, axis=1), 0.0, atol=1e-12)


# -------------------------------------------------------------- RoPE
def test_rope_unit_vector_closed_form():
    s, d, base = 50, 16, 10000.0
    cos, sin = M.rope_tables(s, d, base, np.float64)
    for i in range(d // 2):
        x = np.zeros((1, s, 1, d))
        x[..., i] = 1.0
        y = M.rope(x, cos, sin)
        ang = np.arange(s) * base ** (-2.0 * i / d)
        np.testing.assert_allclose(y[0, :, 0, i], np.cos(ang), atol=1e-15)
        np.testing.assert_allclose(y[0, :, 0, i + d // 2], np.sin(ang), atol=1e-15)
        others = np.delete(y[0, :, 0], [i, i + d // 2], axis=1)
        assert np.all(others == 0)


def test_rope_norm_inverse_and_relative_position():
    s, d, c = 40, 32, 7
    rng = np.random.default_rng(2)
    cos, sin = M.rope_tables(s + c, d, 10000.0, np.float64)
    q = rng.standard_normal((1, s, 2, d))
    k = rng.standard_normal((1, s, 2, d))
    qr = M.rope(q, cos[:s], sin[:s])
    half = d // 2
    pair = lambda z: z[..., :half] ** 2 + z[..., half:] ** 2
    np.testing.assert_allclose(pair(qr), pair(q), rtol=1e-12)
    np.testing.assert_allclose(M.rope(qr, cos[:s], sin[:s], inverse=True), q, atol=1e-13)
    kr = M.rope(k, cos[:s], sin[:s])
    q2, k2 = M.rope(q, cos[c:], sin[c:]), M.rope(k, cos[c:], sin[c:])
    S1 = np.einsum("qd,kd->qk", qr[0, :, 0], kr[0, :, 0])
    S2 = np.einsum("qd,kd->qk", q2[0, :, 0], k2[0, :, 0])
    np.testing.assert_allclose(S1, S2, atol=1e-10)


# --------------------------------------------------------- attention
def test_attention_zero_queries_is_causal_mean():
    b, s, nq, nkv, d = 2, 9, 4, 2, 8
    rng = np.random.default_rng(3)
    k = rng.standard_normal((b, s, nkv, d))
    v = rng.standard_normal((b, s, nkv, d))
    o = M.attention(np.zeros((b, s, nq, d)), k, v)
    cum = np.cumsum(v, axis=1) / np.arange(1, s + 1)[None, :, None, None]
    for j in range(nq):
        np.testing.assert_allclose(o[:, :, j], cum[:, :, j // 2], rtol=1e-12)
    np.testing.assert_allclose(M.attention_lse(np.zeros((b, s, nq, d)), k)[0, :, 0],
                               np.log(np.arange(1, s + 1)), rtol=1e-12)


def test_attention_head_mapping_row0_and_rows():
    b, s, nq, nkv, d = 1, 12, 6, 2, 4
    rng = np.random.default_rng(4)
    q = rng.standard_normal((b, s, nq, d))
    k = rng.standard_normal((b, s, nkv, d))
    v = np.zeros((b, s, nkv, d))
    v[:, :, 0] = 1.0
    v[:, :, 1] = -2.0
    o = M.attention(q, k, v)
    np.testing.assert_allclose(o[:, :, :3], 1.0, rtol=1e-12)     # heads 0..2 read kv head 0
    np.testing.assert_allclose(o[:, :, 3:], -2.0, rtol=1e-12)    # heads 3..5 read kv head 1
    v = rng.standard_normal((b, s, nkv, d))
    o = M.attention(q, k, v)
    for j in range(nq):
        np.testing.assert_allclose(o[:, 0, j], v[:, 0, j // 3], rtol=1e-12)
    rows = [0, 5, 11]
    np.testing.assert_allclose(M.attention_rows(q, k, v, rows), o[:, rows], rtol=1e-12)
    P = M._scores(q[0, :, 0], k[0, :, 0], 0.5)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(np.triu(P, 1) == 0)


# -------------------------------------------------- cross-entropy / misc
def test_cross_entropy_uniform_and_gradient():
    V = 37
    lab = np.array([3, -1, 0, 36])
    loss, dl, lse = M.cross_entropy(np.zeros((4, V)), lab, 1.0)
    assert abs(loss - math.log(V)) < 1e-15
    np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-16)
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((4, V))
    loss, dl, _ = M.cross_entropy(lg, lab, 0.5)
    p = np.exp(lg) / np.exp(lg).sum(1, keepdims=True)
    ref = p.copy()
    ref[np.arange(4), np.maximum(lab, 0)] -= 1
    ref[1] = 0
    np.testing.assert_allclose(dl, ref * 0.5 / 3, rtol=1e-12, atol=1e-16)
    brute = np.mean([-math.log(p[i, lab[i]]) for i in (0, 2, 3)])
    assert abs(loss - brute) < 1e-12


def test_swiglu_derivative_and_values():
    a = np.linspace(-8, 8, 101)
    h = 1e-6
    u = np.full_like(a, 1.7)
    da, du = M.swiglu_bwd(np.ones_like(a), a, u)
    fd = (M.swiglu(a + h, u) - M.swiglu(a - h, u)) / (2 * h)
    np.testing.assert_allclose(da, fd, rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(du, M.swiglu(a, np.ones_like(a)), rtol=1e-15)
    assert M.swiglu(np.array([0.0]), np.array([5.0]))[0] == 0.0


def test_embedding_scatter_add_brute_force():
    rng = np.random.default_rng(6)
    tok = np.array([[3, 1, 3, 3], [0, 1, 7, 3]])
    dx0 = rng.standard_normal((8, 5))
    dE = M.embed_bwd(dx0, tok, 9)
    ref = np.zeros((9, 5))
    for t, row in enumerate(tok.reshape(-1)):
        ref[row] += dx0[t]
    np.testing.assert_array_equal(dE, ref)
    assert np.all(dE[[2, 4, 5, 6, 8]] == 0)


# ------------------------------------------------------------- AdamW
def test_adamw_first_step_closed_form_and_decay():
    hp = AdamWHparams(lr=1e-3)
    rng = np.random.default_rng(7)
    p = rng.standard_normal(1000)
    g = rng.standard_normal(1000)
    p1, m, v = p.copy(), np.zeros(1000), np.zeros(1000)
    adamw_step(p1, g, m, v, 1, hp)
    expect = p * (1 - hp.lr * hp.weight_decay) - hp.lr * g / (np.abs(g) + hp.eps)
    np.testing.assert_allclose(p1, expect, rtol=1e-12)
    p2, m, v = p.copy(), np.zeros(1000), np.zeros(1000)
    adamw_step(p2, np.zeros(1000), m, v, 1, hp)
    np.testing.assert_array_equal(p2, p * (1 - hp.lr * hp.weight_decay))


def test_adamw_three_steps_match_torch():
    hp = AdamWHparams(lr=1e-3)
    rng = np.random.default_rng(8)
    p0 = rng.standard_normal(4096).astype(np.float32) * 0.02
    grads = [rng.standard_normal(4096).astype(np.float32) * 1e-3 for _ in range(3)]
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    tp = torch.nn.Parameter(torch.tensor(p0))
    opt = torch.optim.AdamW([tp], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps,
                            weight_decay=hp.weight_decay, foreach=False)
    for t, g in enumerate(grads, start=1):
        adamw_step(p, g, m, v, t, hp)
        tp.grad = torch.tensor(g)
        opt.step()
    np.testing.assert_allclose(p, tp.detach().numpy(), rtol=2e-6, atol=1e-9)


# ------------------------------------------- streamed == whole, bit-exact
def _small_cfgs():
    c1 = PRESETS["C1"]
    c2s = PRESETS["C2"].replace(name="small-4L", n_layers=4, micro_batch=1, seq_len=256)
    return [c1, c2s]


@pytest.mark.parametrize("which", [0, 1])
def test_streamed_equals_whole_bit_exact(which):
    cfg = _small_cfgs()[which]
    Ks = sorted({1, 2, cfg.n_layers})
    tok, lab = make_batch(cfg, 1)
    st = HostState(cfg, np.float32)
    st.load_weights(weight_stream(cfg, 0))
    loss_w, G = M.forward_backward_whole(st.params(), tok[0], lab[0], cfg, 1.0)
    for K in Ks:
        gf = {g: np.zeros_like(st.master[g]) for g in st.groups}
        stats = {}
        loss_s = M.forward_backward_streamed(st.master, tok[0], lab[0], cfg, 1.0, K, gf, False,
                                             stats)
        assert loss_s == loss_w
        assert stats["checkpoints"] == -(-cfg.n_layers // K)
        for g in st.groups:
            np.testing.assert_array_equal(gf[g], L.pack(cfg, g, G[g]), err_msg=f"K={K} g={g}")


def test_train_step_streamed_equals_whole_with_accumulation():
    cfg = PRESETS["C1"].replace(grad_accum=2)
    tok, lab = make_batch(cfg, 1)
    a, b = HostState(cfg), HostState(cfg)
    a.load_weights(weight_stream(cfg, 0))
    b.load_weights(weight_stream(cfg, 0))
    for step in (1, 2):
        tok, lab = make_batch(cfg, step)
        la = train_step(a, tok, lab, step, mode="streamed", K=1)
        lb = train_step(b, tok, lab, step, mode="whole")
        assert la == lb
        for g in a.groups:
            np.testing.assert_array_equal(a.master[g], b.master[g])


# ---------------------------------------------------------- initial loss
@pytest.mark.parametrize("which", ["C1", "C2"])
def test_initial_loss_near_lnV(which):
    cfg = PRESETS[which]
    if which == "C2":           # the statistic depends on h and V only
        cfg = cfg.replace(micro_batch=1, seq_len=256, n_layers=2)
    st = HostState(cfg)
    st.load_weights(weight_stream(cfg, 0))
    tok, lab = make_batch(cfg, 1)
    loss, _ = M.forward_backward_whole(st.params(), tok[0], lab[0], cfg, 1.0)
    expect = math.log(cfg.vocab) + 0.0002 * cfg.hidden
    assert abs(float(loss) - expect) < 0.05, (float(loss), expect)


def test_zero_matrices_give_ln_v():
    cfg = PRESETS["C1"]
    st = HostState(cfg)
    st.load_weights(weight_stream(cfg, 0))
    P = st.params()
    for g in P:
        for n, a in P[g].items():
            if a.ndim == 2 and n != "emb":
                a[...] = 0
    tok, lab = make_batch(cfg, 1)
    loss, G = M.forward_backward_whole(P, tok[0], lab[0], cfg, 1.0)
    assert abs(float(loss) - math.log(cfg.vocab)) < 1e-6
