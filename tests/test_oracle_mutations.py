"""Planted mistakes in the oracle must be caught by its pins.

Each case patches one oracle function with a plausible slip (on the CPU,
inside this process only) and asserts that at least one pin that does not
use the oracle's own output as reference fails.  This checks the strength of
the pins, not the HIP path.
"""
import contextlib

import numpy as np
import pytest

import oracle.model as M
import tests.test_oracle_pins as P

_orig = {n: getattr(M, n) for n in ["rope", "rmsnorm_bwd", "swiglu_bwd", "attention", "_scores",
                                     "rope_tables", "rmsnorm", "cross_entropy"]}


def _gqa_modulo(q, k, v):
    b, s, nq, d = q.shape
    nkv = k.shape[2]
    o = np.empty_like(q)
    for bi in range(b):
        for j in range(nq):
            p = _orig["_scores"](q[bi, :, j], k[bi, :, j % nkv], 1 / np.sqrt(d))
            o[bi, :, j] = p @ v[bi, :, j % nkv]
    return o


def _no_mask(qh, kh, scale):
    S = (qh @ kh.T) * scale
    E = np.exp(S - S.max(1, keepdims=True))
    return E / E.sum(1, keepdims=True)


def _ce_no_shift(logits, labels, gs):
    loss, dl, lse = _orig["cross_entropy"](logits, labels, gs)
    return loss, dl * 2.0, lse


MUTATIONS = {
    "rope_backward_not_inverted": ("rope", lambda x, c, s, inverse=False: _orig["rope"](x, c, s, False)),
    "rope_forward_sign": ("rope", lambda x, c, s, inverse=False: _orig["rope"](x, c, s, not inverse)),
    "rope_base_wrong": ("rope_tables", lambda s, d, b, dt: _orig["rope_tables"](s, d, 2 * b, dt)),
    "rmsnorm_bwd_drops_projection": ("rmsnorm_bwd", lambda dn, x, r, g: (r * dn * g, np.sum(dn * x * r, 0))),
    "rmsnorm_eps_outside_sqrt": ("rmsnorm", lambda x, g, eps: (x / (np.sqrt(np.mean(x * x, -1, keepdims=True)) + eps) * g,
                                                             1 / (np.sqrt(np.mean(x * x, -1, keepdims=True)) + eps))),
    "silu_derivative_missing_term": ("swiglu_bwd", lambda dm, a, u: (dm * u * M.sigmoid(a), dm * a * M.sigmoid(a))),
    "gqa_modulo_mapping": ("attention", _gqa_modulo),
    "causal_mask_missing": ("_scores", _no_mask),
    "score_scale_missing": ("_scores", lambda q, k, s: _orig["_scores"](q, k, 1.0)),
    "dlogits_scaled_twice": ("cross_entropy", _ce_no_shift),
}

PINS = ["test_fd_directional_all_params", "test_fd_per_element_every_tensor",
        "test_rmsnorm_closed_forms", "test_rmsnorm_bwd_orthogonal_to_input_when_eps_zero",
        "test_rope_unit_vector_closed_form", "test_rope_norm_inverse_and_relative_position",
        "test_attention_zero_queries_is_causal_mean", "test_attention_head_mapping_row0_and_rows",
        "test_cross_entropy_uniform_and_gradient", "test_swiglu_derivative_and_values",
        "test_zero_matrices_give_ln_v"]


@contextlib.contextmanager
def _patched(attr, fn):
    setattr(M, attr, fn)
    try:
        yield
    finally:
        setattr(M, attr, _orig[attr])


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation):
    attr, fn = MUTATIONS[mutation]
    failed = []
    with _patched(attr, fn):
        for name in PINS:
            try:
                getattr(P, name)()
            except Exception:
                failed.append(name)
    assert failed, f"no pin caught {mutation}"


# ------------------------------------------- accumulation and step loss
import inspect
import textwrap

import oracle.train as TR
import tests.test_oracle_accumulation as A

TRAIN_MUTATIONS = {
    "accumulation_not_scaled": ("scale = 1.0 / acc", "scale = 1.0"),
    "step_loss_summed": ("np.mean(losses)", "np.sum(losses)"),
}
ACC_PINS = ["test_repeated_microbatch_equals_single_step",
            "test_two_microbatches_average_their_gradients_and_losses"]


@pytest.mark.parametrize("mutation", sorted(TRAIN_MUTATIONS))
def test_planted_accumulation_mistake_is_caught(mutation):
    old, new = TRAIN_MUTATIONS[mutation]
    src = textwrap.dedent(inspect.getsource(TR.train_step))
    assert src.count(old) == 1, "the planted slip no longer matches the oracle's source"
    ns = dict(vars(TR))
    exec(compile(src.replace(old, new), TR.__file__, "exec"), ns)
    orig = TR.train_step
    TR.train_step = ns["train_step"]
    failed = []
    try:
        for name in ACC_PINS:
            try:
                getattr(A, name)()
            except Exception:
                failed.append(name)
    finally:
        TR.train_step = orig
    assert failed, f"no pin caught {mutation}"


# ---------------------------------------------------- mixture-of-experts block
import oracle.moe as MOE
import tests.test_oracle_moe as TM

_moe_orig = {n: getattr(MOE, n) for n in ["route", "ffn_backward", "expert_weights"]}


def _route_smallest(n2, w_router, k):
    r, sel, g = _moe_orig["route"](n2, w_router, k)
    sel2 = np.argsort(r, axis=1, kind="stable")[:, :k]
    sl = np.take_along_axis(r, sel2, axis=1)
    z = np.exp(sl - sl.max(axis=1, keepdims=True))
    return r, sel2, z / z.sum(axis=1, keepdims=True)


def _route_unnormalised(n2, w_router, k):
    r, sel, g = _moe_orig["route"](n2, w_router, k)
    return r, sel, np.exp(np.take_along_axis(r, sel, axis=1))


def _bwd_no_softmax_projection(W, c, df, cfg):
    # dr = g * dg instead of g * (dg - sum g dg): re-derive with a patched gate grad
    dn2, grads = _moe_orig["ffn_backward"](W, c, df, cfg)
    T = df.shape[0]
    g, sel = c["g"], c["sel"]
    dg = np.zeros_like(g)
    h = df.shape[1]
    for e in range(cfg.n_experts):
        p = c["per"][e]
        dg[p["tok"], p["slot"]] = np.sum(df[p["tok"]] * p["o"], axis=1)
    right = g * (dg - np.sum(g * dg, axis=1, keepdims=True))
    wrong = g * dg
    dr_r, dr_w = np.zeros((T, cfg.n_experts)), np.zeros((T, cfg.n_experts))
    np.put_along_axis(dr_r, sel, right, axis=1)
    np.put_along_axis(dr_w, sel, wrong, axis=1)
    grads["w_router"] = dr_w.T @ c["n2"]
    return dn2 - dr_r @ W["w_router"] + dr_w @ W["w_router"], grads


def _experts_shifted(W, e, h, Fe):
    return _moe_orig["expert_weights"](W, (e + 1) % (W["w_router"].shape[0]), h, Fe)


MOE_MUTATIONS = {
    "moe_selects_smallest_logits": ("route", _route_smallest),
    "moe_gates_not_normalised": ("route", _route_unnormalised),
    "moe_softmax_backward_projection_dropped": ("ffn_backward", _bwd_no_softmax_projection),
    "moe_wrong_expert_weights": ("expert_weights", _experts_shifted),
}
MOE_PINS = ["test_fd_directional_all_params_with_moe", "test_equal_experts_reduce_to_dense_swiglu",
            "test_top_k_equal_to_e_is_the_softmax_mixture", "test_routing_and_combine_brute_force",
            "test_moe_matches_torch_autograd_float64"]


@pytest.mark.parametrize("mutation", sorted(MOE_MUTATIONS))
def test_planted_moe_mistake_is_caught(mutation):
    attr, fn = MOE_MUTATIONS[mutation]
    failed = []
    setattr(MOE, attr, fn)
    try:
        for name in MOE_PINS:
            try:
                getattr(TM, name)()
            except Exception:
                failed.append(name)
    finally:
        setattr(MOE, attr, _moe_orig[attr])
    assert failed, f"no pin caught {mutation}"
