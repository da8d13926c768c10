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
