"""Streamed training steps through the C ABI against the CPU oracle.

Bar (bf16 compute, fp32 accumulate): loss within 1e-2 absolute, per-tensor
gradient relative L2 <= 2e-2, master weights relative L2 <= 1e-3 after the
steps.  Pipeline invariants: the checkpoint interval, the slab-pool size and
the CPU worker's timing must not change a single bit of the gradients.
"""
import os

import numpy as np
import pytest

from oracle import layout as OL
from oracle.train import HostState, train_step
from synth_inputs import PRESETS, make_batch, weight_stream
from tests.gpu_util import rel_l2

pytestmark = pytest.mark.gpu

LOSS_TOL, GRAD_TOL, WEIGHT_TOL = 1e-2, 2e-2, 1e-3


def _session(cfg, **kw):
    from host_memory_centric_stateless_amd import Session
    s = Session(cfg, **kw)
    s.load_weights(weight_stream(cfg, 0))
    return s


def _tensors(cfg, flat_by_group):
    out = {}
    for g, flat in flat_by_group.items():
        for name, _, off, n in OL.group_layout(cfg, g)[0]:
            out[(g, name)] = np.asarray(flat[off:off + n], dtype=np.float64)
    return out


def _compare_steps(cfg, steps, report):
    sess = _session(cfg)
    st = HostState(cfg, np.float32)
    st.load_weights(weight_stream(cfg, 0))
    worst = {"loss": 0.0, "grad": 0.0, "weight": 0.0}
    try:
        for step in range(1, steps + 1):
            tok, lab = make_batch(cfg, step)
            print(f"{cfg.name}: step {step} gpu", flush=True)
            gl = sess.forward_backward(tok, lab)
            print(f"{cfg.name}: step {step} oracle", flush=True)
            ol = train_step(st, tok, lab, step)
            worst["loss"] = max(worst["loss"], abs(gl - ol))
            gg, og = _tensors(cfg, sess.grad), _tensors(cfg, st.grad)
            for k in og:
                e = rel_l2(gg[k], og[k])
                report.setdefault(f"grad {k}", []).append(e)
                worst["grad"] = max(worst["grad"], e)
            from host_memory_centric_stateless_amd import mt_adamw_hparams, mt_adamw_step
            mt_adamw_step(sess.ctx, mt_adamw_hparams(cfg.lr, 0.9, 0.999, 1e-8, 0.01), step)
            gw, ow = _tensors(cfg, sess.master), _tensors(cfg, st.master)
            for k in ow:
                e = rel_l2(gw[k], ow[k])
                report.setdefault(f"weight {k}", []).append(e)
                if step == steps:
                    worst["weight"] = max(worst["weight"], e)
            print(f"{cfg.name}: step {step} loss gpu {gl:.6f} oracle {ol:.6f} "
                  f"worst grad {worst['grad']:.3e}", flush=True)
    finally:
        stats = sess.stats()
        sess.close()
    return worst, stats


def test_c1_three_steps_match_oracle():
    cfg = PRESETS["C1"]
    report = {}
    worst, stats = _compare_steps(cfg, 3, report)
    for k, v in sorted(report.items()):
        print(k, " ".join(f"{x:.2e}" for x in v))
    print("stats", stats)
    assert worst["loss"] <= LOSS_TOL
    assert worst["grad"] <= GRAD_TOL
    assert worst["weight"] <= WEIGHT_TOL
    # K = 1: 2 layers forward, 1 recomputed, 2 backward per micro-batch
    assert stats["layer_forwards"] == 3 * 3 and stats["layer_backwards"] == 3 * 2


def _grads_after_one_step(cfg, **kw):
    sess = _session(cfg, **kw)
    try:
        tok, lab = make_batch(cfg, 1)
        loss = sess.forward_backward(tok, lab)
        return loss, {g: a.copy() for g, a in sess.grad.items()}, sess.stats()
    finally:
        sess.close()


def test_pipeline_invariants_bit_exact():
    cfg = PRESETS["C1"].replace(grad_accum=2)
    base_loss, base, _ = _grads_after_one_step(cfg, ckpt_interval=1)
    for kw in ({"ckpt_interval": 2}, {"n_grad_slabs": 1}, {"n_grad_slabs": 2}):
        print("variant", kw, flush=True)
        loss, g, stats = _grads_after_one_step(cfg, **kw)
        assert loss == base_loss, kw
        for k in base:
            np.testing.assert_array_equal(g[k], base[k], err_msg=str((kw, k)))
    os.environ["MT_TEST_WORKER_DELAY_US"] = "3000"
    try:
        loss, g, stats = _grads_after_one_step(cfg, ckpt_interval=1, n_grad_slabs=2)
    finally:
        del os.environ["MT_TEST_WORKER_DELAY_US"]
    assert stats["slab_waits"] > 0
    for k in base:
        np.testing.assert_array_equal(g[k], base[k], err_msg=f"delayed worker {k}")


def test_call_order_state_machine():
    from host_memory_centric_stateless_amd import (MT_E_STATE, MtError, mt_adamw_hparams,
                                                   mt_adamw_step, mt_backward, mt_flush_grads,
                                                   mt_forward)
    cfg = PRESETS["C1"]
    sess = _session(cfg)
    try:
        hp = mt_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01)
        with pytest.raises(MtError) as e:
            mt_backward(sess.ctx, 0)
        assert e.value.status == MT_E_STATE
        with pytest.raises(MtError) as e:
            mt_adamw_step(sess.ctx, hp, 1)
        assert e.value.status == MT_E_STATE
        tok, lab = make_batch(cfg, 1)
        mt_forward(sess.ctx, tok[0].reshape(-1), lab[0].reshape(-1), 1.0)
        with pytest.raises(MtError) as e:
            mt_forward(sess.ctx, tok[0].reshape(-1), lab[0].reshape(-1), 1.0)
        assert e.value.status == MT_E_STATE
        with pytest.raises(MtError) as e:
            mt_flush_grads(sess.ctx)
        assert e.value.status == MT_E_STATE
        mt_backward(sess.ctx, 0)
        mt_flush_grads(sess.ctx)
        mt_adamw_step(sess.ctx, hp, 1)
        bad = tok[0].reshape(-1).copy()
        bad[3] = cfg.vocab
        with pytest.raises(MtError):
            mt_forward(sess.ctx, bad, lab[0].reshape(-1), 1.0)
    finally:
        sess.close()
