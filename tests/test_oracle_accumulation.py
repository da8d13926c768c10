"""Pins of the oracle's gradient accumulation and step loss.

Global batch via gradient accumulation (travelaiplan, 怎麼開始): a step of
``acc`` micro-batches must compute the gradient of the MEAN loss over its
micro-batches, i.e. the host gradient is the average of the micro-batch
gradients, and the reported step loss is the average of the micro-batch
losses (reading O5).  These checks do not use train_step's own arithmetic as
the reference:

* repeating one micro-batch ``acc`` times is the same optimisation problem as
  that micro-batch alone, so loss, gradients and updated weights must equal
  the acc = 1 step bit for bit (halving and adding two equal halves is exact);
* with two different micro-batches the accumulated gradient must equal the
  average of the two single-micro-batch gradients of the whole-model driver
  at grad_scale 1, and the step loss the average of their losses.
"""
import numpy as np

from oracle import layout as L
from oracle import model as M
from oracle import train as T
from synth_inputs import PRESETS, make_batch, weight_stream


def _state(cfg):
    st = T.HostState(cfg, np.float32)
    st.load_weights(weight_stream(cfg, 0))
    return st


def test_repeated_microbatch_equals_single_step():
    cfg1 = PRESETS["C1"]
    tok, lab = make_batch(cfg1, 1)
    one = _state(cfg1)
    loss1 = T.train_step(one, tok, lab, 1, K=1)
    for acc in (2, 4):
        cfg = cfg1.replace(grad_accum=acc)
        rep = _state(cfg)
        loss_r = T.train_step(rep, np.repeat(tok, acc, 0), np.repeat(lab, acc, 0), 1, K=1)
        assert loss_r == loss1, (acc, loss_r, loss1)
        for g in one.groups:
            np.testing.assert_array_equal(rep.grad[g], one.grad[g], err_msg=f"acc={acc} grad {g}")
            np.testing.assert_array_equal(rep.master[g], one.master[g],
                                          err_msg=f"acc={acc} master {g}")


def test_two_microbatches_average_their_gradients_and_losses():
    cfg = PRESETS["C1"].replace(grad_accum=2)
    tok, lab = make_batch(cfg, 2)
    st = _state(cfg)
    P = st.params()
    singles = [M.forward_backward_whole(P, tok[i], lab[i], cfg, 1.0) for i in range(2)]
    expect = {g: (L.pack(cfg, g, singles[0][1][g]) + L.pack(cfg, g, singles[1][1][g])) / 2
              for g in st.groups}
    expect_loss = (float(singles[0][0]) + float(singles[1][0])) / 2
    loss = T.train_step(st, tok, lab, 1, K=1)
    assert abs(loss - expect_loss) <= 1e-6 * abs(expect_loss), (loss, expect_loss)
    for g in st.groups:
        np.testing.assert_allclose(st.grad[g], expect[g], rtol=1e-5, atol=1e-9,
                                   err_msg=f"group {g}")
