"""Pins of the oracle's flat layout and host-state accounting.

Layout: offsets follow the closed-form rule (each tensor at the next multiple
of 256 elements, groups in data-flow order) and pack/unpack round-trips bit
for bit.  Accounting: the byte-per-parameter constants reproduce the memory
figures the pages print (tests/golden/host_state_bytes.txt, each line cited).
"""
import os

import numpy as np
import pytest

from oracle import accounting as A
from oracle import layout as L
from synth_inputs import PRESETS, FD_TINY, make_weights

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "host_state_bytes.txt")


def _rup(n):
    return -(-n // 256) * 256


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_layer_offsets_closed_form(name):
    cfg = PRESETS[name]
    h, F = cfg.hidden, cfg.ffn
    qd, kvd = cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    sizes = [h, qd * h, kvd * h, kvd * h, h * qd, h, F * h, F * h, h * F]
    ent, total = L.group_layout(cfg, 0)
    off = 0
    for (nm, shape, o, n), sz in zip(ent, sizes):
        assert o == _rup(off) and n == sz, nm
        off = o + n
    assert total == _rup(off)
    p_layer = h * qd + 2 * h * kvd + qd * h + 3 * h * F + 2 * h
    assert total == p_layer            # every dim here is a multiple of 256


def test_published_layer_sizes():
    # per-layer element counts of the 7B- and 14B-shaped decoders
    assert L.group_layout(PRESETS["C3"], 0)[1] == 202_383_360
    assert L.group_layout(PRESETS["C4"], 0)[1] == 275_261_440
    assert L.param_count(PRESETS["C3"]) == 6_738_415_616
    assert L.param_count(PRESETS["C4"]) == 14_769_689_600


def test_padding_and_round_trip():
    cfg = FD_TINY                       # h = 16: gains need padding
    W = make_weights(cfg, 0)
    for g, tensors in W.items():
        ent, total = L.group_layout(cfg, g)
        assert all(o % 256 == 0 for _, _, o, _ in ent)
        flat = L.pack(cfg, g, tensors)
        back = L.unpack(cfg, g, flat)
        for nm, a in tensors.items():
            np.testing.assert_array_equal(back[nm], a)
        mask = np.ones(total, bool)
        for _, _, o, n in ent:
            mask[o:o + n] = False
        assert np.all(flat[mask] == 0)


def test_page_memory_figures():
    rows = [l.split(None, 4) for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) == 4
    per = {12: A.MIXED_STATE_BYTES_PER_PARAM, 16: A.FP32_STATE_BYTES_PER_PARAM,
           2: A.BF16_WORKING_BYTES_PER_PARAM}
    for n, bpp, total, tol, _src in rows:
        got = float(n) * per[int(bpp)]
        assert abs(got - float(total)) <= float(tol) * float(total), (n, bpp, got, total)
    assert A.host_state_bytes(10 ** 9) == 16 * 10 ** 9
