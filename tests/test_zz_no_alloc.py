"""The allocation-free RMSNorm backward (mtk_rmsnorm_bwd_noalloc) against the
workspace entry point it mirrors (mtk_rmsnorm_bwd), through the C ABI.

Both run the same kernels in the same order, so results must agree bit for
bit: on two calls in a row (the second with a smaller input, so the shared
scratch still holds the first call's partials), and a size beyond the fixed
scratch must be refused before anything is launched.
"""
import numpy as np
import pytest
import torch

import host_memory_centric_stateless_amd as mt
from synth_inputs import random_array
from tests.gpu_util import bf16_dev, dev, f32_dev

pytestmark = pytest.mark.gpu


def _inputs(T, h, seed):
    x = random_array((T, h), seed=seed, std=2.0)
    g = 1.0 + random_array((h,), seed=seed + 1, std=0.2)
    dn = random_array((T, h), seed=seed + 2)
    resid = random_array((T, h), seed=seed + 3)
    xd = f32_dev(x)
    gd = bf16_dev(g)
    out = torch.empty((T, h), dtype=torch.bfloat16, device=dev())
    rstd = torch.empty(T, dtype=torch.float32, device=dev())
    mt.mtk_rmsnorm_fwd(xd, gd, out, rstd, T, h, 1e-5)
    return f32_dev(dn), xd, rstd, gd, f32_dev(resid)


def _outputs(T, h):
    return (torch.full((T, h), float("nan"), dtype=torch.float32, device=dev()),
            torch.zeros((T, h), dtype=torch.bfloat16, device=dev()),
            torch.full((h,), float("nan"), dtype=torch.float32, device=dev()))


@pytest.mark.parametrize("shapes", [((8200, 5120), (300, 1024))])
def test_noalloc_rmsnorm_bwd_matches_workspace_entry_point(shapes):
    for i, (T, h) in enumerate(shapes):
        print(f"noalloc rmsnorm bwd call {i}: T={T} h={h}", flush=True)
        dn, x, rstd, g, resid = _inputs(T, h, 40 + 10 * i)
        dx_a, dxb_a, dg_a = _outputs(T, h)
        ws = torch.empty(mt.mtk_rmsnorm_bwd_workspace(T, h), dtype=torch.uint8, device=dev())
        mt.mtk_rmsnorm_bwd(dn, x, rstd, g, resid, dx_a, dxb_a, dg_a, ws, T, h)
        dx_b, dxb_b, dg_b = _outputs(T, h)
        mt.mtk_rmsnorm_bwd_noalloc(dn, x, rstd, g, resid, dx_b, dxb_b, dg_b, T, h)
        torch.cuda.synchronize()
        assert torch.equal(dx_a, dx_b)
        assert torch.equal(dxb_a.view(torch.int16), dxb_b.view(torch.int16))
        assert torch.equal(dg_a, dg_b)
        assert bool(torch.isfinite(dg_b).all())


def test_noalloc_rejects_sizes_beyond_its_scratch():
    T, h = 100_000, 16384   # partials of 2048 x 16384 fp32 = 128 MiB > the fixed 48 MiB
    assert mt.mtk_rmsnorm_bwd_workspace(T, h) > mt.mtk_noalloc_scratch_bytes()
    dummy = torch.empty(16, dtype=torch.float32, device=dev())
    with pytest.raises(mt.MtError) as e:
        mt.mtk_rmsnorm_bwd_noalloc(dummy, dummy, dummy, dummy, None, dummy, None, dummy, T, h)
    assert e.value.status == mt.MT_E_NOMEM
