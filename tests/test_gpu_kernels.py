"""Per-kernel parity of the gfx950 kernels (through the C ABI) with the CPU
oracle on seeded inputs.  Shapes are ragged and span several tiles.

Tolerances follow the arithmetic: operands are bf16 (the oracle is fed the
same bf16 values in float64), accumulation is fp32, so fp32 outputs agree to
~1e-5 of their scale and bf16 outputs to half a bf16 ulp (2^-9) plus that.
"""
import math

import numpy as np
import pytest
import torch

import host_memory_centric_stateless_amd as mt
from oracle import model as OM
from synth_inputs import random_array
from tests.gpu_util import bf16_dev, bf16_round, dev, f32_dev, host, rel_max

pytestmark = pytest.mark.gpu

BF16_REL = 2.0 ** -8


def _gemm_ref(layout, A, B):
    """C[m, n] = sum_k A(m, k) B(n, k) for the given storage layouts."""
    a = A if layout != mt.MT_GEMM_TN else A.T
    b = B if layout == mt.MT_GEMM_NT else B.T
    return a @ b.T


@pytest.mark.parametrize("layout", [mt.MT_GEMM_NT, mt.MT_GEMM_NN, mt.MT_GEMM_TN])
@pytest.mark.parametrize("shape", [(200, 136, 88), (264, 392, 520), (512, 256, 4096),
                                   (2056, 1288, 200), (4096, 4096, 256),
                                   # 256 x 256 tiles with row and column tails: direct-to-LDS
                                   # loads (K a multiple of 128), then register-staged (K tail)
                                   (4104, 3080, 384), (4104, 3080, 328)])
def test_gemm_layouts_f32_bf16(layout, shape):
    M, N, K = shape
    print(f"gemm layout={layout} shape={shape}", flush=True)
    A = random_array((M, K) if layout != mt.MT_GEMM_TN else (K, M), seed=1)
    B = random_array((N, K) if layout == mt.MT_GEMM_NT else (K, N), seed=2)
    Ad, Bd = bf16_dev(A), bf16_dev(B)
    lda = A.shape[1]
    ldb = B.shape[1]
    ref = _gemm_ref(layout, bf16_round(A), bf16_round(B))
    C32 = torch.empty((M, N), dtype=torch.float32, device=dev())
    mt.mtk_gemm(layout, mt.MT_EPI_F32, M, N, K, Ad, lda, Bd, ldb, C32, N)
    assert rel_max(host(C32), ref) < 2e-5
    C16 = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    mt.mtk_gemm(layout, mt.MT_EPI_BF16, M, N, K, Ad, lda, Bd, ldb, C16, N)
    got = host(C16)
    assert np.all(np.abs(got - ref) <= BF16_REL * np.abs(ref) + 2e-5 * np.max(np.abs(ref)))
    # residual add and accumulate epilogues, with a padded output stride
    R = random_array((M, N + 8), seed=3)
    Cr = f32_dev(np.zeros((M, N + 8), np.float32))
    mt.mtk_gemm(layout, mt.MT_EPI_F32_RESID, M, N, K, Ad, lda, Bd, ldb, Cr, N + 8,
                R=f32_dev(R), ldr=N + 8)
    out = host(Cr)
    assert rel_max(out[:, :N], ref + R[:, :N]) < 2e-5
    assert np.all(out[:, N:] == 0)
    Ca = f32_dev(R[:, :N])
    mt.mtk_gemm(layout, mt.MT_EPI_F32_ACCUM, M, N, K, Ad, lda, Bd, ldb, Ca, N)
    assert rel_max(host(Ca), ref + R[:, :N]) < 2e-5


@pytest.mark.parametrize("T,h,F", [(136, 256, 688), (304, 512, 1408), (1032, 256, 1048),
                                   (4104, 256, 2056)])  # the last on 256 x 256 direct-to-LDS tiles
def test_gemm_swiglu_forward_and_backward(T, h, F):
    print(f"swiglu T={T} h={h} F={F}", flush=True)
    n2 = random_array((T, h), seed=4)
    Wgu = random_array((2 * F, h), seed=5, std=0.05)
    gu = torch.empty((T, 2 * F), dtype=torch.bfloat16, device=dev())
    m = torch.empty((T, F), dtype=torch.bfloat16, device=dev())
    mt.mtk_gemm(mt.MT_GEMM_NT, mt.MT_EPI_SWIGLU, T, F, h, bf16_dev(n2), h, bf16_dev(Wgu), h, m, F,
                gu=gu, ldgu=2 * F, ffn=F)
    a = bf16_round(n2) @ bf16_round(Wgu[:F]).T
    u = bf16_round(n2) @ bf16_round(Wgu[F:]).T
    g = host(gu)
    scale = max(np.max(np.abs(a)), np.max(np.abs(u)))
    assert np.all(np.abs(g[:, :F] - a) <= BF16_REL * np.abs(a) + 2e-5 * scale)
    assert np.all(np.abs(g[:, F:] - u) <= BF16_REL * np.abs(u) + 2e-5 * scale)
    mref = OM.swiglu(a, u)
    assert np.all(np.abs(host(m) - mref) <= BF16_REL * np.abs(mref) + 1e-4 * np.max(np.abs(mref)))
    # backward: dm = dy Wd (NN), fused with the SwiGLU derivative, a/u from gu
    dy = random_array((T, h), seed=6)
    Wd = random_array((h, F), seed=7, std=0.05)
    dgu = torch.empty((T, 2 * F), dtype=torch.bfloat16, device=dev())
    mt.mtk_gemm(mt.MT_GEMM_NN, mt.MT_EPI_SWIGLU_BWD, T, F, h, bf16_dev(dy), h, bf16_dev(Wd), F,
                dgu, 2 * F, gu=gu, ldgu=2 * F, ffn=F)
    dm = bf16_round(dy) @ bf16_round(Wd)
    da, du = OM.swiglu_bwd(dm, g[:, :F], g[:, F:])
    got = host(dgu)
    for x, r in ((got[:, :F], da), (got[:, F:], du)):
        assert np.all(np.abs(x - r) <= BF16_REL * np.abs(r) + 1e-4 * np.max(np.abs(r)))


@pytest.mark.parametrize("T,h", [(300, 256), (77, 1024), (130, 5120), (64, 4096)])
def test_rmsnorm_forward_backward(T, h):
    print(f"rmsnorm T={T} h={h}", flush=True)
    x = random_array((T, h), seed=8, std=2.0)
    g = 1.0 + random_array((h,), seed=9, std=0.2)
    gb = bf16_round(g)
    out = torch.empty((T, h), dtype=torch.bfloat16, device=dev())
    rstd = torch.empty(T, dtype=torch.float32, device=dev())
    xd = f32_dev(x)
    gd = bf16_dev(g)
    mt.mtk_rmsnorm_fwd(xd, gd, out, rstd, T, h, 1e-5)
    n_ref, r_ref = OM.rmsnorm(x.astype(np.float64), gb, 1e-5)
    assert np.max(np.abs(host(rstd) - r_ref[:, 0]) / r_ref[:, 0]) < 2e-6
    got = host(out)
    assert np.all(np.abs(got - n_ref) <= BF16_REL * np.abs(n_ref) + 1e-6)
    dn = random_array((T, h), seed=10)
    resid = random_array((T, h), seed=11)
    dx = torch.empty((T, h), dtype=torch.float32, device=dev())
    dxb = torch.empty((T, h), dtype=torch.bfloat16, device=dev())
    dg = torch.empty(h, dtype=torch.float32, device=dev())
    ws = torch.empty(mt.mtk_rmsnorm_bwd_workspace(T, h), dtype=torch.uint8, device=dev())
    mt.mtk_rmsnorm_bwd(f32_dev(dn), xd, rstd, gd, f32_dev(resid), dx, dxb, dg, ws, T, h)
    dx_ref, dg_ref = OM.rmsnorm_bwd(dn.astype(np.float64), x.astype(np.float64), r_ref, gb)
    assert rel_max(host(dx), dx_ref + resid) < 1e-5
    assert rel_max(host(dg), dg_ref) < 1e-5
    assert np.all(np.abs(host(dxb) - (dx_ref + resid)) <= BF16_REL * np.abs(dx_ref + resid) + 1e-5)


@pytest.mark.parametrize("b,s,nq,nkv,d", [(2, 128, 4, 2, 64), (1, 256, 5, 1, 128),
                                         (2, 128, 2, 2, 16),   # eight-pair kernel, one thread per head
                                         (1, 128, 3, 1, 24)])  # d not a multiple of 16: one pair per thread
def test_rope_forward_inverse(b, s, nq, nkv, d):
    T = b * s
    W = (nq + 2 * nkv) * d
    x = random_array((T, W), seed=12)
    cos, sin = mt.mt_host_rope_table(s, d, 10000.0)
    qkv = bf16_dev(x)
    mt.mtk_rope(qkv, T, s, nq, nkv, d, f32_dev(cos), f32_dev(sin), 0)
    got = host(qkv)
    xb = bf16_round(x)
    qk = xb[:, :(nq + nkv) * d].reshape(b, s, nq + nkv, d)
    ref = OM.rope(qk, cos.astype(np.float64), sin.astype(np.float64)).reshape(T, -1)
    assert np.all(np.abs(got[:, :(nq + nkv) * d] - ref) <= BF16_REL * np.abs(ref) + 1e-6)
    np.testing.assert_array_equal(got[:, (nq + nkv) * d:], xb[:, (nq + nkv) * d:])
    mt.mtk_rope(qkv, T, s, nq, nkv, d, f32_dev(cos), f32_dev(sin), 1)
    back = host(qkv)
    assert rel_max(back, xb) < 2e-2


# (T, seq, nq, nkv, d, K): the fused QKV projection with RoPE in the epilogue.
# The first two run on 128 x 128 tiles, the others on 256 x 256 direct-to-LDS
# tiles (the last with a ragged row tail and T not a multiple of the sequence).
@pytest.mark.parametrize("T,s,nq,nkv,d,K", [(256, 128, 4, 2, 64, 256), (384, 384, 10, 2, 128, 392),
                                            (4096, 2048, 8, 8, 128, 256),
                                            (4104, 1024, 16, 4, 64, 384)])
def test_gemm_rope_epilogue(T, s, nq, nkv, d, K):
    print(f"gemm rope T={T} s={s} nq={nq} nkv={nkv} d={d} K={K}", flush=True)
    N = (nq + 2 * nkv) * d
    A = random_array((T, K), seed=21)
    B = random_array((N, K), seed=22, std=0.05)
    cos, sin = mt.mt_host_rope_table(s, d, 10000.0)
    out = torch.empty((T, N), dtype=torch.bfloat16, device=dev())
    mt.mtk_gemm(mt.MT_GEMM_NT, mt.MT_EPI_ROPE, T, N, K, bf16_dev(A), K, bf16_dev(B), K, out, N,
                rope_cos=f32_dev(cos), rope_sin=f32_dev(sin), rope_cols=(nq + nkv) * d,
                rope_seq=s, rope_dim=d)
    y = bf16_round(A) @ bf16_round(B).T          # the projection, float64
    pos = np.arange(T) % s
    ref = y.copy()
    qk = y[:, :(nq + nkv) * d].reshape(1, T, nq + nkv, d)
    ref[:, :(nq + nkv) * d] = OM.rope(qk, cos[pos].astype(np.float64),
                                      sin[pos].astype(np.float64)).reshape(T, -1)
    got = host(out)
    # one rounding of the fp32 result (the rotation adds fp32 error only)
    assert np.all(np.abs(got - ref) <= BF16_REL * np.abs(ref) + 3e-5 * np.max(np.abs(ref)))


ATTN_CASES = [(2, 256, 4, 2, 64), (1, 384, 4, 4, 128), (1, 256, 10, 2, 128), (2, 128, 16, 16, 64)]


def _attn_inputs(b, s, nq, nkv, d, seed):
    T = b * s
    qkv = random_array((T, (nq + 2 * nkv) * d), seed=seed)
    xb = bf16_round(qkv)
    q = xb[:, :nq * d].reshape(b, s, nq, d)
    k = xb[:, nq * d:(nq + nkv) * d].reshape(b, s, nkv, d)
    v = xb[:, (nq + nkv) * d:].reshape(b, s, nkv, d)
    return qkv, q, k, v


@pytest.mark.parametrize("b,s,nq,nkv,d", ATTN_CASES)
def test_attention_forward(b, s, nq, nkv, d):
    print(f"attn fwd b={b} s={s} nq={nq} nkv={nkv} d={d}", flush=True)
    T = b * s
    qkv, q, k, v = _attn_inputs(b, s, nq, nkv, d, 13)
    o = torch.empty((T, nq * d), dtype=torch.bfloat16, device=dev())
    lse = torch.empty((nq, T), dtype=torch.float32, device=dev())
    mt.mtk_attention_fwd(bf16_dev(qkv), o, lse, b, s, nq, nkv, d)
    ref = OM.attention(q, k, v).reshape(T, nq * d)
    assert rel_max(host(o), ref) < 1e-2
    lref = OM.attention_lse(q, k).reshape(T, nq).T
    assert np.max(np.abs(host(lse) - lref)) < 2e-3


@pytest.mark.parametrize("b,s,nq,nkv,d", ATTN_CASES)
def test_attention_backward(b, s, nq, nkv, d):
    print(f"attn bwd b={b} s={s} nq={nq} nkv={nkv} d={d}", flush=True)
    T = b * s
    qkv, q, k, v = _attn_inputs(b, s, nq, nkv, d, 14)
    dO = random_array((T, nq * d), seed=15)
    qd = bf16_dev(qkv)
    o = torch.empty((T, nq * d), dtype=torch.bfloat16, device=dev())
    lse = torch.empty((nq, T), dtype=torch.float32, device=dev())
    mt.mtk_attention_fwd(qd, o, lse, b, s, nq, nkv, d)
    dq = torch.zeros((T, (nq + 2 * nkv) * d), dtype=torch.bfloat16, device=dev())
    ws = torch.empty(mt.mtk_attention_bwd_workspace(b, s, nq, nkv, d), dtype=torch.uint8,
                     device=dev())
    mt.mtk_attention_bwd(qd, o, bf16_dev(dO), lse, ws, dq, b, s, nq, nkv, d)
    rq, rk, rv = OM.attention_bwd(q, k, v, bf16_round(dO).reshape(b, s, nq, d))
    got = host(dq)
    assert rel_max(got[:, :nq * d], rq.reshape(T, -1)) < 2e-2
    assert rel_max(got[:, nq * d:(nq + nkv) * d], rk.reshape(T, -1)) < 2e-2
    assert rel_max(got[:, (nq + nkv) * d:], rv.reshape(T, -1)) < 2e-2


@pytest.mark.parametrize("b,s,nq,nkv,d", ATTN_CASES)
def test_attention_backward_rope(b, s, nq, nkv, d):
    """dq and dk leave the kernels rotated back to the pre-RoPE q and k."""
    print(f"attn bwd rope b={b} s={s} nq={nq} nkv={nkv} d={d}", flush=True)
    T = b * s
    qkv, q, k, v = _attn_inputs(b, s, nq, nkv, d, 24)
    dO = random_array((T, nq * d), seed=25)
    qd = bf16_dev(qkv)
    o = torch.empty((T, nq * d), dtype=torch.bfloat16, device=dev())
    lse = torch.empty((nq, T), dtype=torch.float32, device=dev())
    mt.mtk_attention_fwd(qd, o, lse, b, s, nq, nkv, d)
    cos, sin = mt.mt_host_rope_table(s, d, 10000.0)
    dq = torch.zeros((T, (nq + 2 * nkv) * d), dtype=torch.bfloat16, device=dev())
    ws = torch.empty(mt.mtk_attention_bwd_workspace(b, s, nq, nkv, d), dtype=torch.uint8,
                     device=dev())
    mt.mtk_attention_bwd_rope(qd, o, bf16_dev(dO), lse, ws, dq, b, s, nq, nkv, d, f32_dev(cos),
                              f32_dev(sin))
    rq, rk, rv = OM.attention_bwd(q, k, v, bf16_round(dO).reshape(b, s, nq, d))
    c64, s64 = cos.astype(np.float64), sin.astype(np.float64)
    rq = OM.rope(rq, c64, s64, inverse=True)
    rk = OM.rope(rk, c64, s64, inverse=True)
    got = host(dq)
    assert rel_max(got[:, :nq * d], rq.reshape(T, -1)) < 2e-2
    assert rel_max(got[:, nq * d:(nq + nkv) * d], rk.reshape(T, -1)) < 2e-2
    assert rel_max(got[:, (nq + nkv) * d:], rv.reshape(T, -1)) < 2e-2


@pytest.mark.parametrize("T,V", [(300, 1024), (64, 32000)])
def test_cross_entropy(T, V):
    logits = random_array((T, V), seed=16, std=3.0)
    rng = np.random.default_rng(17)
    labels = rng.integers(0, V, size=T).astype(np.int32)
    labels[::7] = -1
    nv = int((labels >= 0).sum())
    dl = torch.empty((T, V), dtype=torch.bfloat16, device=dev())
    rows = torch.empty(T, dtype=torch.float32, device=dev())
    loss = torch.empty(1, dtype=torch.float32, device=dev())
    lab_d = torch.from_numpy(labels).to(dev())
    mt.mtk_cross_entropy(f32_dev(logits), V, lab_d, T, V, 0.5, nv, dl, V, rows, loss)
    ref_loss, ref_dl, _ = OM.cross_entropy(logits.astype(np.float64), labels, 0.5)
    assert abs(host(loss)[0] - ref_loss) < 1e-5 * abs(ref_loss)
    got = host(dl)
    assert np.all(np.abs(got - ref_dl) <= BF16_REL * np.abs(ref_dl) + 1e-9)
    assert np.all(got[labels < 0] == 0)
