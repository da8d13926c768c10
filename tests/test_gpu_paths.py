"""Paths of the GPU implementation that the per-config parity runs do not
reach on their own, each checked against the CPU oracle or bit for bit:

* flash attention whose scores climb by far more than the forward's lazy
  rescale slack from one key tile to the next, so the running maximum moves
  (and the output accumulator is rescaled) on most tiles;
* overlapped-optimizer steps that return without a flush, against the
  oracle's own training steps (losses, weights after three steps);
* the flat copies: the ping-pong weight buffers hold exactly the
  round-to-nearest-even bf16 copy of a streamed unit's fp32 master (lqnn 三.1:
  pinned pre-flattened per-layer copies, flat device buffers), and the slab
  drain's copy kernel moves bytes unchanged;
* device memory: a training step allocates nothing on the device beyond the
  caller's arena (zhichai design point 2: the GPU holds only the current
  layer's parameters and gradients; lqnn 三.4: transient memory of 1-2 layers
  plus a few activations).
"""
import math

import numpy as np
import pytest
import torch

import host_memory_centric_stateless_amd as mt
from oracle import model as OM
from oracle.train import HostState, train_step
from synth_inputs import PRESETS, make_batch, random_array, weight_stream
from tests.gpu_util import bf16_dev, bf16_round, dev, f32_dev, host, rel_l2, rel_max
from tests.test_gpu_step import LOSS_TOL, _session, _tensors

pytestmark = pytest.mark.gpu


# ------------------------------------------------ attention with score spikes
def _climbing_qkv(b, s, nq, nkv, d, seed, climb_nats):
    """q/k whose causal scores rise (heads of even kv index) or fall (odd) by
    about climb_nats over the sequence, plus noise: a query's maximum then
    moves on almost every 64-key tile."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    c = 8.0
    gam = climb_nats * math.sqrt(d) / c
    pos = np.arange(s, dtype=np.float64) / s
    q = 0.3 * rng.standard_normal((b, s, nq, d))
    k = 0.3 * rng.standard_normal((b, s, nkv, d))
    v = rng.standard_normal((b, s, nkv, d))
    grp = nq // nkv
    for j in range(nq):
        q[:, :, j, :] += c * u * (1.0 if (j // grp) % 2 == 0 else -1.0)
    for g in range(nkv):
        k[:, :, g, :] += gam * pos[None, :, None] * u[None, None, :]
    T = b * s
    qkv = np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], axis=1)
    xb = bf16_round(qkv.astype(np.float32))
    return (qkv.astype(np.float32), xb[:, :nq * d].reshape(b, s, nq, d),
            xb[:, nq * d:(nq + nkv) * d].reshape(b, s, nkv, d), xb[:, (nq + nkv) * d:].reshape(b, s, nkv, d))


@pytest.mark.parametrize("b,s,nq,nkv,d", [(1, 512, 4, 2, 128), (2, 384, 4, 4, 64)])
def test_attention_with_climbing_scores(b, s, nq, nkv, d):
    print(f"attn climbing scores b={b} s={s} nq={nq} nkv={nkv} d={d}", flush=True)
    T = b * s
    qkv, q, k, v = _climbing_qkv(b, s, nq, nkv, d, 31, climb_nats=80.0)
    # the rise over one 64-key tile is well above the 8 log2-unit slack
    sc = np.einsum("d,sd->s", q[0, s - 1, 0], k[0, :, 0]) / math.sqrt(d)
    assert (sc[-64:].max() - sc[-128:-64].max()) / math.log(2) > 8
    qd = bf16_dev(qkv)
    o = torch.empty((T, nq * d), dtype=torch.bfloat16, device=dev())
    lse = torch.empty((nq, T), dtype=torch.float32, device=dev())
    mt.mtk_attention_fwd(qd, o, lse, b, s, nq, nkv, d)
    ref = OM.attention(q, k, v).reshape(T, nq * d)
    assert rel_max(host(o), ref) < 1e-2
    lref = OM.attention_lse(q, k).reshape(T, nq).T
    assert np.max(np.abs(host(lse) - lref) / np.maximum(1.0, np.abs(lref))) < 2e-4
    dO = random_array((T, nq * d), seed=32)
    dq = torch.zeros((T, (nq + 2 * nkv) * d), dtype=torch.bfloat16, device=dev())
    ws = torch.empty(mt.mtk_attention_bwd_workspace(b, s, nq, nkv, d), dtype=torch.uint8,
                     device=dev())
    mt.mtk_attention_bwd(qd, o, bf16_dev(dO), lse, ws, dq, b, s, nq, nkv, d)
    dOb = bf16_round(dO).reshape(b, s, nq, d)
    ref = OM.attention_bwd(q, k, v, dOb)
    # Conditioning of the backward at these inputs: the same oracle after a
    # relative perturbation of every input by half a bf16 ulp (2^-9, random
    # sign).  With peaked probabilities and a large key component shared by
    # all keys, dq = dS k / sqrt(d) cancels heavily (the rows of dS sum to
    # zero), so any bf16 rounding of its operands moves it by about this much.
    rng = np.random.default_rng(33)
    pert = [x * (1.0 + 2.0 ** -9 * rng.choice([-1.0, 1.0], size=x.shape)) for x in (q, k, v, dOb)]
    moved = OM.attention_bwd(*pert)
    got = host(dq)
    for name, x, r, m in (("dq", got[:, :nq * d], ref[0], moved[0]),
                          ("dk", got[:, nq * d:(nq + nkv) * d], ref[1], moved[1]),
                          ("dv", got[:, (nq + nkv) * d:], ref[2], moved[2])):
        e2 = rel_l2(x, r.reshape(T, -1))
        floor = rel_l2(m.reshape(T, -1), r.reshape(T, -1))
        print(f"  {name}: rel L2 {e2:.2e} (half-ulp input perturbation moves it {floor:.2e})",
              flush=True)
        assert e2 <= max(1e-2, 2.0 * floor), name


# ----------------------------------------- overlapped steps without a flush
def test_overlapped_steps_without_flush_match_oracle():
    """Three Session.step(overlap_optimizer=True, flush=False) steps (each
    unit's AdamW runs on the host as its last slab lands, and the next forward
    waits per unit) against three oracle train_steps from the same start."""
    cfg = PRESETS["C1"].replace(grad_accum=2)
    sess = _session(cfg)
    st = HostState(cfg, np.float32)
    st.load_weights(weight_stream(cfg, 0))
    try:
        for step in (1, 2, 3):
            tok, lab = make_batch(cfg, step)
            gl = sess.step(tok, lab, step, overlap_optimizer=True, flush=False)
            ol = train_step(st, tok, lab, step)
            print(f"step {step}: loss gpu {gl:.6f} oracle {ol:.6f}", flush=True)
            assert abs(gl - ol) <= LOSS_TOL
        sess.flush()
        gw, ow = _tensors(cfg, sess.master), _tensors(cfg, st.master)
        gg, og = _tensors(cfg, sess.grad), _tensors(cfg, st.grad)
    finally:
        sess.close()
    werr = {k: rel_l2(gw[k], ow[k]) for k in ow}
    gerr = {k: rel_l2(gg[k], og[k]) for k in og}
    for k in sorted(ow):
        print("weight", k, f"{werr[k]:.2e}", "last-step grad", f"{gerr[k]:.2e}")
    # the same bound as the flushed C1 trajectory (bf16 gradient sign flips in
    # AdamW's first steps put the matrices ~5e-3 apart; a blunder ~1e-1)
    assert max(werr.values()) <= 1e-2
    # the third step's gradient is taken at weights that differ by the above,
    # and a 2^-9 relative change of the weights alone moves these gradients by
    # 1-2e-2 (the weight-copy floor of the configuration tests): only the
    # fault bound of those tests applies
    assert max(gerr.values()) <= 5e-2


# -------------------------------------------------------------- flat copies
def test_weight_buffers_hold_rne_copy_of_a_unit():
    """After a step, and after a step that streams the copies an AdamW update
    rewrote, each ping-pong buffer holds bit for bit the round-to-nearest-even
    bf16 of one streamed unit's fp32 master (torch's CPU cast, independent of
    the library's)."""
    cfg = PRESETS["C1"]
    sess = _session(cfg)
    try:
        n_unit = sess.req.unit_elems

        def candidates():
            out = {}
            for g in list(range(cfg.n_layers)) + [mt.MT_GROUP_HEAD]:
                m = torch.from_numpy(sess.master[g].copy()).to(torch.bfloat16).view(torch.int16)
                out[g] = m
            return out

        def check(tag, cands):
            torch.cuda.synchronize()
            for b, buf in enumerate(sess.wbuf):
                bits = buf[:2 * n_unit].view(torch.int16).cpu()
                hits = [g for g, m in cands.items() if torch.equal(bits[:m.numel()], m)]
                print(f"{tag}: buffer {b} holds unit(s) {hits}", flush=True)
                assert hits, f"{tag}: buffer {b} is no unit's RNE copy"

        # the buffers are filled during a step from the masters as they were
        # when it began (step 2 streams the copies step 1's AdamW rewrote)
        for step in (1, 2):
            cands = candidates()
            tok, lab = make_batch(cfg, step)
            sess.step(tok, lab, step, overlap_optimizer=(step == 2))
            check(f"after step {step}", cands)
    finally:
        sess.close()


@pytest.mark.parametrize("wgs", [1, 4, 32])
def test_copy_kernel_moves_bytes_unchanged(wgs):
    """The slab drain's copy kernel (mtk_copy) moves every byte unchanged.
    (Its host-side use, draining slabs into pinned host memory, is checked
    bit for bit against the DMA engine by the pipeline-invariant test: both
    drains give identical host gradients.)"""
    n = (5 << 20) + 48
    src = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device=dev())
    dst = torch.zeros_like(src)
    mt.mtk_copy(dst, src, n, wgs)
    back = torch.zeros_like(src)
    mt.mtk_copy(back, dst, n, wgs)
    torch.cuda.synchronize()
    assert torch.equal(dst, src) and torch.equal(back, src)


# ----------------------------------------------------------- device memory
def test_device_memory_is_the_arena():
    """A C2 step on the device uses exactly the caller's arena: torch's peak
    allocation equals the sizes mt_device_requirements gives, and the device's
    free memory does not drop during the step (the library allocates no device
    memory of its own)."""
    cfg = PRESETS["C2"]
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    sess = _session(cfg)
    try:
        r = sess.req
        parts = [r.weight_buf] * 2 + [r.grad_slab] * cfg.n_grad_slabs + \
                [r.window, r.checkpoints, r.workspace]
        arena = sum(max(int(p), 256) for p in parts)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        tok, lab = make_batch(cfg, 1)
        sess.step(tok, lab, 1)
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        peak = torch.cuda.max_memory_allocated() - base
        print(f"arena {arena / 2**30:.3f} GiB (device_total {r.device_total / 2**30:.3f}), "
              f"torch peak {peak / 2**30:.3f} GiB, free before/after step "
              f"{free0 / 2**30:.3f}/{free1 / 2**30:.3f} GiB", flush=True)
        assert r.device_total <= arena
        # torch's caching allocator may hand out a block up to ~1 MiB larger
        # than asked (it does not split off small remainders of large blocks)
        assert arena <= peak <= arena + (2 << 20) * len(parts)
        assert free0 - free1 < 64 << 20
    finally:
        sess.close()
