"""libmt on the CPU: exported symbols, layout and memory accounting, host
kernels (bf16 cast, AdamW, accumulate, RoPE table) against the oracle and
torch, and argument errors that are rejected before any HIP call."""
import ctypes as C
import math
import os
import re

import numpy as np
import pytest
import torch

import host_memory_centric_stateless_amd as mt
from oracle import layout as OL
from oracle import model as OM
from oracle.adamw import AdamWHparams, adamw_step
from synth_inputs import PRESETS

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")


def _declared():
    names = set()
    for f in os.listdir(INCLUDE):
        if f.endswith(".h"):
            src = open(os.path.join(INCLUDE, f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(mtk?_[a-z0-9_]+)\s*\(", src))
    return names


def test_every_declared_symbol_is_exported():
    declared = _declared()
    assert len(declared) >= 20
    for name in declared:
        assert hasattr(mt.lib(), name), name
    assert declared == set(mt.EXPORTED)


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_layout_matches_oracle(name):
    cfg = PRESETS[name]
    c = mt.make_config(cfg)
    for g in [OL.EMBED, 0, cfg.n_layers - 1, OL.HEAD]:
        descs, total = mt.mt_layout(c, g)
        ent, ototal = OL.group_layout(cfg, g)
        assert total == ototal
        assert [(d[0], d[1], d[2]) for d in descs] == [(e[0], e[2], e[3]) for e in ent]


@pytest.mark.parametrize("name", ["M1", "M2"])
def test_moe_layout_matches_oracle(name):
    """Both structure groups of a mixture-of-experts model: every block's
    layout (dense and MoE) equals the oracle's, and the host-state bytes
    count both."""
    from synth_inputs import MOE_PRESETS
    cfg = MOE_PRESETS[name]
    c = mt.make_config(cfg)
    for g in [OL.EMBED] + list(range(cfg.n_layers)) + [OL.HEAD]:
        descs, total = mt.mt_layout(c, g)
        ent, ototal = OL.group_layout(cfg, g)
        assert total == ototal
        assert [(d[0], d[1], d[2]) for d in descs] == [(e[0], e[2], e[3]) for e in ent]
    r = mt.mt_device_requirements(c)
    assert r.host_state == 16 * OL.param_count(cfg)
    bad = cfg.replace(n_experts=6)
    with pytest.raises(mt.MtError):
        mt.mt_device_requirements(mt.make_config(bad))


def test_layout_rejects_bad_group_and_config():
    c = mt.make_config(PRESETS["C1"])
    with pytest.raises(mt.MtError):
        mt.mt_layout(c, 2)
    bad = mt.make_config(PRESETS["C1"].replace(hidden=100))
    with pytest.raises(mt.MtError):
        mt.mt_layout(bad, 0)
    with pytest.raises(mt.MtError):
        mt.mt_device_requirements(mt.make_config(PRESETS["C1"].replace(head_dim=96)))


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_device_requirements(name):
    cfg = PRESETS[name]
    r = mt.mt_device_requirements(mt.make_config(cfg))
    assert r.host_state == 16 * OL.param_count(cfg)
    P = OL.group_layout(cfg, 0)[1]
    assert r.unit_elems >= P
    assert r.weight_buf == -(-r.unit_elems * 2 // 256) * 256
    assert r.grad_slab == -(-r.unit_elems * 2 // 256) * 256          # bf16 slabs (default)
    r32 = mt.mt_device_requirements(mt.make_config(cfg, slab_bf16=False))
    assert r32.grad_slab == -(-r.unit_elems * 4 // 256) * 256        # fp32 slabs
    # the whole vocabulary is covered by head chunks that each fit one unit
    H = OL.group_layout(cfg, OL.HEAD)[1]
    assert r.head_chunks * r.unit_elems >= H
    assert r.device_total == (2 * r.weight_buf + cfg.n_grad_slabs * r.grad_slab + r.window
                              + r.checkpoints + r.workspace)
    # device memory does not grow with depth (only the checkpoint list does)
    r2 = mt.mt_device_requirements(mt.make_config(cfg.replace(n_layers=2 * cfg.n_layers)))
    assert r2.window == r.window and r2.weight_buf == r.weight_buf
    assert r2.workspace == r.workspace


def test_requirements_published_shapes():
    r3 = mt.mt_device_requirements(mt.make_config(PRESETS["C3"]))
    r4 = mt.mt_device_requirements(mt.make_config(PRESETS["C4"]))
    assert (r3.unit_elems, r3.head_chunks) == (202_383_360, 1)
    assert (r4.unit_elems, r4.head_chunks) == (275_261_440, 3)
    assert r4.device_total < 288e9 and r3.device_total < 288e9


def test_cast_bf16_matches_torch_including_ties_and_specials():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100_003).astype(np.float32) * 10
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-42, 3.0e38, -3.3e38,
                         np.finfo(np.float32).max, np.finfo(np.float32).tiny], np.float32)
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, specials, ties, -ties])
    out = np.empty(x.size, np.uint16)
    mt.mt_host_cast_bf16(x, out, threads=3)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(out, ref)
    nan = np.array([np.nan, -np.nan], np.float32)
    o2 = np.empty(2, np.uint16)
    mt.mt_host_cast_bf16(nan, o2)
    assert np.all((o2 & 0x7F80) == 0x7F80) and np.all(o2 & 0x7F)


def test_host_adamw_matches_oracle_fp32_bitwise_and_fp64():
    rng = np.random.default_rng(1)
    n = 300_001
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    grads = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(3)]
    grads[1][::7] = 0.0
    hp = mt.mt_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    ohp = AdamWHparams(lr=1e-3)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    bf = np.empty(n, np.uint16)
    q, qm, qv = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    d, dm, dv = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        mt.mt_host_adamw(p, g, m, v, bf, hp, t, threads=4)
        adamw_step(q, g, qm, qv, t, ohp)
        adamw_step(d, g.astype(np.float64), dm, dv, t, ohp)
    np.testing.assert_array_equal(p, q)          # same fp32 arithmetic, same order
    np.testing.assert_array_equal(m, qm)
    np.testing.assert_array_equal(v, qv)
    assert np.max(np.abs(p - d) / np.maximum(np.abs(d), 1e-3)) < 1e-6
    ref = torch.from_numpy(p).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf, ref)


def test_host_accumulate():
    rng = np.random.default_rng(2)
    a = rng.standard_normal(1_000_003).astype(np.float32)
    b = rng.standard_normal(a.size).astype(np.float32)
    g = np.zeros_like(a)
    mt.mt_host_accumulate(g, a, 0, threads=5)
    np.testing.assert_array_equal(g, a)
    mt.mt_host_accumulate(g, b, 1, threads=5)
    np.testing.assert_array_equal(g, a + b)


@pytest.mark.parametrize("slab_bf16", [True, False])
@pytest.mark.parametrize("accumulate", [0, 1])
def test_host_adamw_slab_equals_accumulate_then_adamw(slab_bf16, accumulate):
    """The optimizer thread's fused pass (add the last slab, then AdamW) must
    give bit for bit what the separate accumulate and AdamW give."""
    rng = np.random.default_rng(7)
    n = 1_000_003
    master = rng.standard_normal(n).astype(np.float32) * np.float32(0.02)
    grad0 = rng.standard_normal(n).astype(np.float32) * np.float32(1e-3)
    m0 = rng.standard_normal(n).astype(np.float32) * np.float32(1e-4)
    v0 = np.abs(rng.standard_normal(n)).astype(np.float32) * np.float32(1e-7)
    g32 = rng.standard_normal(n).astype(np.float32) * np.float32(1e-3)
    slab = ((g32.view(np.uint32) + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16) \
        if slab_bf16 else g32
    slab_f32 = (slab.astype(np.uint32) << np.uint32(16)).view(np.float32) if slab_bf16 else slab
    hp = mt.mt_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    a = [x.copy() for x in (master, grad0, m0, v0)]
    bf_a = np.zeros(n, np.uint16)
    mt.mt_host_accumulate(a[1], slab_f32, accumulate, threads=3)
    mt.mt_host_adamw(a[0], a[1], a[2], a[3], bf_a, hp, 2, threads=3)
    b = [x.copy() for x in (master, grad0, m0, v0)]
    bf_b = np.zeros(n, np.uint16)
    mt.mt_host_adamw_slab(b[0], b[1], b[2], b[3], bf_b, slab, accumulate, hp, 2, threads=5)
    for x, y, name in zip(a + [bf_a], b + [bf_b], ["master", "grad", "m", "v", "bf16"]):
        np.testing.assert_array_equal(x, y, err_msg=name)


def test_host_triad_computes_and_times():
    """The host-memory bandwidth probe computes a = b + s c and reports a
    positive time; bad arguments are rejected."""
    n = 1 << 16
    rng = np.random.default_rng(3)
    b = rng.standard_normal(n, dtype=np.float32)
    c = rng.standard_normal(n, dtype=np.float32)
    a = np.empty_like(b)
    t = mt.mt_host_triad(a, b, c, 0.5, reps=2, threads=2)
    assert t > 0
    np.testing.assert_array_equal(a, b + np.float32(0.5) * c)
    with pytest.raises(mt.MtError):
        mt.mt_host_triad(a[:0], b[:0], c[:0], 0.5)

@pytest.mark.parametrize("s,d", [(128, 64), (4096, 128), (131072, 128)])
def test_rope_table_matches_oracle(s, d):
    c, sn = mt.mt_host_rope_table(s, d, 10000.0)
    oc, osn = OM.rope_tables(s, d, 10000.0, np.float32)
    # both form the angle in float64 and round once to fp32; libm pow and
    # numpy power may differ by a few float64 ulps in theta, which positions up
    # to 131072 amplify, so bound the absolute error by one fp32 ulp at 1.0
    for a, b in ((c, oc), (sn, osn)):
        assert np.max(np.abs(a - b)) <= 2.0 ** -23
        assert np.mean(a == b) > 0.9999


def test_create_rejects_bad_arena_before_any_gpu_call():
    cfg = mt.make_config(PRESETS["C1"])
    req = mt.mt_device_requirements(cfg)
    a = mt.mt_device_arena()
    with pytest.raises(mt.MtError) as e:       # null pointers
        mt.mt_create(cfg, a)
    assert e.value.status == mt.MT_E_ARG
    base = 1 << 40
    a.weight_buf[0], a.weight_buf[1] = base, base + 2 ** 30
    for i in range(PRESETS["C1"].n_grad_slabs):
        a.grad_slab[i] = base + (4 + i) * 2 ** 30
    a.window, a.checkpoints, a.workspace = base + 2 ** 35, base + 2 ** 36, base + 2 ** 37
    a.stream_prefetch, a.stream_compute, a.stream_offload = 1, 2, 2
    with pytest.raises(mt.MtError) as e:       # two streams alias
        mt.mt_create(cfg, a)
    assert e.value.status == mt.MT_E_ARG
    a.stream_offload = 3
    a.weight_buf_bytes = req.weight_buf - 256  # arena too small
    a.grad_slab_bytes, a.window_bytes = req.grad_slab, req.window
    a.checkpoints_bytes, a.workspace_bytes = req.checkpoints, req.workspace
    with pytest.raises(mt.MtError) as e:
        mt.mt_create(cfg, a)
    assert e.value.status == mt.MT_E_NOMEM


def test_kernel_entry_points_reject_bad_shapes():
    with pytest.raises(mt.MtError):
        mt.mtk_gemm(mt.MT_GEMM_NT, mt.MT_EPI_F32, 12, 16, 16, 1 << 30, 16, 1 << 30, 16, 1 << 30,
                    16, stream=0)              # M not a multiple of 8
    with pytest.raises(mt.MtError):
        mt.mtk_gemm(mt.MT_GEMM_NN, mt.MT_EPI_SWIGLU, 16, 16, 16, 1 << 30, 16, 1 << 30, 16,
                    1 << 30, 32, gu=1 << 30, ldgu=32, ffn=16, stream=0)  # SWIGLU needs NT
    with pytest.raises(mt.MtError):
        mt.mtk_attention_fwd(1 << 30, 1 << 30, 1 << 30, 1, 100, 4, 4, 64, stream=0)
    with pytest.raises(mt.MtError):
        mt.mtk_attention_fwd(1 << 30, 1 << 30, 1 << 30, 1, 128, 4, 3, 64, stream=0)
    with pytest.raises(mt.MtError):
        mt.mtk_rmsnorm_fwd(1 << 30, 1 << 30, 1 << 30, 1 << 30, 4, 6, 1e-5, stream=0)


def _kernel_metadata():
    """(name, vgpr_count, vgpr spills, scratch bytes) of every gfx950 kernel in
    the built libmt.so, read from the code objects' metadata notes."""
    import shutil
    import subprocess
    import tempfile
    llvm = "/opt/rocm/llvm/bin"
    tools = [shutil.which("objcopy"), os.path.join(llvm, "clang-offload-bundler"),
             os.path.join(llvm, "llvm-readelf")]
    if not all(t and os.path.exists(t) for t in tools):
        pytest.skip("binutils / ROCm LLVM tools not found")
    so = os.path.join(os.path.dirname(mt.__file__), "libmt.so")
    out = []
    with tempfile.TemporaryDirectory() as d:
        fb = os.path.join(d, "fatbin")
        subprocess.run([tools[0], "--dump-section", f".hip_fatbin={fb}", so, os.path.join(d, "x")],
                       check=True, capture_output=True)
        data = open(fb, "rb").read()
        magic = b"__CLANG_OFFLOAD_BUNDLE__"
        starts = [m.start() for m in re.finditer(re.escape(magic), data)]
        for n, s in enumerate(starts):
            part = os.path.join(d, f"b{n}")
            with open(part, "wb") as f:
                f.write(data[s:starts[n + 1] if n + 1 < len(starts) else len(data)])
            co = part + ".co"
            subprocess.run([tools[1], "--type=o", "--unbundle", f"--input={part}", f"--output={co}",
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950"], check=True,
                           capture_output=True)
            notes = subprocess.run([tools[2], "--notes", co], check=True, capture_output=True,
                                   text=True).stdout
            for blk in notes.split("  - .agpr_count")[1:]:
                def field(k):
                    m = re.search(r"\." + k + r":\s+(\S+)", blk)
                    return m.group(1) if m else None
                out.append((field("name"), int(field("vgpr_count")),
                            int(field("vgpr_spill_count")),
                            int(field("private_segment_fixed_size"))))
    assert out, "no kernel metadata found"
    return out


def test_kernel_register_budget():
    """Two waves per SIMD of the 256 x 256 GEMM (8 waves) and of the attention
    kernels (2 workgroups of 4 waves per CU) must leave room for one wave of
    the 4-workgroup gradient-drain copy kernel, which runs beside them for the
    whole backward: 2 x 248 + 16 <= 512 VGPRs per lane (granule 8).  Otherwise
    a product of exactly 256 tiles loses the drain's CUs and runs a second
    round.  The fused dK/dV kernel runs one wave per SIMD: 496 + 16 <= 512.
    No kernel may spill or use scratch."""
    meta = _kernel_metadata()
    names = [m[0] for m in meta]
    assert any("gemm_kernel" in n for n in names) and any("attn_fwd" in n for n in names)
    assert any("gemm_direct_kernel" in n for n in names)
    assert any("attn_bwd_dkdv" in n for n in names)
    for name, vgpr, spill, scratch in meta:
        assert spill == 0 and scratch == 0, (name, spill, scratch)
        if "attn_bwd_dkdv" in name:
            assert vgpr <= 496, (name, vgpr)
        elif ("gemm_kernel" in name and "256ELi256" in name) or "gemm_direct" in name or "attn_" in name:
            assert vgpr <= 248, (name, vgpr)
        if "copy16" in name:
            assert vgpr <= 16, (name, vgpr)


@pytest.mark.parametrize("offset", [0, 1, 3, 7])
def test_host_streamed_outputs_at_unaligned_addresses(offset):
    """The written-only outputs (the bf16 working copy, a gradient set rather
    than added to) leave through a staging block and 32-byte non-temporal
    stores with plain copies for the unaligned head and tail; at any element
    offset the result must equal the scalar definition bit for bit."""
    rng = np.random.default_rng(11)
    n = 70_001  # several staging blocks and a ragged tail
    hp = mt.mt_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01)

    def views(*arrs):  # the same values starting `offset` elements into a larger buffer
        out = []
        for a in arrs:
            big = np.zeros(a.size + offset, a.dtype)
            v = big[offset:]
            v[...] = a
            out.append(v)
        return out

    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g32 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    slab = ((g32.view(np.uint32) + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16)
    zero = np.zeros(n, np.float32)
    # reference: the aligned arrays through the same calls
    ra = [master.copy(), zero.copy(), zero.copy(), zero.copy(), np.zeros(n, np.uint16)]
    mt.mt_host_adamw_slab(*ra, slab, 0, hp, 1, threads=3)
    ua = views(master, zero, zero, zero, np.zeros(n, np.uint16))
    mt.mt_host_adamw_slab(*ua, views(slab)[0], 0, hp, 1, threads=3)
    for x, y, name in zip(ra, ua, ["master", "grad", "m", "v", "bf16"]):
        np.testing.assert_array_equal(x, y, err_msg=name)
    # the grad written by the set path is the slab value itself
    np.testing.assert_array_equal(ua[1], (slab.astype(np.uint32) << np.uint32(16)).view(np.float32))
    # the bf16 copy is the RNE rounding of the updated master
    ref = torch.from_numpy(np.ascontiguousarray(ua[0])).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ua[4], ref)
    # plain AdamW with a bf16 copy, and the fp32 set-accumulate
    rb = [master.copy(), g32.copy(), zero.copy(), zero.copy(), np.zeros(n, np.uint16)]
    mt.mt_host_adamw(*rb, hp, 1, threads=2)
    ub = views(master, g32, zero, zero, np.zeros(n, np.uint16))
    mt.mt_host_adamw(*ub, hp, 1, threads=2)
    for x, y in zip(rb, ub):
        np.testing.assert_array_equal(x, y)
    (acc,) = views(np.full(n, np.float32(7.0)))
    mt.mt_host_accumulate(acc, views(g32)[0], 0, threads=4)
    np.testing.assert_array_equal(acc, g32)


def test_default_drain_workgroups_rule():
    """Three drain workgroups only for bf16 slabs with more than one pass per
    step (the drain then trails into the next micro-batch's forward); four
    otherwise (one pass per step, or fp32 slabs with twice the bytes)."""
    c3, c2 = PRESETS["C3"], PRESETS["C2"]
    assert c3.grad_accum == 4
    assert mt.default_drain_workgroups(c3) == 3
    assert mt.default_drain_workgroups(c3, slab_bf16=False) == mt.DEFAULT_DRAIN_WORKGROUPS == 4
    assert mt.default_drain_workgroups(c3, micro_batches_per_pass=4) == 4  # one pass per step
    assert mt.default_drain_workgroups(c3, micro_batches_per_pass=2) == 3  # two passes
    assert mt.default_drain_workgroups(c3.replace(grad_accum=1)) == 4
    assert c2.grad_accum == 1 and mt.default_drain_workgroups(c2) == 4  # 4 sequences, one pass
    # the session passes the rule's value unless the caller chooses one
    cfg = mt.make_config(c3, drain_workgroups=mt.default_drain_workgroups(c3))
    assert cfg.drain_workgroups == 3
