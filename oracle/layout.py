"""Flat per-group parameter layout (oracle's own implementation).

Method: every layer's weights live as one pre-flattened array so that a
single copy moves a whole layer (lqnn, 三.1 "layer_pinned_flats" and the two
fixed-size flat GPU buffers; zhichai, 性能与能力: flat tensor layout keeps
host memory linear in the parameter count).

Reading of the layout (the pages give no element order): tensors of a group
follow the block's data flow -- attn_norm, wq, wk, wv, wo, mlp_norm, w_gate,
w_up, w_down; the head group is final_norm, w_head; the embedding group is
emb.  A mixture-of-experts block (its own structure group, lqnn 四: layers are
grouped by parameter structure, MoE layers forming their own group) holds
attn_norm .. mlp_norm, then w_router [E, h], w_gu [E * 2F_e, h] (expert e's
gate rows, then its up rows) and w_down [E * h, F_e] (expert e's [h, F_e]).
Matrices are row-major [out, in].  Every tensor starts at a multiple of
256 elements and the flat length is rounded up to 256, so fp32 host arrays,
bf16 working copies and fp32 gradient slabs share one set of element offsets.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np

ALIGN = 256
EMBED = -1
HEAD = -2


def _round_up(n: int, a: int = ALIGN) -> int:
    return (n + a - 1) // a * a


def group_shapes(cfg, group: int) -> List[Tuple[str, Tuple[int, ...]]]:
    h, F, V = cfg.hidden, cfg.ffn, cfg.vocab
    qd = cfg.n_heads * cfg.head_dim
    kvd = cfg.n_kv_heads * cfg.head_dim
    if group == EMBED:
        return [("emb", (V, h))]
    if group == HEAD:
        return [("final_norm", (h,)), ("w_head", (V, h))]
    assert 0 <= group < cfg.n_layers
    if getattr(cfg, "n_experts", 0) > 0 and group % cfg.moe_every == cfg.moe_every - 1:
        # a mixture-of-experts block: its own parameter structure (lqnn 四)
        E, Fe = cfg.n_experts, cfg.expert_ffn
        return [("attn_norm", (h,)), ("wq", (qd, h)), ("wk", (kvd, h)), ("wv", (kvd, h)),
                ("wo", (h, qd)), ("mlp_norm", (h,)), ("w_router", (E, h)),
                ("w_gu", (E * 2 * Fe, h)), ("w_down", (E * h, Fe))]
    return [("attn_norm", (h,)), ("wq", (qd, h)), ("wk", (kvd, h)), ("wv", (kvd, h)),
            ("wo", (h, qd)), ("mlp_norm", (h,)), ("w_gate", (F, h)), ("w_up", (F, h)),
            ("w_down", (h, F))]


def group_layout(cfg, group: int) -> Tuple[List[Tuple[str, Tuple[int, ...], int, int]], int]:
    """[(name, shape, offset, numel)], flat_numel."""
    out = []
    off = 0
    for name, shape in group_shapes(cfg, group):
        off = _round_up(off)
        n = int(np.prod(shape))
        out.append((name, shape, off, n))
        off += n
    return out, _round_up(off)


def pack(cfg, group: int, tensors: Dict[str, np.ndarray], dtype=np.float32) -> np.ndarray:
    entries, total = group_layout(cfg, group)
    flat = np.zeros(total, dtype=dtype)
    for name, shape, off, n in entries:
        a = np.asarray(tensors[name])
        assert a.shape == tuple(shape), (name, a.shape, shape)
        flat[off:off + n] = a.reshape(-1)
    return flat


def unpack(cfg, group: int, flat: np.ndarray) -> Dict[str, np.ndarray]:
    """Views of the tensors inside ``flat`` (no copy)."""
    entries, total = group_layout(cfg, group)
    assert flat.shape == (total,), (flat.shape, total)
    return {name: flat[off:off + n].reshape(shape) for name, shape, off, n in entries}


def param_count(cfg) -> int:
    """Parameters of the model (padding excluded)."""
    n = 0
    for g in [EMBED] + list(range(cfg.n_layers)) + [HEAD]:
        for _, shape in group_shapes(cfg, g):
            n += int(np.prod(shape))
    return n
