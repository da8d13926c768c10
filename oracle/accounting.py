"""Byte accounting of the host-resident state (oracle).

zhichai intro and lqnn 一 put the persistent state of mixed-precision Adam
training at about 12 bytes per parameter (bf16 weight + bf16 grad + fp32
m and v); travelaiplan 核心功能 1 sizes full-precision training at
"parameters x 4 bytes x about 4" (fp32 master, grad, m, v = 16 bytes per
parameter, lqnn 二); lqnn 一 gives 2 bytes per parameter for bf16 weights.
The method keeps the 16 B/param fp32 state on the host plus a 2 B/param
pinned bf16 working copy that is streamed to the GPU (lqnn 三.1).
"""
from __future__ import annotations

from . import layout as L

FP32_STATE_BYTES_PER_PARAM = 4 * 4      # master, grad, m, v
BF16_WORKING_BYTES_PER_PARAM = 2        # pinned streamed copy
MIXED_STATE_BYTES_PER_PARAM = 2 + 2 + 4 + 4


def host_state_bytes(n_params: int) -> int:
    return FP32_STATE_BYTES_PER_PARAM * n_params


def pinned_working_bytes(n_params: int) -> int:
    return BF16_WORKING_BYTES_PER_PARAM * n_params


def flat_elements(cfg) -> int:
    """Elements of all flat groups (padding included)."""
    return sum(L.group_layout(cfg, g)[1] for g in [L.EMBED] + list(range(cfg.n_layers)) + [L.HEAD])
