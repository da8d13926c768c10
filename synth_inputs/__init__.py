"""Seeded synthetic inputs for the layer-streamed training step.

This module is shared by the CPU oracle (``oracle/``) and the HIP path
(``host_memory_centric_stateless_amd``).  It holds no arithmetic of the
training method: it only names the model shapes, draws random numbers in a
fixed order and derives next-token labels from drawn token ids.

Shapes follow the five Llama-style decoder configurations the method is
measured on (tiny 2-layer, small 8-layer, 7B-shaped, 14B-shaped GQA and the
131,072-token long-context 7B-shaped stack).  The pages publish no dataset
for this path, so uniform random token ids stand in for training text.

Draw order (fixed, part of the recipe): one ``numpy.random.default_rng(seed)``
stream; groups in the order embedding, decoder layers 0..L-1, head; inside a
group the tensors in the order listed by :func:`tensor_specs`.  Every matrix is
``standard_normal(numel, float32) * 0.02``; RMSNorm gains are 1.0 and draw
nothing.  Token ids for optimizer step ``k`` come from ``default_rng(1000 + k)``
as ``integers(0, vocab, size=(grad_accum, micro_batch, seq_len), int32)``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterator, List, Tuple

import numpy as np

GROUP_EMBED = -1
GROUP_HEAD = -2


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    micro_batch: int
    seq_len: int
    grad_accum: int = 1
    ckpt_interval: int = 4
    n_grad_slabs: int = 12
    rms_eps: float = 1e-5
    rope_base: float = 10000.0
    lr: float = 1e-3
    steps: int = 3
    # mixture-of-experts blocks (a second parameter-structure group): block l is
    # an MoE block when n_experts > 0 and l % moe_every == moe_every - 1
    n_experts: int = 0
    top_k: int = 2
    expert_ffn: int = 0
    moe_every: int = 1

    def is_moe(self, layer: int) -> bool:
        return self.n_experts > 0 and layer % self.moe_every == self.moe_every - 1

    @property
    def tokens_per_microbatch(self) -> int:
        return self.micro_batch * self.seq_len

    def replace(self, **kw) -> "ModelConfig":
        return dataclasses.replace(self, **kw)


PRESETS: Dict[str, ModelConfig] = {
    # tiny: 2 layers, hidden 256, 4 heads of 64, FFN 688, vocab 1024, 2 x 128 tokens, K = 1
    "C1": ModelConfig("tiny-2L-h256", 2, 256, 4, 4, 64, 688, 1024, 2, 128,
                      grad_accum=1, ckpt_interval=1),
    # small: 8 layers, hidden 1024, 16 heads of 64, FFN 2816, vocab 32000, 4 x 2048 tokens
    "C2": ModelConfig("small-8L-h1024", 8, 1024, 16, 16, 64, 2816, 32000, 4, 2048,
                      grad_accum=1, ckpt_interval=4),
    # 7B-shaped: 32 layers, hidden 4096, 32 heads of 128, FFN 11008, vocab 32000, 1 x 4096, acc 4
    "C3": ModelConfig("llama-7B-shape", 32, 4096, 32, 32, 128, 11008, 32000, 1, 4096,
                      grad_accum=4, ckpt_interval=4),
    # 14B-shaped GQA: 48 layers, hidden 5120, 40 q / 8 kv heads of 128, FFN 13824, vocab 152064
    "C4": ModelConfig("gqa-14B-shape", 48, 5120, 40, 8, 128, 13824, 152064, 1, 4096,
                      grad_accum=1, ckpt_interval=4),
    # long context: 4 layers of the 7B shape, 1 x 131072 tokens, causal
    "C5": ModelConfig("llama-7B-shape-4L-s131072", 4, 4096, 32, 32, 128, 11008, 32000, 1, 131072,
                      grad_accum=1, ckpt_interval=4),
    # the pages' long-context claim (a 7B model at 512K tokens on one GPU): 4 layers of the 7B
    # shape on one sequence of 524,288 tokens, a checkpoint before every layer
    "C6": ModelConfig("llama-7B-shape-4L-s524288", 4, 4096, 32, 32, 128, 11008, 32000, 1, 524288,
                      grad_accum=1, ckpt_interval=1),
}

# Tiny GQA shape used for finite-difference checks of the oracle.
FD_TINY = ModelConfig("fd-tiny-gqa", 2, 16, 4, 2, 4, 24, 32, 2, 8, grad_accum=1, ckpt_interval=1)
# The same with its second block a mixture of 4 experts (top 2) of width 12.
FD_TINY_MOE = FD_TINY.replace(name="fd-tiny-moe", n_experts=4, top_k=2, expert_ffn=12, moe_every=2)

# Mixture-of-experts shapes (the pages' second structure group): the tiny
# decoder with every second block an MoE of 8 experts (top 2, expert width
# 256), and a small one at hidden 1024.
MOE_PRESETS: Dict[str, ModelConfig] = {
    "M1": PRESETS["C1"].replace(name="tiny-moe-2L-h256-e8", n_experts=8, top_k=2, expert_ffn=256,
                                moe_every=2),
    "M2": PRESETS["C2"].replace(name="small-moe-4L-h1024-e8", n_layers=4, micro_batch=2,
                                n_experts=8, top_k=2, expert_ffn=1408, moe_every=2,
                                ckpt_interval=2),
    # 7B-shaped attention with every second block a mixture of 8 experts (top 2) of width
    # 2816 (about a quarter of the dense FFN, a multiple of 128), 8 layers, 2 x 4096 tokens
    # per micro-batch
    "M3": PRESETS["C3"].replace(name="moe-7B-shape-8L-e8", n_layers=8, micro_batch=2,
                                grad_accum=1, n_experts=8, top_k=2, expert_ffn=2816,
                                moe_every=2, ckpt_interval=4),
}


def tensor_specs(cfg: ModelConfig, group: int) -> List[Tuple[str, Tuple[int, ...], str]]:
    """(name, shape, kind) of every tensor of a parameter group, in draw order.

    kind is ``"gain"`` (RMSNorm gain, initialised to 1) or ``"matrix"``
    (drawn N(0, 0.02)).  Matrices are [out, in].
    """
    h, F, V = cfg.hidden, cfg.ffn, cfg.vocab
    qd = cfg.n_heads * cfg.head_dim
    kvd = cfg.n_kv_heads * cfg.head_dim
    if group == GROUP_EMBED:
        return [("emb", (V, h), "matrix")]
    if group == GROUP_HEAD:
        return [("final_norm", (h,), "gain"), ("w_head", (V, h), "matrix")]
    if not 0 <= group < cfg.n_layers:
        raise ValueError(f"group {group} out of range")
    if cfg.is_moe(group):
        E, Fe = cfg.n_experts, cfg.expert_ffn
        return [
            ("attn_norm", (h,), "gain"),
            ("wq", (qd, h), "matrix"),
            ("wk", (kvd, h), "matrix"),
            ("wv", (kvd, h), "matrix"),
            ("wo", (h, qd), "matrix"),
            ("mlp_norm", (h,), "gain"),
            ("w_router", (E, h), "matrix"),
            ("w_gu", (E * 2 * Fe, h), "matrix"),   # expert e: gate rows, then up rows
            ("w_down", (E * h, Fe), "matrix"),     # expert e: rows e*h .. e*h + h - 1
        ]
    return [
        ("attn_norm", (h,), "gain"),
        ("wq", (qd, h), "matrix"),
        ("wk", (kvd, h), "matrix"),
        ("wv", (kvd, h), "matrix"),
        ("wo", (h, qd), "matrix"),
        ("mlp_norm", (h,), "gain"),
        ("w_gate", (F, h), "matrix"),
        ("w_up", (F, h), "matrix"),
        ("w_down", (h, F), "matrix"),
    ]


def group_order(cfg: ModelConfig) -> List[int]:
    return [GROUP_EMBED] + list(range(cfg.n_layers)) + [GROUP_HEAD]


def weight_stream(cfg: ModelConfig, seed: int = 0, std: float = 0.02
                  ) -> Iterator[Tuple[int, str, np.ndarray]]:
    """Yield (group, name, fp32 array) for every tensor, in draw order.

    Consumers copy each array into their own storage and drop it, so the
    whole model never has to exist twice in host memory.
    """
    rng = np.random.default_rng(seed)
    for g in group_order(cfg):
        for name, shape, kind in tensor_specs(cfg, g):
            if kind == "gain":
                arr = np.ones(shape, dtype=np.float32)
            else:
                n = int(np.prod(shape))
                arr = rng.standard_normal(n, dtype=np.float32)
                arr *= np.float32(std)
                arr = arr.reshape(shape)
            yield g, name, arr


def make_weights(cfg: ModelConfig, seed: int = 0) -> Dict[int, Dict[str, np.ndarray]]:
    """All weights as {group: {name: array}} (small configurations only)."""
    out: Dict[int, Dict[str, np.ndarray]] = {}
    for g, name, arr in weight_stream(cfg, seed):
        out.setdefault(g, {})[name] = arr
    return out


def make_batch(cfg: ModelConfig, step: int) -> Tuple[np.ndarray, np.ndarray]:
    """Token ids and next-token labels for optimizer step ``step`` (1-based).

    Returns (tokens, labels), both int32 of shape (grad_accum, micro_batch,
    seq_len).  ``labels[..., t] = tokens[..., t + 1]`` and the last position of
    every sequence is -1 (ignored).
    """
    rng = np.random.default_rng(1000 + step)
    tok = rng.integers(0, cfg.vocab, size=(cfg.grad_accum, cfg.micro_batch, cfg.seq_len),
                       dtype=np.int32)
    lab = np.full_like(tok, -1)
    lab[..., :-1] = tok[..., 1:]
    return tok, lab


def random_array(shape, seed: int, std: float = 1.0, dtype=np.float32) -> np.ndarray:
    """Seeded N(0, std^2) array for per-kernel parity inputs."""
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape)) if len(shape) else 1
    return (rng.standard_normal(n, dtype=np.float32) * np.float32(std)).reshape(shape).astype(dtype)
