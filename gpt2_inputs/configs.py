"""Model shapes and run settings of the GPT-2 workloads.

The shapes are the four GPT-2 scales of the AxonLM README ("Model Scales")
and the char-level toy of "GPT From Scratch" ("Problem": 4 layers, 4 heads,
128 dims, block 64, 65 characters).  Run settings (micro-batch, accumulation
steps, precision) describe synthetic workloads at those scales.

Tensor names and shapes per block follow the GPT-2 pre-LN decoder: LayerNorm,
fused QKV projection (3C x C, with bias), attention output projection
(C x C), LayerNorm, MLP C -> 4C -> C, all with biases; final LayerNorm; the
lm_head is tied to wte and adds no tensor.  Per-block tensors are stacked with
a leading layer axis.
"""

from __future__ import annotations

from collections import OrderedDict
from dataclasses import dataclass, field


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layer: int
    n_head: int
    n_embd: int
    block_size: int
    vocab_size: int          # ids and targets lie in [0, vocab_size)
    padded_vocab_size: int   # rows of wte and width of the softmax
    tied: bool = True        # lm_head is wte (False: its own (Vp, C) tensor "lm_head")
    qkv_bias: bool = True    # the QKV projection has a bias

    @property
    def head_dim(self) -> int:
        return self.n_embd // self.n_head


@dataclass(frozen=True)
class RunConfig:
    name: str
    shape: ModelShape
    micro_batch: int
    grad_accum: int
    seq_len: int
    precision: str            # "fp32", "bf16" or "fp16"
    tokens: str               # "uniform" or "zipf"
    lr: float
    weight_decay: float = 0.1
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    max_norm: float = 1.0
    zipf_s: float = 1.1
    seed_weights: int = 0
    seed_tokens: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def tokens_per_step(self) -> int:
        return self.micro_batch * self.grad_accum * self.seq_len


SHAPES = {
    "toy": ModelShape("toy", 4, 4, 128, 64, 65, 65),
    "gpt2-124m": ModelShape("gpt2-124m", 12, 12, 768, 1024, 50257, 50304),
    "gpt2-355m": ModelShape("gpt2-355m", 24, 16, 1024, 1024, 50257, 50304),
    "gpt2-774m": ModelShape("gpt2-774m", 36, 20, 1280, 1024, 50257, 50304),
    "gpt2-1558m": ModelShape("gpt2-1558m", 48, 25, 1600, 1024, 50257, 50304),
    # the untied variant of Genesis ("Model Specs": 163,009,536 parameters at
    # vocab 50,257; its own lm_head and no QKV bias), vocabulary padded
    "genesis-163m": ModelShape("genesis-163m", 12, 12, 768, 1024, 50257, 50304, tied=False, qkv_bias=False),
}

RUNS = {
    "toy": RunConfig("toy", SHAPES["toy"], 4, 1, 64, "fp32", "uniform", 1e-3),
    "gpt2-124m": RunConfig("gpt2-124m", SHAPES["gpt2-124m"], 16, 4, 1024, "bf16", "zipf", 6e-4),
    "gpt2-355m": RunConfig("gpt2-355m", SHAPES["gpt2-355m"], 8, 8, 1024, "bf16", "zipf", 6e-4),
    "gpt2-774m": RunConfig("gpt2-774m", SHAPES["gpt2-774m"], 4, 8, 1024, "bf16", "zipf", 6e-4),
    "gpt2-1558m": RunConfig("gpt2-1558m", SHAPES["gpt2-1558m"], 4, 16, 1024, "bf16", "zipf", 6e-4),
    "genesis-163m": RunConfig("genesis-163m", SHAPES["genesis-163m"], 16, 4, 1024, "bf16", "zipf", 6e-4),
}

_GLOBAL_FIRST = ("wte", "wpe")
_PER_LAYER = ("ln1_w", "ln1_b", "qkv_w", "qkv_b", "proj_w", "proj_b",
              "ln2_w", "ln2_b", "fc_w", "fc_b", "fcproj_w", "fcproj_b")
_GLOBAL_LAST = ("lnf_w", "lnf_b")


def per_layer_names() -> tuple:
    return _PER_LAYER


def param_shapes(s: ModelShape) -> "OrderedDict[str, tuple]":
    """Name -> array shape, in the canonical order (per-block tensors stacked)."""
    C, L = s.n_embd, s.n_layer
    per = {
        "ln1_w": (C,), "ln1_b": (C,),
        "qkv_w": (3 * C, C), "qkv_b": (3 * C,),
        "proj_w": (C, C), "proj_b": (C,),
        "ln2_w": (C,), "ln2_b": (C,),
        "fc_w": (4 * C, C), "fc_b": (4 * C,),
        "fcproj_w": (C, 4 * C), "fcproj_b": (C,),
    }
    out = OrderedDict()
    out["wte"] = (s.padded_vocab_size, C)
    out["wpe"] = (s.block_size, C)
    for n in _PER_LAYER:
        if n == "qkv_b" and not s.qkv_bias:
            continue
        out[n] = (L,) + per[n]
    out["lnf_w"] = (C,)
    out["lnf_b"] = (C,)
    if not s.tied:
        out["lm_head"] = (s.padded_vocab_size, C)
    return out


def n_params(s: ModelShape) -> int:
    tot = 0
    for shp in param_shapes(s).values():
        k = 1
        for d in shp:
            k *= d
        tot += k
    return tot
