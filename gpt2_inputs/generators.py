"""Seeded generators: initial parameters and synthetic token streams.

Everything is drawn with numpy's PCG64 so that the oracle and the GPU path
receive the very same arrays.  No arithmetic of the training step lives here.
"""

from __future__ import annotations

import math
from collections import OrderedDict

import numpy as np

from .configs import ModelShape, param_shapes

INIT_STD = 0.02
_RESIDUAL_PROJECTIONS = ("proj_w", "fcproj_w")
_ONES = ("ln1_w", "ln2_w", "lnf_w")


def init_params(s: ModelShape, seed: int = 0) -> "OrderedDict[str, np.ndarray]":
    """fp32 parameters in canonical order.

    Weight matrices, wte and wpe ~ N(0, 0.02); the two residual projections of
    every block (attention output and MLP output) ~ N(0, 0.02 / sqrt(2 L));
    biases 0; LayerNorm gains 1 and shifts 0 (AxonLM README, "Key Features").
    Draws happen in canonical order from one PCG64 stream.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = OrderedDict()
    resid_std = INIT_STD / math.sqrt(2.0 * s.n_layer)
    for name, shp in param_shapes(s).items():
        if name.endswith("_b"):
            out[name] = np.zeros(shp, np.float32)
        elif name in _ONES:
            out[name] = np.ones(shp, np.float32)
        else:
            std = resid_std if name in _RESIDUAL_PROJECTIONS else INIT_STD
            a = rng.standard_normal(shp, dtype=np.float32)
            a *= np.float32(std)
            out[name] = a
    return out


def uniform_tokens(n: int, vocab: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def zipf_probabilities(vocab: int, s: float = 1.1) -> np.ndarray:
    """P(id = r) proportional to (r + 1)^-s on [0, vocab) (rank = id)."""
    w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    return w / w.sum()


def zipf_tokens(n: int, vocab: int, seed: int, s: float = 1.1) -> np.ndarray:
    """Inverse-CDF draws from the finite Zipf law on [0, vocab)."""
    cdf = np.cumsum(zipf_probabilities(vocab, s))
    rng = np.random.Generator(np.random.PCG64(seed))
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="left")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def token_stream(kind: str, n: int, vocab: int, seed: int, zipf_s: float = 1.1) -> np.ndarray:
    if kind == "uniform":
        return uniform_tokens(n, vocab, seed)
    if kind == "zipf":
        return zipf_tokens(n, vocab, seed, zipf_s)
    raise ValueError(f"unknown token distribution {kind!r}")


def micro_batches(stream: np.ndarray, k: int, B: int, T: int):
    """k consecutive (x, y) windows of shape (B, T); y is x shifted by one."""
    need = k * B * T + 1
    if stream.shape[0] < need:
        raise ValueError(f"stream of {stream.shape[0]} ids is too short for {k}x{B}x{T}")
    out = []
    for i in range(k):
        lo = i * B * T
        x = stream[lo:lo + B * T].reshape(B, T).copy()
        y = stream[lo + 1:lo + B * T + 1].reshape(B, T).copy()
        out.append((x, y))
    return out
