"""Seeded synthetic inputs for the online-quantized W8A8 / W4A8 linear layer.

This module only draws random numbers and casts them to fp16. It holds none of
the method's arithmetic (no quantization, no matmul, no dequant), so both the
HIP path and the CPU oracle may be fed from it without sharing any of the
method's code.

The shapes follow the single-op latency tables of the Cider README (section
"性能 (Apple M5 Pro) / 单算子延迟": [N=10240, K=2560] and [N=2560, K=10240],
M from 1 to 8192) and the Qwen3-VL-2B prefill linear layers of its end-to-end
VLM table. No model weights or activation traces are available, so these
stand in for them:

* x: standard normal fp32, with round(1% of K) channels (the same channels for
  every row) multiplied by 20 in fp32 to mimic activation outliers (the
  README's notes section warns that outliers are what breaks min-max W8A8),
  then cast once to fp16 (round-to-nearest-even).
* W: 0.02 * standard normal fp32, cast once to fp16.

Random streams: numpy PCG64 fed by SeedSequence(seed).spawn(3), giving one
stream each for the x values, the outlier-channel choice and the W values.
W therefore does not depend on M, so an M sweep shares its weights.
"""
from __future__ import annotations

import numpy as np

__all__ = ["streams", "n_outliers", "outlier_channels", "activations", "weights",
           "stack_layer_shapes", "stack_weight_seed"]


def streams(seed: int = 0):
    """Three independent PCG64 generators: (x values, outlier choice, W values)."""
    children = np.random.SeedSequence(seed).spawn(3)
    return [np.random.Generator(np.random.PCG64(c)) for c in children]


def n_outliers(K: int, frac: float = 0.01) -> int:
    """Number of outlier channels: round(frac*K), Python's round (ties to even)."""
    return int(round(frac * K))


def outlier_channels(K: int, seed: int = 0, frac: float = 0.01) -> np.ndarray:
    _, g_o, _ = streams(seed)
    return np.sort(g_o.permutation(K)[: n_outliers(K, frac)])


def activations(M: int, K: int, seed: int = 0, frac: float = 0.01,
                gain: float = 20.0) -> np.ndarray:
    """fp16 [M, K] activations, N(0,1) with round(frac*K) outlier channels x gain."""
    g_x, _, _ = streams(seed)
    x = g_x.standard_normal((M, K), dtype=np.float32)
    cols = outlier_channels(K, seed, frac)
    x[:, cols] *= np.float32(gain)
    return x.astype(np.float16)


def weights(N: int, K: int, seed: int = 0, std: float = 0.02) -> np.ndarray:
    """fp16 [N, K] weights (row = output channel, K contiguous), N(0, std)."""
    _, _, g_w = streams(seed)
    w = g_w.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(std)
    return w.astype(np.float16)


# Qwen3-VL-2B-shaped prefill linear stack (hidden 2048, MLP 6144, GQA with
# 16 query heads and 8 KV heads of width 128): (name, out_features, in_features).
_STACK = (("q", 2048, 2048), ("k", 1024, 2048), ("v", 1024, 2048),
          ("o", 2048, 2048), ("gate", 6144, 2048), ("up", 6144, 2048),
          ("down", 2048, 6144))


def stack_layer_shapes():
    """The seven projections of one decoder layer as (name, N, K)."""
    return _STACK


def stack_weight_seed(layer: int, name: str) -> int:
    """Seed for the weight of one projection of one layer (distinct per matrix)."""
    idx = [s[0] for s in _STACK].index(name)
    return 1000 + 7 * layer + idx
