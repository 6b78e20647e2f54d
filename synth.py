"""Seeded synthetic inputs, shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method (no quantization, no matmul):
only random draws and the shapes of the workloads.  Both the HIP path and the
CPU oracle receive the arrays it returns.

Every tensor comes from ``numpy.random.default_rng([SEED, cfg, layer, slot, role])``
so any single tensor can be regenerated on its own.  Values are
``standard_normal(float32) * float32(sigma)``: sigma 0.02 for weights, the
head's source table and biases, 1.0 for activations.  The heavy-tailed
variant multiplies round(0.001 * numel) distinct positions (at least one) of
each activation tensor by 50.

Shapes (the page "ONNX export, quantization and the browser runtime" measures
stock GPT-2 small; its section "Quantization" counts 48 body weights and a
[768, 50257] head table; the dense model is the 3.8B dense entry at the small
end of the zero-tvm page's model roster, whose tokenizer is Phi-3's, with
Phi-3-mini widths):
  * GPT-2 small body: 12 layers x (768x2304 QKV, 768x768 out, 768x3072 fc,
    3072x768 proj), with biases;
  * 3.8B dense body: 32 layers x (3072x9216 QKV, 3072x3072 out,
    3072x16384 gate+up, 8192x3072 down), no biases;
  * head: [768, 50257].
"""
from __future__ import annotations

import numpy as np

SEED = 1234

ROLE_W, ROLE_X, ROLE_BIAS, ROLE_OUTLIER, ROLE_TOKENS = 0, 1, 2, 3, 4

# workload ids used as the ``cfg`` component of the seed
CFG_SINGLE, CFG_GPT2_DECODE, CFG_HEAD, CFG_GPT2_PREFILL, CFG_DENSE38 = 0, 1, 2, 3, 4

GPT2_LAYERS = 12
GPT2_SHAPES = ((768, 2304), (768, 768), (768, 3072), (3072, 768))  # (K, N) per slot
GPT2_HIDDEN = 768
GPT2_VOCAB = 50257
GPT2_PROMPT = 58

DENSE38_LAYERS = 32
DENSE38_SHAPES = ((3072, 9216), (3072, 3072), (3072, 16384), (8192, 3072))

SIGMA_W = 0.02
SIGMA_X = 1.0
OUTLIER_FRAC = 0.001
OUTLIER_FACTOR = 50.0


def rng(cfg: int, layer: int, slot: int, role: int, seed: int = SEED) -> np.random.Generator:
    return np.random.default_rng([seed, cfg, layer, slot, role])


def normal(shape, sigma: float, key) -> np.ndarray:
    g = rng(*key)
    return g.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)


def weights(K: int, N: int, cfg: int, layer: int = 0, slot: int = 0) -> np.ndarray:
    """fp32 [K, N] ~ N(0, 0.02)."""
    return normal((K, N), SIGMA_W, (cfg, layer, slot, ROLE_W))


def bias(N: int, cfg: int, layer: int = 0, slot: int = 0) -> np.ndarray:
    """fp32 [N] ~ N(0, 0.02)."""
    return normal((N,), SIGMA_W, (cfg, layer, slot, ROLE_BIAS))


def activations(M: int, K: int, cfg: int, layer: int = 0, slot: int = 0,
                outliers: bool = False) -> np.ndarray:
    """fp32 [M, K] ~ N(0, 1); with ``outliers`` 0.1% of entries are multiplied by 50."""
    x = normal((M, K), SIGMA_X, (cfg, layer, slot, ROLE_X))
    if outliers and x.size:
        count = max(1, int(round(OUTLIER_FRAC * x.size)))
        pos = rng(cfg, layer, slot, ROLE_OUTLIER).choice(x.size, size=count, replace=False)
        flat = x.reshape(-1)
        flat[pos] *= np.float32(OUTLIER_FACTOR)
    return x


def head_table(K: int = GPT2_HIDDEN, N: int = GPT2_VOCAB, cfg: int = CFG_HEAD) -> np.ndarray:
    """fp32 [K, N] ~ N(0, 0.02): the source of the int8 tied head."""
    return normal((K, N), SIGMA_W, (cfg, 0, 0, ROLE_W))


def tokens(T: int, N: int, cfg: int, layer: int = 0) -> np.ndarray:
    """int64 [T] uniform in [0, N)."""
    return rng(cfg, layer, 0, ROLE_TOKENS).integers(0, N, size=T, dtype=np.int64)


def body(name: str):
    """The (layer, slot, K, N) list of a body pass, in execution order."""
    if name == "gpt2":
        layers, shapes = GPT2_LAYERS, GPT2_SHAPES
    elif name == "dense38":
        layers, shapes = DENSE38_LAYERS, DENSE38_SHAPES
    else:
        raise ValueError(name)
    return [(l, s, K, N) for l in range(layers) for s, (K, N) in enumerate(shapes)]
