"""Seeded synthetic inputs shared by the GPU path's tests, the oracle's tests
and the benchmark.

This module draws random tensors and nothing else: it holds none of the
quantization or GEMM arithmetic.  Every tensor is drawn as float32 from
numpy.random.default_rng(SeedSequence([seed, tensor_id])), scaled by its
standard deviation, and rounded to BF16 by torch's CPU conversion (round to
nearest even).  Values are returned as float32 arrays holding BF16 values.

Tensor ids: X=1, W=2, dY=3, outlier-channel choice=4, MoE routing=5.
"""
from __future__ import annotations

import math

import numpy as np

ID_X, ID_W, ID_DY, ID_OUTLIER, ID_ROUTING = 1, 2, 3, 4, 5


def rng_for(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tensor_id]))


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round a float32 array to BF16 with torch's CPU cast; float32 out."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def normal_bf16(shape, std: float, seed: int, tensor_id: int) -> np.ndarray:
    """N(0, std^2) samples rounded to BF16 (std is the standard deviation)."""
    g = rng_for(seed, tensor_id)
    x = g.standard_normal(shape, dtype=np.float32) * np.float32(std)
    return to_bf16_values(x)


def outlier_channels(K: int, frac: float, seed: int) -> np.ndarray:
    """ceil(frac*K) distinct channel indices, drawn without replacement."""
    g = rng_for(seed, ID_OUTLIER)
    n = int(math.ceil(frac * K))
    return np.sort(g.choice(K, size=n, replace=False))


def activations_with_outliers(M: int, K: int, seed: int, frac: float = 0.01,
                              factor: float = 50.0, tensor_id: int = ID_X) -> np.ndarray:
    """N(0,1) activations whose chosen channels (1 % by default) are scaled by
    `factor` for every token, then rounded to BF16."""
    g = rng_for(seed, tensor_id)
    x = g.standard_normal((M, K), dtype=np.float32)
    ch = outlier_channels(K, frac, seed)
    x[:, ch] *= np.float32(factor)
    return to_bf16_values(x)


def zipf_top8_routing(num_tokens: int, num_experts: int, top_k: int,
                      alpha: float, seed: int) -> np.ndarray:
    """Expert ids [num_tokens, top_k], distinct per token.

    Expert popularity is proportional to rank^-alpha over a seeded random
    permutation of the experts; each token takes top_k distinct experts by
    Gumbel-top-k on the log-popularities.
    """
    g = rng_for(seed, ID_ROUTING)
    perm = g.permutation(num_experts)
    logp = np.empty(num_experts)
    logp[perm] = -alpha * np.log(np.arange(1, num_experts + 1))
    gumbel = -np.log(-np.log(g.random((num_tokens, num_experts))))
    return np.argsort(-(logp[None, :] + gumbel), axis=1)[:, :top_k]


def segment_offsets(expert_ids: np.ndarray, num_experts: int) -> np.ndarray:
    """Rows sorted by expert: int32 offsets [E+1] of each expert's segment."""
    counts = np.bincount(expert_ids.reshape(-1), minlength=num_experts)
    off = np.zeros(num_experts + 1, dtype=np.int64)
    off[1:] = np.cumsum(counts)
    return off.astype(np.int32)
