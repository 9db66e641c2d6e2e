"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds only random draws and dtype casts of inputs; none of the method's
arithmetic lives here.  Both the CPU oracle (through the tests and the benchmark) and the
HIP library consume what it returns, so neither side depends on the other.

The shapes stand in for the models the pages measure, which are not available here:

* dense 4B decoder projections (hidden 2560, intermediate 9728, 8 KV heads of 128), as in the
  W8A8 prefill/decode tables of "feat(quantization): support compressed-tensors W8A8 and
  mixed modules" (Benchmark / Performance Impact, Offline performance, TP1);
* dense 8B decoder projections (hidden 4096, intermediate 12288), the batch-1 decode anchor
  of "Day 6 — Quantize It Yourself" (The math);
* a 16B mixture-of-experts block, 64 routed experts (2048 -> 1408 gate/up, 1408 -> 2048
  down) plus 2 shared experts, top-6 routing, as in "Phase 5a: int8 weight-only
  quantization" (Summary).

Value distributions: weights N(0, 0.02); activations N(0, 1); outlier input dims scaled by
100 (the emergent outlier channels described in "Day 6 — Quantize It Yourself", The
mechanism, block 3).  Every draw comes from ``numpy.random.Generator(PCG64(seed))`` in a
fixed order; 16-bit inputs are drawn in float32 and rounded to nearest even by torch.
"""
from __future__ import annotations

import numpy as np
import torch

# (N, K) = (out_features, in_features) of each projection.
DENSE_4B = {
    "q": (4096, 2560), "k": (1024, 2560), "v": (1024, 2560), "o": (2560, 4096),
    "gate": (9728, 2560), "up": (9728, 2560), "down": (2560, 9728),
}
DENSE_8B = {
    "q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096), "o": (4096, 4096),
    "gate": (12288, 4096), "up": (12288, 4096), "down": (4096, 12288),
}
MOE_16B = {"gate": (1408, 2048), "up": (1408, 2048), "down": (2048, 1408)}
MOE_ROUTED, MOE_SHARED, MOE_TOP = 64, 2, 6

# Projections that read the same layer input run as one GEMM over their concatenated
# weights (per-channel scales concatenated alike): the same products as separate launches.
DENSE_4B_FUSED = {"qkv": ("q", "k", "v"), "o": ("o",), "gate_up": ("gate", "up"),
                  "down": ("down",)}

DENSE_8B_FUSED = {"qkv": ("q", "k", "v"), "o": ("o",), "gate_up": ("gate", "up"),
                  "down": ("down",)}

PREFILL_4B_TOKENS = (128, 512, 2048)
DECODE_8B_BATCH = (1, 4, 8)
MOE_TOKENS = (1, 4, 16, 64)
PREFILL_8B_TOKENS = (4096, 16384)


def rng(seed: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """float32 numpy -> bfloat16 CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)


def to_f16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.float16)


def bits16(t: torch.Tensor) -> np.ndarray:
    """The uint16 bit patterns of a bfloat16/float16 CPU tensor."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def outlier_count(k: int, frac: float) -> int:
    return max(1, int(round(frac * k)))


def weight(g: np.random.Generator, n: int, k: int, std: float = 0.02) -> np.ndarray:
    return (g.standard_normal((n, k), dtype=np.float32) * np.float32(std)).astype(np.float32)


def activations(g: np.random.Generator, m: int, k: int, outlier_frac: float = 0.0,
                outlier_scale: float = 100.0, n_outliers: int | None = None) -> np.ndarray:
    """N(0,1) rows with a few input dims (the same for every token) scaled up."""
    x = g.standard_normal((m, k), dtype=np.float32)
    if n_outliers is None and outlier_frac > 0:
        n_outliers = outlier_count(k, outlier_frac)
    if n_outliers:
        cols = g.choice(k, n_outliers, replace=False)
        x[:, cols] *= np.float32(outlier_scale)
    return x


def tiny_w8a8(seed: int = 0) -> dict:
    """The tiny W8A8 case: fp32 weight [256, 512] ~ N(0, 0.02) with 2 all-zero output
    channels and 1 input column x50; fp32 activations [4, 512] ~ N(0, 1) with 2 hidden dims
    x100; fp32 output, no bias."""
    g = rng(seed)
    w = weight(g, 256, 512)
    zero_rows = g.choice(256, 2, replace=False)
    w[zero_rows, :] = 0.0
    col = g.choice(512, 1, replace=False)
    w[:, col] *= np.float32(50.0)
    x = activations(g, 4, 512, n_outliers=2)
    return {"w": w, "x": x, "zero_rows": np.sort(zero_rows)}


def moe_expert_ids(g: np.random.Generator, t: int, routed: int = MOE_ROUTED,
                   top: int = MOE_TOP, shared: int = MOE_SHARED) -> np.ndarray:
    """[t, top + shared] int32: ``top`` distinct uniform routed ids per token, then the
    always-on shared experts ``routed .. routed + shared - 1``."""
    ids = np.empty((t, top + shared), np.int32)
    for i in range(t):
        ids[i, :top] = g.choice(routed, top, replace=False)
        ids[i, top:] = np.arange(routed, routed + shared, dtype=np.int32)
    return ids


def moe_weights(g: np.random.Generator, n: int, k: int,
                experts: int = MOE_ROUTED + MOE_SHARED) -> np.ndarray:
    """[experts, n, k] float32 ~ N(0, 0.02), to be cast to bf16 by the caller."""
    return (g.standard_normal((experts, n, k), dtype=np.float32) * np.float32(0.02))


def norm_weight(g: np.random.Generator, k: int, std: float = 0.1) -> np.ndarray:
    """[k] float32 RMS-norm weights ~ 1 + N(0, std^2), to be cast to bf16 by the caller."""
    return (np.float32(1.0) + g.standard_normal(k, dtype=np.float32) * np.float32(std))


def router_logits(g: np.random.Generator, t: int, routed: int = MOE_ROUTED) -> np.ndarray:
    """[t, routed] float32 router logits ~ N(0, 1): independent and identically distributed,
    so the top-k experts are uniform over the routed ones, as the uniform-random expert ids
    above are."""
    return g.standard_normal((t, routed), dtype=np.float32)
