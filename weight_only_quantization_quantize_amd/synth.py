"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and converts them to the storage type
of each input (fp16, or bf16 bit patterns).  It holds none of the
quantization or matrix arithmetic: both the CPU oracle and the GPU library
receive the arrays made here.

Shapes and distributions stand in for the pages' workloads, which are real
LLM weights and activations (OPT / LLaMA layers, wikitext-2 and pile-val
calibration text) that are not available here:

* weights ~ N(0, 0.02) (the standard deviation used by the group-size
  experiment of "Quantising Large Language Models ...", section
  "Post-training methods for 4-bit weights"); the decode-GEMV shape also
  carries 0.1% outlier weights drawn from N(0, 0.5);
* activations ~ N(0, 1), with 1% of the input channels scaled by 50 where
  the workload asks for outlier channels (the emergent outlier features of
  "Quantising ...", section "Why LLMs are hard to quantise");
* the AWQ-style per-input-channel scale s = (mean over 512 calibration
  tokens of |x_k|)^0.5, from calibration tokens drawn like the activations
  (the mean-|x| statistic recorded by forward hooks in "MIT 6.5940 Lab 4 +
  Lab 5", Lab 4 setup).

Seeds: each workload draws from its own block of seeds (1000s for the
1024 x 1024 decode shape, 2000s for 8192 x 8192, 3000s for the LLaMA-2-7B
linears, 4000s for the small batch, 5000s for the prefill; see ``WORKLOADS``).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

WEIGHT_STD = 0.02
OUTLIER_WEIGHT_STD = 0.5
OUTLIER_WEIGHT_FRACTION = 0.001
OUTLIER_CHANNEL_FRACTION = 0.01
OUTLIER_CHANNEL_GAIN = 50.0
CALIBRATION_TOKENS = 512


def _normal_f32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    z = rng.standard_normal(size=shape, dtype=np.float32)
    return (z * np.float32(std)).astype(np.float32)


def weights(N: int, K: int, seed: int, std: float = WEIGHT_STD) -> np.ndarray:
    """fp16 [N, K] weights, N(0, std) drawn in fp32 then rounded to fp16."""
    rng = np.random.default_rng(seed)
    return _normal_f32(rng, (N, K), std).astype(np.float16)


def weights_with_outliers(
    N: int,
    K: int,
    seed_w: int,
    seed_pos: int,
    seed_val: int,
    fraction: float = OUTLIER_WEIGHT_FRACTION,
    std: float = WEIGHT_STD,
    outlier_std: float = OUTLIER_WEIGHT_STD,
) -> np.ndarray:
    """fp16 [N, K] N(0, std) weights with round(fraction*N*K) entries (uniform
    positions without replacement) replaced by N(0, outlier_std) draws."""
    W = weights(N, K, seed_w, std)
    count = int(round(fraction * N * K))
    pos = np.random.default_rng(seed_pos).choice(N * K, size=count, replace=False)
    vals = _normal_f32(np.random.default_rng(seed_val), (count,), outlier_std).astype(np.float16)
    flat = W.reshape(-1)
    flat[pos] = vals
    return W


def outlier_channels(K: int, seed: int, fraction: float = OUTLIER_CHANNEL_FRACTION) -> np.ndarray:
    """Sorted indices of round(fraction*K) input channels chosen uniformly."""
    count = int(round(fraction * K))
    return np.sort(np.random.default_rng(seed).choice(K, size=count, replace=False))


def activations_f32(
    M: int, K: int, seed: int, channels: Optional[np.ndarray] = None, gain: float = OUTLIER_CHANNEL_GAIN
) -> np.ndarray:
    """fp32 [M, K] activations ~ N(0, 1); listed channels multiplied by gain."""
    x = np.random.default_rng(seed).standard_normal(size=(M, K), dtype=np.float32)
    if channels is not None and len(channels):
        x[:, channels] *= np.float32(gain)
    return x


def correlated_activations(T: int, K: int, seed: int, rank: int = 16, noise: float = 0.3) -> np.ndarray:
    """fp16 [T, K] calibration activations with correlated channels: a
    rank-``rank`` mixture of N(0, 1) draws plus N(0, noise^2) noise (a stand-in
    for real hidden states, whose channels are far from independent)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(size=(T, rank))
    a = rng.standard_normal(size=(rank, K))
    x = z @ a + noise * rng.standard_normal(size=(T, K))
    return x.astype(np.float32).astype(np.float16)


def to_f16(x32: np.ndarray) -> np.ndarray:
    return np.asarray(x32, dtype=np.float32).astype(np.float16)


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of fp32 values, round-to-nearest-even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations(M: int, K: int, seed: int, dtype: str = "f16", channels=None) -> np.ndarray:
    """Activations in storage form: fp16 values, or bf16 bit patterns."""
    x32 = activations_f32(M, K, seed, channels)
    return to_f16(x32) if dtype == "f16" else to_bf16_bits(x32)


def awq_scale(K: int, seed_cal: int, channels: Optional[np.ndarray], tokens: int = CALIBRATION_TOKENS) -> np.ndarray:
    """Per-input-channel scale s_k = (mean_t |x_cal[t, k]|)^0.5 in fp32, from
    ``tokens`` calibration rows drawn like the activations (fp16-rounded)."""
    xc = to_f16(activations_f32(tokens, K, seed_cal, channels)).astype(np.float32)
    return np.sqrt(np.abs(xc).mean(axis=0, dtype=np.float64)).astype(np.float32)


# --------------------------------------------------------------------------
# Workloads.  Each entry returns the inputs of one linear layer.
# --------------------------------------------------------------------------

@dataclass
class Linear:
    name: str
    M: int
    N: int
    K: int
    W: np.ndarray                       # fp16 [N, K]
    X: np.ndarray                       # fp16 [M, K] or bf16 bits [M, K]
    xdtype: str = "f16"
    act_scale: Optional[np.ndarray] = None   # fp32 [K]
    extra: Dict = field(default_factory=dict)


def decode_1k() -> Linear:
    """M=1, K=N=1024, W ~ N(0, 0.02) (seed 1001), x ~ N(0, 1) (seed 1002)."""
    return Linear("decode_1x1024x1024", 1, 1024, 1024, weights(1024, 1024, 1001), activations(1, 1024, 1002))


def decode_8k(N: int = 8192, K: int = 8192) -> Linear:
    """Decode GEMV M=1, K=N=8192: N(0,0.02) weights (seed 2001) with 0.1% of
    entries (positions seed 2002) redrawn from N(0, 0.5) (seed 2003); x ~ N(0,1)
    (seed 2004)."""
    W = weights_with_outliers(N, K, 2001, 2002, 2003)
    return Linear(f"decode_1x{K}x{N}", 1, N, K, W, activations(1, K, 2004))


# LLaMA-2-7B decoder linears as (name, N, K): q, k, v, o, gate, up, down.
LLAMA7B_LINEARS: List[Tuple[str, int, int]] = [
    ("q_proj", 4096, 4096),
    ("k_proj", 4096, 4096),
    ("v_proj", 4096, 4096),
    ("o_proj", 4096, 4096),
    ("gate_proj", 11008, 4096),
    ("up_proj", 11008, 4096),
    ("down_proj", 4096, 11008),
]


def llama7b_linear(i: int, with_weights: bool = True) -> Linear:
    """LLaMA-2-7B-shaped decode linear i (0..6): W ~ N(0, 0.02) (seed 3000+10i);
    x ~ N(0,1) with 1% of channels x50 (channels and values seed 3100+i); AWQ
    scale from 512 calibration tokens with the same outlier channels (seed 3200+i)."""
    name, N, K = LLAMA7B_LINEARS[i]
    ch = outlier_channels(K, 3100 + i)
    x32 = activations_f32(1, K, 3100 + i, ch)
    s = awq_scale(K, 3200 + i, ch)
    W = weights(N, K, 3000 + 10 * i) if with_weights else None
    return Linear(f"{name}_1x{K}x{N}", 1, N, K, W, to_f16(x32), "f16", s, {"channels": ch})


def small_batch(M: int, xdtype: str = "f16", N: int = 28672, K: int = 8192,
                W: Optional[np.ndarray] = None) -> Linear:
    """Small-batch GEMM, M in {4, 16, 64}, K=8192, N=28672: W ~ N(0,0.02)
    (seed 4001; pass a previous call's W to skip regenerating it), X ~ N(0,1)
    (seed 4002) stored as fp16 or bf16."""
    W = weights(N, K, 4001) if W is None else W
    return Linear(f"small_batch_{M}x{K}x{N}_{xdtype}", M, N, K, W, activations(M, K, 4002, xdtype), xdtype)


def prefill(M: int = 2048, N: int = 11008, K: int = 4096) -> Linear:
    """Prefill GEMM M=2048, K=4096, N=11008: X ~ N(0,1) with 1% of channels x50
    (seed 5001), W ~ N(0, 0.02) (seed 5002)."""
    ch = outlier_channels(K, 5001)
    X = to_f16(activations_f32(M, K, 5001, ch))
    return Linear(f"prefill_{M}x{K}x{N}", M, N, K, weights(N, K, 5002), X, "f16", None, {"channels": ch})


WORKLOADS = {
    "decode_1k": "M=1 K=N=1024, 4-bit asymmetric g128",
    "decode_8k": "M=1 K=N=8192 decode GEMV, 3/4-bit, symmetric and asymmetric, g128",
    "llama7b_linear": "LLaMA-2-7B decode linears at M=1 with AWQ scale, 3/4-bit g128",
    "small_batch": "M in {4,16,64}, K=8192, N=28672, fp16/bf16 activations, 4-bit asymmetric g128",
    "prefill": "M=2048, K=4096, N=11008 prefill GEMM, 4-bit asymmetric g128",
}
