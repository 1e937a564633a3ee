"""Element-wise bound on a GEMV / GEMM output against the fp64 oracle.

Test infrastructure: the relative-L2 bar over a whole output can hide one
wrong row (at N = 8192 a row that is 10% off adds about 1e-3), so every
parity test also bounds each output element by the rounding the kernels
perform.  For output (m, n), with x' = x / s the exact scaled activation and
w_hat the oracle's exact dequantized weight:

* input roundings: x' rounded once to fp16 (unit roundoff 2^-11) and, on the
  MFMA paths that round the weight, w_hat rounded once to fp16 (2^-11); bf16
  paths keep 16-bit hi + lo pairs (about 2^-16).  Relative error per product
  at most 2^-10.
* fp32 accumulation: the largest summands any kernel forms are
  x' * S * (MAGIC + u) with MAGIC = 1024 (the fp16 code widening 1024 + u,
  whose offset is removed once per group); every summand and partial sum is
  rounded to fp32 (unit roundoff 2^-24).  Within a group of G weights a term
  passes through at most about 2G roundings (an MFMA chain of G / 32 steps
  that sums 32 products each, then the group's correction).
* the output: y is rounded once from fp32 to fp16 (2^-11) or bf16 (2^-8).

Rounding errors are modelled as independent, zero-mean and bounded by the unit
roundoff (the probabilistic model of Higham and Mary, "A New Approach to
Probabilistic Rounding Error Analysis", SIAM J. Sci. Comput. 41(5), 2019).
A sum of such errors weighted by terms t_i stays below lambda * u * ||t||_2
except with probability 2 exp(-lambda^2 / 2) (Hoeffding); lambda = 8 puts
that below 3e-14 per element.  So

  |y - y_ref| <= (1 + u_T) * E + u_T * |y_ref| + 2^-24,
  E = 8 * (2^-10 * ||x' o w_hat_n||_2 + 2^-24 * sqrt(2 G) * (1024 + 2^b) * ||x' o S_n||_2),

where S_n is row n's scale repeated over its groups.  The worst-case form of
the same bound (L1 norms instead of L2, 2G * 2^-24 instead of sqrt(2G) *
2^-24) holds without the model but is about sqrt(K) times looser, too loose
to see a wrong row; the model's bound is about 1% of a typical output at
K = 8192.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

LAMBDA = 8.0
INPUT_ROUNDING = 2.0 ** -10
ACC_ROUNDING = 2.0 ** -24
MAGIC = 1024.0
OUT_ROUNDING = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def output_bound(X64: np.ndarray, w_hat: np.ndarray, scales: np.ndarray, bits: int, group_size: int,
                 act_scale: Optional[np.ndarray], y_ref: np.ndarray, out_dtype: str) -> np.ndarray:
    """Per-element bound [M, N] for outputs y of X64 [M, K] (exact activation
    values) times w_hat [N, K] (exact dequantized weights) with per-group
    scales [N, K / G]."""
    X64 = np.atleast_2d(np.asarray(X64, dtype=np.float64))
    if act_scale is not None:
        X64 = X64 / np.asarray(act_scale, dtype=np.float32).astype(np.float64)[None, :]
    x2 = X64 * X64
    w = np.asarray(w_hat, dtype=np.float64)
    a2 = np.sqrt(x2 @ (w * w).T)
    S = np.repeat(np.asarray(scales, dtype=np.float64), group_size, axis=1)
    t2 = np.sqrt(x2 @ (S * S).T) * (MAGIC + 2.0 ** bits)
    E = LAMBDA * (INPUT_ROUNDING * a2 + ACC_ROUNDING * np.sqrt(2.0 * group_size) * t2)
    u_t = OUT_ROUNDING[out_dtype]
    return (1.0 + u_t) * E + u_t * np.abs(np.atleast_2d(y_ref)) + 2.0 ** -24


def check_elementwise(y: np.ndarray, y_ref: np.ndarray, bound: np.ndarray):
    """(ok, worst ratio |y - y_ref| / bound, index of the worst element)."""
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    y_ref = np.atleast_2d(np.asarray(y_ref, dtype=np.float64))
    r = np.abs(y - y_ref) / bound
    i = np.unravel_index(int(np.argmax(r)), r.shape)
    return bool(np.all(np.isfinite(y)) and r[i] <= 1.0), float(r[i]), tuple(int(v) for v in i)
