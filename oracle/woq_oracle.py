"""CPU oracle for group-wise weight-only RTN quantization, the layout-v2 packed
stream, dequantization, and the dequantize-GEMV/GEMM that consumes it.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain, obviously-correct
statement of what the GPU library computes.  Only the test suite, the smoke
check in ``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of ``bench.py``
may import it.  The product path (the HIP library and its Python binding)
never imports, calls or links anything here, and this module imports nothing
from the product.

Sources (the five pages on weight-only quantization):

* "Quantising Large Language Models for Efficient Inference", section
  "Post-training methods for 4-bit weights": symmetric group-wise quantisation
  of a weight row (scale = max|w| / qmax per group, q = clip(round(w/scale),
  -qmax-1, qmax), dequant q*scale); one scale (and zero point) per group of
  64-128 weights.
* "CMU 11-868 L19-L20 Model Quantization", section "absmax and zero-point":
  absmax and zero-point quantizers; a zero range is replaced by 1; the
  zero-point is a rounded integer offset; dequant is (q - zp) / scale.
* "LLM Quantization: 160GB Model on a Laptop", sections "Symmetric
  Quantization" (scale = max_abs / (2^(bits-1) - 1), round(value/scale),
  quantized*scale, worked example) and "Asymmetric Quantization"
  (scale = (max - min) / (qmax - qmin)).
* "Quantising Large Language Models ...", section "Why LLMs are hard to
  quantise": the per-channel scaling identity Y = (X diag(s)^-1)(diag(s) W);
  "MIT 6.5940 Lab 4 + Lab 5", Lab 4 Question 2: multiply a salient weight
  channel by s and divide the activation by s.
* "MIT 6.5940 Lab 4 + Lab 5", Lab 4 "Starting point and setup": pseudo
  quantization = quantize to integers then dequantize immediately.
* "Quantising Large Language Models ...", section "Weight-only vs
  weight-and-activation quantisation": W4A16 weights are dequantised on the
  fly inside the matrix-multiplication kernel.

Readings taken where the pages leave a step open (each is listed, with its
reason, in the design notes of the repository):

* Rounding is round-half-to-even (numpy ``rint``), as in the numpy and torch
  snippets; the JavaScript snippet's half-up rounding is not used.
* Arithmetic that decides a stored value (scale, zero-point, code) is IEEE
  binary32, one correctly-rounded operation per step, the precision the GPU
  kernel uses; the scale is stored as IEEE binary16 (round-to-nearest-even,
  subnormals kept) and the codes are computed with the stored scale.
* Symmetric codes are clipped to [-2^(b-1), 2^(b-1)-1] and stored unsigned as
  u = q + 2^(b-1); an all-zero group (scale 0) stores u = 2^(b-1).
* Asymmetric: range r = max - min (replaced by 1 when 0), S = f16(r/(2^b-1)),
  zero-point Z = clip(rne(-min/S), 0, 2^b-1) (an integer, stored in fp16),
  u = clip(rne(w/S) + Z, 0, 2^b-1); a scale that underflows to 0 gives Z = 0
  and u = 0.
* The AWQ fold multiplies W[n,k] by s[k] in binary32 before the group
  statistics; the GEMV/GEMM divides x by s (exactly, in fp64, here).
* Dequantization and products are exact / fp64: w_hat = (u - Z) * S.
* AWQ search: alpha on the grid i / n (n = 20), s = max(mean|x|, 1e-4)^alpha
  with no further normalization, error = ||X W^T - (X/s) Q(W s)^T||_F^2 over
  the calibration tokens, first minimum wins.
* GPTQ: lambda = 0.01 * mean(diag(2 X^T X)); channels with a zero diagonal get
  1 and their weights are zeroed; group parameters come from the current
  (updated) weights when a group's first column is reached.

Parity pins for every function here live in ``tests/test_oracle.py``.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = [
    "Quantized",
    "fold_act_scale",
    "quantize",
    "pack_v2",
    "unpack_v2",
    "packed_row_bytes",
    "dequantize",
    "bf16_bits_to_f64",
    "activations_f64",
    "gemm",
    "quantize_pack",
    "rel_l2",
    "awq_alphas",
    "awq_channel_mean",
    "awq_scale_for",
    "awq_loss",
    "awq_search",
    "codes_with_params",
    "gptq_upper_factor",
    "gptq",
    "reconstruction_loss",
]


@dataclass
class Quantized:
    """Result of group-wise RTN quantization of an [N, K] weight matrix.

    codes  : uint8 [N, K], unsigned codes u in [0, 2^bits - 1]
    scales : float16 [N, K // group_size]
    zeros  : float16 [N, K // group_size] (asymmetric) or None (symmetric:
             the implied zero is 2^(bits-1))
    """

    codes: np.ndarray
    scales: np.ndarray
    zeros: Optional[np.ndarray]
    bits: int
    group_size: int
    asymmetric: bool


def fold_act_scale(W: np.ndarray, act_scale: Optional[np.ndarray]) -> np.ndarray:
    """AWQ fold: w'[n, k] = fl32(W[n, k] * s[k]).

    Follows the per-channel scaling identity of "Quantising Large Language
    Models ...", section "Why LLMs are hard to quantise"
    (Y = (X diag(s)^-1)(diag(s) W)), and Lab 4 Question 2 of "MIT 6.5940 Lab 4
    + Lab 5" (scale a weight channel up by s, the activation down by s).
    One binary32 multiply per weight; without a scale the fp16 weights are
    widened exactly.
    """
    w = np.asarray(W).astype(np.float32)
    if act_scale is None:
        return w
    s = np.asarray(act_scale, dtype=np.float32)
    assert s.shape == (w.shape[1],)
    return np.multiply(w, s[None, :], dtype=np.float32)


def quantize(
    W: np.ndarray,
    bits: int,
    group_size: int,
    asymmetric: bool,
    act_scale: Optional[np.ndarray] = None,
) -> Quantized:
    """Group-wise round-to-nearest quantization of W [N, K] (fp16 values).

    Groups are ``group_size`` consecutive weights of one row along K, starting
    at k = 0 (the reshape of "Quantising Large Language Models ...", section
    "Post-training methods for 4-bit weights").

    Symmetric (absmax): per group a = max|w|, S = f16(fl32(a / qmax)) with
    qmax = 2^(bits-1) - 1 ("LLM Quantization: 160GB Model on a Laptop",
    section "Symmetric Quantization"; "Quantising ..." group-wise code);
    q = clip(rne(fl32(w / S)), -2^(bits-1), 2^(bits-1) - 1); u = q + 2^(bits-1).

    Asymmetric (zero-point): r = fl32(max - min), r := 1 if r == 0 ("CMU
    11-868 L19-L20", section "absmax and zero-point"); S = f16(fl32(r / qu))
    with qu = 2^bits - 1 ("LLM Quantization ...", section "Asymmetric
    Quantization"); Z = clip(rne(fl32(-min / S)), 0, qu);
    u = clip(rne(fl32(w / S)) + Z, 0, qu).
    """
    W = np.asarray(W)
    assert W.ndim == 2
    N, K = W.shape
    assert bits in (2, 3, 4, 8) and group_size > 0 and K % group_size == 0
    w = fold_act_scale(W, act_scale)
    g = w.reshape(N, K // group_size, group_size)

    if not asymmetric:
        half = 2 ** (bits - 1)
        qmax = np.float32(half - 1)
        a = np.abs(g).max(axis=2)
        S = np.divide(a, qmax, dtype=np.float32).astype(np.float16)
        S32 = S.astype(np.float32)[:, :, None]
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.rint(np.divide(g, S32, dtype=np.float32))
        q = np.where(S32 == 0, np.float32(0), q)
        q = np.clip(q, -half, half - 1)
        u = (q + half).astype(np.uint8)
        return Quantized(u.reshape(N, K), S, None, bits, group_size, False)

    qu = np.float32(2 ** bits - 1)
    mn = g.min(axis=2)
    mx = g.max(axis=2)
    r = np.subtract(mx, mn, dtype=np.float32)
    r = np.where(r == 0, np.float32(1), r).astype(np.float32)
    S = np.divide(r, qu, dtype=np.float32).astype(np.float16)
    S32 = S.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        Zf = np.rint(np.divide(-mn, S32, dtype=np.float32))
        Zf = np.where(S32 == 0, np.float32(0), Zf)
        # Z is an integer; adding +0 stores an integer zero as +0, never -0
        Zf = np.clip(Zf, 0, qu) + np.float32(0)
        q = np.rint(np.divide(g, S32[:, :, None], dtype=np.float32))
    q = np.where(S32[:, :, None] == 0, -Zf[:, :, None], q)
    u = np.clip(q + Zf[:, :, None], 0, qu).astype(np.uint8)
    return Quantized(u.reshape(N, K), S, Zf.astype(np.float16), bits, group_size, True)


def packed_row_bytes(K: int, bits: int) -> int:
    """Bytes of one packed row: K * bits / 8."""
    assert (K * bits) % 8 == 0
    return K * bits // 8


def pack_v2(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack unsigned codes [N, K] into layout v2, uint8 [N, K*bits/8].

    Layout v2 (little-endian 32-bit words, rows back to back):

    * 4-bit (as in layout v1): word j of a row holds k in [8j, 8j+8); the code
      of k = 8j + 2t + h (t in 0..3, h in 0..1) sits at bits
      [16h + 4t, 16h + 4t + 4).
    * 3-bit: a 12-byte unit j (words w0, w1, w2) holds k in [32j, 32j+32); for
      i = k - 32j = 2t + h (t in 0..15, h in 0..1) the code of pair t < 15 sits
      whole in word w_(t // 5) at bits [16h + 3(t % 5), +3); the code of pair
      15 is split, its bit b (b = 0, 1, 2) at bit 16h + 15 of word w_b.

    Written element by element from that definition (slow on purpose).
    """
    codes = np.asarray(codes)
    N, K = codes.shape
    if bits == 4:
        assert K % 8 == 0
        words = np.zeros((N, K // 8), dtype=np.uint32)
        for j in range(K // 8):
            for t in range(4):
                for h in range(2):
                    k = 8 * j + 2 * t + h
                    words[:, j] |= (codes[:, k].astype(np.uint32) & 0xF) << np.uint32(16 * h + 4 * t)
    elif bits == 3:
        assert K % 32 == 0
        words = np.zeros((N, K // 32, 3), dtype=np.uint32)
        for j in range(K // 32):
            for i in range(32):
                t, h = divmod(i, 2)
                u = codes[:, 32 * j + i].astype(np.uint32) & 7
                if t < 15:
                    words[:, j, t // 5] |= u << np.uint32(16 * h + 3 * (t % 5))
                else:
                    for b in range(3):
                        words[:, j, b] |= ((u >> np.uint32(b)) & 1) << np.uint32(16 * h + 15)
        words = words.reshape(N, -1)
    else:
        raise ValueError("layout v2 is defined for 3 and 4 bits")
    return np.ascontiguousarray(words.astype("<u4")).view(np.uint8).reshape(N, packed_row_bytes(K, bits))


def unpack_v2(packed: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Inverse of :func:`pack_v2`: uint8 [N, K*bits/8] -> codes uint8 [N, K]."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    words = packed.reshape(N, -1).view("<u4").astype(np.uint32)
    codes = np.zeros((N, K), dtype=np.uint8)
    if bits == 4:
        for j in range(K // 8):
            for t in range(4):
                for h in range(2):
                    codes[:, 8 * j + 2 * t + h] = (words[:, j] >> np.uint32(16 * h + 4 * t)) & 0xF
    elif bits == 3:
        words = words.reshape(N, K // 32, 3)
        for j in range(K // 32):
            for i in range(32):
                t, h = divmod(i, 2)
                if t < 15:
                    u = (words[:, j, t // 5] >> np.uint32(16 * h + 3 * (t % 5))) & 7
                else:
                    u = sum(((words[:, j, b] >> np.uint32(16 * h + 15)) & 1) << np.uint32(b) for b in range(3))
                codes[:, 32 * j + i] = u
    else:
        raise ValueError("layout v2 is defined for 3 and 4 bits")
    return codes


def dequantize(q: Quantized) -> np.ndarray:
    """Pseudo-quantization's second half: w_hat = (u - Z) * S, exact in fp64.

    "MIT 6.5940 Lab 4 + Lab 5", Lab 4 setup (quantize then dequantize);
    dequant formulas of "CMU 11-868 L19-L20" ((q - zp)/scale) and "Quantising
    ..." (q * scale).  |u - Z| <= 2^bits - 1 and S has 11 significant bits, so
    every product is exact in binary64.
    """
    N, K = q.codes.shape
    G = q.group_size
    S = np.repeat(q.scales.astype(np.float64), G, axis=1)
    if q.zeros is None:
        Z = np.float64(2 ** (q.bits - 1))
    else:
        Z = np.repeat(q.zeros.astype(np.float64), G, axis=1)
    return (q.codes.astype(np.float64) - Z) * S


def bf16_bits_to_f64(bits16: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 numbers given as their uint16 bit patterns."""
    b = np.asarray(bits16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def activations_f64(X: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of activations stored as fp16 values or bf16 bits."""
    if dtype == "f16":
        return np.asarray(X, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(X)
    raise ValueError(dtype)


def gemm(X64: np.ndarray, w_hat: np.ndarray, act_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Y = (X diag(s)^-1) W_hat^T with fp64 accumulation.

    X64 is [M, K] (exact fp64 values of the activations), w_hat [N, K].  With
    an AWQ scale the activation is divided by s ("Quantising ...", section
    "Why LLMs are hard to quantise"); the weights already carry the factor s.
    A GEMV is the M = 1 case.
    """
    X64 = np.atleast_2d(np.asarray(X64, dtype=np.float64))
    if act_scale is not None:
        X64 = X64 / np.asarray(act_scale, dtype=np.float32).astype(np.float64)[None, :]
    return X64 @ np.asarray(w_hat, dtype=np.float64).T


def quantize_pack(W, bits, group_size, asymmetric, act_scale=None):
    """quantize + pack_v2: returns (packed uint8 [N, K*bits/8], scales f16, zeros f16|None, Quantized)."""
    q = quantize(W, bits, group_size, asymmetric, act_scale)
    return pack_v2(q.codes, bits), q.scales, q.zeros, q


def rel_l2(y: np.ndarray, y_ref: np.ndarray) -> float:
    """||y - y_ref||_2 / ||y_ref||_2 over the whole output, in fp64."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref.ravel())
    num = np.linalg.norm((y - y_ref).ravel())
    return float(num / den) if den > 0 else float(num)


# --------------------------------------------------------------------------
# AWQ scale search
# --------------------------------------------------------------------------

AWQ_SCALE_FLOOR = 1e-4  # reading: per-channel scales are kept at or above this


def awq_alphas(n_grid: int) -> np.ndarray:
    """The exponents tried: alpha_i = i / n_grid, i = 0 .. n_grid - 1."""
    return np.arange(n_grid, dtype=np.float64) / n_grid


def awq_channel_mean(X64: np.ndarray) -> np.ndarray:
    """Mean absolute activation of each input channel over the calibration
    tokens: the statistic Lab 4's forward hooks record ("MIT 6.5940 Lab 4 +
    Lab 5", Lab 4 "Starting point and setup")."""
    return np.abs(np.asarray(X64, dtype=np.float64)).mean(axis=0)


def awq_scale_for(mean_abs: np.ndarray, alpha: float) -> np.ndarray:
    """s = max(mean|x|, floor)^alpha, in fp32.  alpha = 0 gives s = 1 (plain
    RTN); larger alpha scales the channels that see large activations up."""
    m = np.maximum(np.asarray(mean_abs, dtype=np.float64), AWQ_SCALE_FLOOR)
    return np.power(m, alpha).astype(np.float32)


def awq_loss(X64: np.ndarray, W: np.ndarray, s: np.ndarray, bits: int, group_size: int,
             asymmetric: bool) -> float:
    """Output reconstruction error of one layer for one scale vector:
    || X W^T - (X / s) Q(W s)^T ||_F^2 in fp64, the layer-wise objective of
    "Quantising Large Language Models ...", section "Post-training methods
    for 4-bit weights", with the scale applied as in Lab 4 Question 2 (scale
    the weight channel up, quantize, divide the activation)."""
    X64 = np.asarray(X64, dtype=np.float64)
    y_ref = X64 @ np.asarray(W, dtype=np.float32).astype(np.float64).T
    q = quantize(W, bits, group_size, asymmetric, s)
    y_q = gemm(X64, dequantize(q), s)
    return float(np.sum((y_ref - y_q) ** 2))


def awq_search(X64: np.ndarray, W: np.ndarray, bits: int, group_size: int, asymmetric: bool,
               n_grid: int = 20):
    """Grid search of the AWQ exponent: for each alpha, compute the scale,
    scale the weights up, quantize, scale the activations down and measure
    the output error; the first alpha with the smallest error wins ("MIT
    6.5940 Lab 4 + Lab 5", Question 2, the search loop).

    Returns (losses fp64 [n_grid], best index, best scale fp32 [K])."""
    m = awq_channel_mean(X64)
    losses = np.array([awq_loss(X64, W, awq_scale_for(m, a), bits, group_size, asymmetric)
                       for a in awq_alphas(n_grid)])
    best = int(np.argmin(losses))
    return losses, best, awq_scale_for(m, awq_alphas(n_grid)[best])


# --------------------------------------------------------------------------
# GPTQ
# --------------------------------------------------------------------------

GPTQ_DAMP = 0.01  # reading: lambda = 0.01 * mean(diag(2 X^T X))


def codes_with_params(w: np.ndarray, S: np.ndarray, Z: Optional[np.ndarray], bits: int,
                      asymmetric: bool) -> np.ndarray:
    """Codes of one weight column w [N] (fp32 values) under given per-row
    group parameters S [N] (fp16) and Z [N] (fp16, asymmetric): the same
    element rule as ``quantize`` (rne(fl32(w / S)), clipped; S == 0 gives the
    zero code)."""
    w = np.asarray(w, dtype=np.float32)
    S32 = np.asarray(S, dtype=np.float16).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(np.divide(w, S32, dtype=np.float32))
    if not asymmetric:
        half = 2 ** (bits - 1)
        q = np.where(S32 == 0, np.float32(0), q)
        return (np.clip(q, -half, half - 1) + half).astype(np.uint8)
    qu = np.float32(2 ** bits - 1)
    Zf = np.asarray(Z, dtype=np.float16).astype(np.float32)
    q = np.where(S32 == 0, -Zf, q)
    return np.clip(q + Zf, 0, qu).astype(np.uint8)


def gptq_upper_factor(X64: np.ndarray, damp: float = GPTQ_DAMP):
    """U, upper triangular with U^T U = (2 X^T X + lambda I)^-1, i.e. the
    transposed Cholesky factor of the inverse Hessian ("CMU 11-868 L19-L20",
    section "The algorithm in four steps", step 1), with lambda = damp *
    mean(diag(2 X^T X)).  Input channels that never fire (zero diagonal) get a
    diagonal of 1 and are returned as `dead`."""
    X64 = np.asarray(X64, dtype=np.float64)
    K = X64.shape[1]
    H = 2.0 * (X64.T @ X64)
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    H = H + damp * np.mean(np.diag(H)) * np.eye(K)
    U = np.linalg.cholesky(np.linalg.inv(H)).T
    return U, dead


def gptq(X64: np.ndarray, W: np.ndarray, bits: int, group_size: int, asymmetric: bool,
         damp: float = GPTQ_DAMP, return_errors: bool = False):
    """GPTQ in its plain column-by-column form ("CMU 11-868 L19-L20", section
    "The algorithm in four steps"): for k = 0 .. K-1, quantize column k,
    divide its rounding error by U[k, k] and subtract err * U[k, j] from every
    later column j.  (Blocking and lazy batch updates reorder this arithmetic
    without changing it.)  Group parameters are taken, as the first column of
    each group is reached, from the group's current (already updated) weights,
    by the same rules as ``quantize``.  The updates run in fp64; every rounding
    decision is made on the fp32 value of the current weight.

    Returns a Quantized (and the error matrix E [N, K] with W - w_hat = E U
    when return_errors)."""
    W = np.asarray(W)
    N, K = W.shape
    assert K % group_size == 0
    U, dead = gptq_upper_factor(X64, damp)
    Wf = W.astype(np.float32).astype(np.float64)
    Wf[:, dead] = 0.0
    codes = np.zeros((N, K), np.uint8)
    S = np.zeros((N, K // group_size), np.float16)
    Z = np.zeros((N, K // group_size), np.float16) if asymmetric else None
    E = np.zeros((N, K))
    for k in range(K):
        g = k // group_size
        if k % group_size == 0:
            qg = quantize(Wf[:, k:k + group_size].astype(np.float32), bits, group_size, asymmetric)
            S[:, g] = qg.scales[:, 0]
            if asymmetric:
                Z[:, g] = qg.zeros[:, 0]
        u = codes_with_params(Wf[:, k].astype(np.float32), S[:, g], None if Z is None else Z[:, g], bits, asymmetric)
        codes[:, k] = u
        z = Z[:, g].astype(np.float64) if asymmetric else float(2 ** (bits - 1))
        w_hat = (u.astype(np.float64) - z) * S[:, g].astype(np.float64)
        err = (Wf[:, k] - w_hat) / U[k, k]
        E[:, k] = err
        Wf[:, k + 1:] -= np.outer(err, U[k, k + 1:])
    q = Quantized(codes, S, Z, bits, group_size, asymmetric)
    return (q, E) if return_errors else q


def reconstruction_loss(X64: np.ndarray, W: np.ndarray, q: Quantized) -> float:
    """|| X W^T - X w_hat^T ||_F^2 in fp64: the layer-wise objective GPTQ and
    RTN are compared on ("CMU 11-868 L19-L20", page 16 / L20 page 5)."""
    X64 = np.asarray(X64, dtype=np.float64)
    D = np.asarray(W, dtype=np.float32).astype(np.float64) - dequantize(q)
    return float(np.sum((X64 @ D.T) ** 2))
