"""PyTorch-facing wrappers over the C ABI.

PyTorch provides device memory and the current HIP stream; each function
checks tensor shapes / dtypes / devices, then passes raw pointers to the
library.  Nothing is computed here.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import torch

from . import _lib

_DTYPE = {torch.float16: _lib.WOQ_F16, torch.bfloat16: _lib.WOQ_BF16}


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


# One GEMM workspace per (device, stream), grown on demand and kept for the
# life of the process: calls on one stream run in stream order, so they can
# share it, and allocating it per call cost more host time than a short GEMM.
_WORKSPACES: dict = {}


def _workspace(device: torch.device, stream: int, nbytes: int) -> torch.Tensor:
    key = (device.index, stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require_gpu(*ts: Optional[torch.Tensor]) -> None:
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libwoq works on GPU tensors only")
        if not t.is_contiguous():
            raise ValueError("libwoq needs contiguous tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")


def packed_bytes(N: int, K: int, bits: int) -> int:
    return int(_lib.call("woq_packed_bytes", N, K, bits))


def _check_quantizer(N: int, K: int, bits: int, group_size: int) -> None:
    if bits not in (3, 4):
        raise ValueError(f"bits must be 3 or 4 (got {bits})")
    if N < 1 or K < 32 or K % 32 or group_size < 32 or group_size % 32 or K % group_size:
        raise ValueError(f"need N >= 1, K a positive multiple of 32 and of group_size, group_size a multiple "
                         f"of 32 (got N={N}, K={K}, group_size={group_size})")


def _check_packed(packed: torch.Tensor, scales: torch.Tensor, zeros: Optional[torch.Tensor], N: int, K: int,
                  bits: int, group_size: int) -> None:
    """The packed set of an [N, K] matrix: uint8 codes of N * K * bits / 8
    bytes, fp16 scales (and zeros) of N * (K / group_size) elements."""
    _check_quantizer(N, K, bits, group_size)
    if packed.dtype != torch.uint8 or packed.numel() != N * K * bits // 8:
        raise ValueError(f"packed must be uint8 with N*K*bits/8 = {N * K * bits // 8} elements "
                         f"(got {packed.dtype}, {packed.numel()})")
    ng = N * (K // group_size)
    for name, t in (("scales", scales), ("zeros", zeros)):
        if t is not None and (t.dtype != torch.float16 or t.numel() != ng):
            raise ValueError(f"{name} must be float16 with N*(K/group_size) = {ng} elements "
                             f"(got {t.dtype}, {t.numel()})")


def _check_act_scale(act_scale: Optional[torch.Tensor], K: int) -> None:
    if act_scale is not None and (act_scale.dtype != torch.float32 or tuple(act_scale.shape) != (K,)):
        raise ValueError(f"act_scale must be float32 of shape ({K},) (got {act_scale.dtype}, "
                         f"{tuple(act_scale.shape)})")


def _check_out(out: torch.Tensor, shape: Tuple[int, ...], dtype: torch.dtype, name: str) -> None:
    if out.dtype != dtype or tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)} (got {out.dtype}, {tuple(out.shape)})")


def quantize_pack(
    W: torch.Tensor,
    bits: int = 4,
    group_size: int = 128,
    asymmetric: bool = True,
    act_scale: Optional[torch.Tensor] = None,
    out: Optional[Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]] = None,
):
    """Quantize fp16 W [N, K] -> (packed uint8 [N, K*bits/8], scales fp16 [N, K/G], zeros fp16 | None)."""
    if W.dtype != torch.float16 or W.dim() != 2:
        raise ValueError("W must be a 2-D float16 tensor")
    N, K = W.shape
    _check_quantizer(N, K, bits, group_size)
    _check_act_scale(act_scale, K)
    if out is None:
        packed = torch.empty((N, K * bits // 8), dtype=torch.uint8, device=W.device)
        scales = torch.empty((N, K // group_size), dtype=torch.float16, device=W.device)
        zeros = torch.empty_like(scales) if asymmetric else None
    else:
        packed, scales, zeros = out
        if (zeros is not None) != bool(asymmetric):
            raise ValueError("out must hold zeros exactly when asymmetric")
        _check_packed(packed, scales, zeros, N, K, bits, group_size)
    _require_gpu(W, act_scale, packed, scales, zeros)
    st = _lib.call("woq_quantize_pack", W.data_ptr(), _ptr(act_scale), N, K, bits, group_size, int(asymmetric),
                   packed.data_ptr(), scales.data_ptr(), _ptr(zeros), _stream(W))
    _lib.check(st, "woq_quantize_pack")
    return packed, scales, zeros


def gemv(
    x: torch.Tensor,
    packed: torch.Tensor,
    scales: torch.Tensor,
    zeros: Optional[torch.Tensor],
    N: int,
    K: int,
    bits: int = 4,
    group_size: int = 128,
    act_scale: Optional[torch.Tensor] = None,
    out: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """y [N] = (x / s) @ w_hat^T for x [K] (fp16 or bf16)."""
    if x.dtype not in _DTYPE or x.numel() != K:
        raise ValueError("x must be fp16/bf16 with K elements")
    _check_packed(packed, scales, zeros, N, K, bits, group_size)
    _check_act_scale(act_scale, K)
    if out is not None:
        _check_out(out, (N,), x.dtype, "out")
    y = out if out is not None else torch.empty((N,), dtype=x.dtype, device=x.device)
    _require_gpu(x, act_scale, packed, scales, zeros, y)
    st = _lib.call("woq_w4a16_gemv", x.data_ptr(), _DTYPE[x.dtype], _ptr(act_scale), packed.data_ptr(),
                   scales.data_ptr(), _ptr(zeros), N, K, bits, group_size, int(zeros is not None), y.data_ptr(),
                   None, 0, _stream(x))
    _lib.check(st, "woq_w4a16_gemv")
    return y


def gemm(
    X: torch.Tensor,
    packed: torch.Tensor,
    scales: torch.Tensor,
    zeros: Optional[torch.Tensor],
    N: int,
    K: int,
    bits: int = 4,
    group_size: int = 128,
    act_scale: Optional[torch.Tensor] = None,
    out: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """Y [M, N] = (X / s) @ w_hat^T for X [M, K] (fp16 or bf16)."""
    if X.dtype not in _DTYPE or X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be fp16/bf16 [M, K]")
    M = X.shape[0]
    _check_packed(packed, scales, zeros, N, K, bits, group_size)
    _check_act_scale(act_scale, K)
    if out is not None:
        _check_out(out, (M, N), X.dtype, "out")
    Y = out if out is not None else torch.empty((M, N), dtype=X.dtype, device=X.device)
    _require_gpu(X, act_scale, packed, scales, zeros, Y)
    # bf16 X can run on the fp16 kernels through a per-row rescale: the row
    # factors and the rescaled fp16 copy of X live in a workspace
    ws, ws_bytes = None, 0
    if X.dtype == torch.bfloat16:
        ws_bytes = int(_lib.call("woq_workspace_bytes", M, N, K, bits, group_size))
        if ws_bytes:
            ws = _workspace(X.device, _stream(X), ws_bytes)
    st = _lib.call("woq_w4a16_gemm", X.data_ptr(), _DTYPE[X.dtype], _ptr(act_scale), packed.data_ptr(),
                   scales.data_ptr(), _ptr(zeros), M, N, K, bits, group_size, int(zeros is not None), Y.data_ptr(),
                   _ptr(ws), ws_bytes, _stream(X))
    _lib.check(st, "woq_w4a16_gemm")
    return Y


def dequantize(
    packed: torch.Tensor,
    scales: torch.Tensor,
    zeros: Optional[torch.Tensor],
    N: int,
    K: int,
    bits: int = 4,
    group_size: int = 128,
) -> torch.Tensor:
    """w_hat = (u - Z) * S as float32 [N, K]."""
    _check_packed(packed, scales, zeros, N, K, bits, group_size)
    out = torch.empty((N, K), dtype=torch.float32, device=packed.device)
    _require_gpu(packed, scales, zeros, out)
    st = _lib.call("woq_dequantize", packed.data_ptr(), scales.data_ptr(), _ptr(zeros), N, K, bits, group_size,
                   int(zeros is not None), out.data_ptr(), _stream(packed))
    _lib.check(st, "woq_dequantize")
    return out


def quantize_pack_many(
    Ws: Sequence[torch.Tensor],
    bits: int = 4,
    group_size: int = 128,
    asymmetric: bool = True,
    act_scales: Optional[Sequence[Optional[torch.Tensor]]] = None,
    outs: Optional[Sequence[Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]]] = None,
):
    """quantize_pack over several fp16 matrices [N_i, K_i] that share bits,
    group_size and asymmetric, through woq_quantize_pack_many (up to 32
    matrices per launch).  act_scales[i] (or None) is matrix i's AWQ scale;
    outs[i], if given, its (packed, scales, zeros | None).  Returns one
    (packed, scales, zeros | None) per matrix, byte-equal to quantize_pack's."""
    if not Ws:
        raise ValueError("need at least one matrix")
    if act_scales is not None and len(act_scales) != len(Ws):
        raise ValueError("act_scales must have one entry per matrix")
    if outs is not None and len(outs) != len(Ws):
        raise ValueError("outs must have one entry per matrix")
    results = []
    descs = (_lib.QMatrix * len(Ws))()
    for i, W in enumerate(Ws):
        if W.dtype != torch.float16 or W.dim() != 2:
            raise ValueError(f"matrix {i}: W must be a 2-D float16 tensor")
        N, K = W.shape
        _check_quantizer(N, K, bits, group_size)
        s = None if act_scales is None else act_scales[i]
        _check_act_scale(s, K)
        if outs is None:
            packed = torch.empty((N, K * bits // 8), dtype=torch.uint8, device=W.device)
            scales = torch.empty((N, K // group_size), dtype=torch.float16, device=W.device)
            zeros = torch.empty_like(scales) if asymmetric else None
        else:
            packed, scales, zeros = outs[i]
            if (zeros is not None) != bool(asymmetric):
                raise ValueError(f"matrix {i}: out must hold zeros exactly when asymmetric")
            _check_packed(packed, scales, zeros, N, K, bits, group_size)
        _require_gpu(Ws[0], W, s, packed, scales, zeros)
        descs[i] = _lib.QMatrix(W.data_ptr(), _ptr(s), packed.data_ptr(), scales.data_ptr(), _ptr(zeros), N, K)
        results.append((packed, scales, zeros))
    st = _lib.call("woq_quantize_pack_many", ctypes.addressof(descs), len(Ws), bits, group_size, int(asymmetric),
                   _stream(Ws[0]))
    _lib.check(st, "woq_quantize_pack_many")
    return results


def quantize_pack_fused(
    Ws: Sequence[torch.Tensor],
    bits: int = 4,
    group_size: int = 128,
    asymmetric: bool = True,
    act_scale: Optional[torch.Tensor] = None,
):
    """Quantize several weight matrices that read the same input (q/k/v, or
    gate/up) into one packed set whose rows are theirs, stacked: matrix i
    fills rows [sum(N_<i), sum(N_<=i)) of each output, written in place by one
    woq_quantize_pack_many call.  A single gemv/gemm over N = sum(N_i)
    then serves all of them.  Returns (packed, scales, zeros | None, sizes)."""
    if not Ws:
        raise ValueError("need at least one matrix")
    K = Ws[0].shape[1]
    if any(W.dim() != 2 or W.shape[1] != K for W in Ws):
        raise ValueError("all matrices must be [N_i, K] with the same K")
    sizes = [int(W.shape[0]) for W in Ws]
    N = sum(sizes)
    dev = Ws[0].device
    packed = torch.empty((N, packed_bytes(1, K, bits)), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, K // group_size), dtype=torch.float16, device=dev)
    zeros = torch.empty_like(scales) if asymmetric else None
    outs, row = [], 0
    for n in sizes:
        outs.append((packed[row:row + n], scales[row:row + n], None if zeros is None else zeros[row:row + n]))
        row += n
    quantize_pack_many(Ws, bits, group_size, asymmetric, [act_scale] * len(Ws), outs)
    return packed, scales, zeros, sizes


def gemv_fused(
    x: torch.Tensor,
    packed: torch.Tensor,
    scales: torch.Tensor,
    zeros: Optional[torch.Tensor],
    sizes: Sequence[int],
    K: int,
    bits: int = 4,
    group_size: int = 128,
    act_scale: Optional[torch.Tensor] = None,
) -> Tuple[torch.Tensor, ...]:
    """One GEMV launch over a set made by quantize_pack_fused; returns the
    outputs of the individual matrices as views of one [sum(N_i)] vector."""
    y = gemv(x, packed, scales, zeros, sum(sizes), K, bits, group_size, act_scale)
    return tuple(y.split(list(sizes)))


def awq_search(
    X: torch.Tensor,
    W: torch.Tensor,
    bits: int = 4,
    group_size: int = 128,
    asymmetric: bool = True,
    n_grid: int = 20,
):
    """AWQ exponent search for one layer on calibration activations X [T, K]
    (fp16) and weights W [N, K] (fp16).  Returns (losses fp64 [n_grid],
    best_scale fp32 [K], best_index int32 [1]), all on the device; the
    workspace is allocated here (PyTorch memory) and released on return."""
    if X.dtype != torch.float16 or W.dtype != torch.float16 or X.dim() != 2 or W.dim() != 2:
        raise ValueError("X and W must be 2-D float16 tensors")
    T, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("X and W must share K")
    nbytes = int(_lib.call("woq_awq_search_workspace_bytes", T, N, K, bits, group_size, int(asymmetric)))
    if nbytes == 0:
        raise ValueError("unsupported shape or quantizer for awq_search")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=X.device)
    losses = torch.empty(n_grid, dtype=torch.float64, device=X.device)
    best_scale = torch.empty(K, dtype=torch.float32, device=X.device)
    best_index = torch.empty(1, dtype=torch.int32, device=X.device)
    _require_gpu(X, W, ws, losses, best_scale, best_index)
    st = _lib.call("woq_awq_search", X.data_ptr(), W.data_ptr(), T, N, K, bits, group_size, int(asymmetric), n_grid,
                   losses.data_ptr(), best_scale.data_ptr(), best_index.data_ptr(), ws.data_ptr(), nbytes,
                   _stream(X))
    _lib.check(st, "woq_awq_search")
    return losses, best_scale, best_index


def gptq(
    X: torch.Tensor,
    W: torch.Tensor,
    bits: int = 4,
    group_size: int = 128,
    asymmetric: bool = True,
    damp: float = 0.01,
):
    """GPTQ of fp16 W [N, K] on fp16 calibration activations X [T, K] ->
    (packed, scales, zeros | None) in the same layout as quantize_pack.  The
    workspace is allocated here (PyTorch memory) and released on return."""
    if X.dtype != torch.float16 or W.dtype != torch.float16 or X.dim() != 2 or W.dim() != 2:
        raise ValueError("X and W must be 2-D float16 tensors")
    T, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("X and W must share K")
    nbytes = int(_lib.call("woq_gptq_workspace_bytes", T, N, K, bits, group_size))
    if nbytes == 0:
        raise ValueError("unsupported shape or quantizer for gptq")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=X.device)
    packed = torch.empty((N, K * bits // 8), dtype=torch.uint8, device=W.device)
    scales = torch.empty((N, K // group_size), dtype=torch.float16, device=W.device)
    zeros = torch.empty_like(scales) if asymmetric else None
    _require_gpu(X, W, ws, packed, scales, zeros)
    st = _lib.call("woq_gptq_quantize_pack", X.data_ptr(), W.data_ptr(), T, N, K, bits, group_size, int(asymmetric),
                   float(damp), packed.data_ptr(), scales.data_ptr(), _ptr(zeros), ws.data_ptr(), nbytes, _stream(X))
    _lib.check(st, "woq_gptq_quantize_pack")
    return packed, scales, zeros
