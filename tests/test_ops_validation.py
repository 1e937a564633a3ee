"""The PyTorch binding rejects mis-shaped or mis-typed tensors before any
library call (CPU tensors: each case fails validation first, so nothing
reaches HIP)."""
import pytest
import torch

from weight_only_quantization_quantize_amd import ops

N, K, G = 16, 256, 128


def _set(bits=4, asym=True):
    packed = torch.zeros(N * K * bits // 8, dtype=torch.uint8)
    scales = torch.zeros(N, K // G, dtype=torch.float16)
    zeros = torch.zeros(N, K // G, dtype=torch.float16) if asym else None
    return packed, scales, zeros


def _ok_call(fn, **kw):
    """The call with valid shapes fails only at the device check."""
    with pytest.raises(ValueError, match="GPU tensors only"):
        fn(**kw)


def test_valid_shapes_reach_the_device_check():
    p, s, z = _set()
    _ok_call(lambda: ops.gemv(torch.zeros(K, dtype=torch.float16), p, s, z, N, K, 4, G))
    _ok_call(lambda: ops.gemm(torch.zeros(3, K, dtype=torch.float16), p, s, z, N, K, 4, G))
    _ok_call(lambda: ops.quantize_pack(torch.zeros(N, K, dtype=torch.float16), 4, G, True, out=(p, s, z)))
    _ok_call(lambda: ops.dequantize(p, s, z, N, K, 4, G))


@pytest.mark.parametrize("case, needle", [
    ("packed_short", "packed must be uint8"),
    ("packed_dtype", "packed must be uint8"),
    ("packed_3bit_size_for_4bit", "packed must be uint8"),
    ("scales_short", "scales must be float16"),
    ("scales_dtype", "scales must be float16"),
    ("zeros_short", "zeros must be float16"),
    ("act_scale_dtype", "act_scale must be float32"),
    ("act_scale_shape", "act_scale must be float32"),
    ("out_dtype", "out must be"),
    ("out_shape", "out must be"),
    ("bits", "bits must be 3 or 4"),
    ("group", "group_size"),
])
@pytest.mark.parametrize("op", ["gemv", "gemm"])
def test_matmul_rejects(op, case, needle):
    p, s, z = _set()
    act, out, bits, g = None, None, 4, G
    if case == "packed_short":
        p = p[:-16]
    elif case == "packed_dtype":
        p = p.view(torch.int8)
    elif case == "packed_3bit_size_for_4bit":
        p = torch.zeros(N * K * 3 // 8, dtype=torch.uint8)
    elif case == "scales_short":
        s = s[:-1]
    elif case == "scales_dtype":
        s = s.float()
    elif case == "zeros_short":
        z = z[:-1]
    elif case == "act_scale_dtype":
        act = torch.ones(K, dtype=torch.float16)
    elif case == "act_scale_shape":
        act = torch.ones(K + 1, dtype=torch.float32)
    elif case == "out_dtype":
        out = torch.zeros((N,) if op == "gemv" else (3, N), dtype=torch.float32)
    elif case == "out_shape":
        out = torch.zeros((N + 1,) if op == "gemv" else (3, N + 1), dtype=torch.float16)
    elif case == "bits":
        bits = 5
    elif case == "group":
        g = 96
    with pytest.raises(ValueError, match=needle):
        if op == "gemv":
            ops.gemv(torch.zeros(K, dtype=torch.float16), p, s, z, N, K, bits, g, act, out=out)
        else:
            ops.gemm(torch.zeros(3, K, dtype=torch.float16), p, s, z, N, K, bits, g, act, out=out)


@pytest.mark.parametrize("case, needle", [
    ("packed_short", "packed must be uint8"),
    ("scales_dtype", "scales must be float16"),
    ("zeros_missing", "zeros exactly when asymmetric"),
    ("act_scale_shape", "act_scale must be float32"),
    ("bits", "bits must be 3 or 4"),
])
def test_quantize_pack_rejects(case, needle):
    W = torch.zeros(N, K, dtype=torch.float16)
    p, s, z = _set()
    act = None
    if case == "packed_short":
        p = p[:-1]
    elif case == "scales_dtype":
        s = s.float()
    elif case == "zeros_missing":
        z = None
    elif case == "act_scale_shape":
        act = torch.ones(K // 2, dtype=torch.float32)
    bits = 5 if case == "bits" else 4
    with pytest.raises(ValueError, match=needle):
        ops.quantize_pack(W, bits, G, True, act, out=(p, s, z))
