"""The element-wise output checker used by the GPU parity tests, on the CPU.

It must accept outputs carrying the roundings the kernels perform (fp16 x / s,
fp32 sums of magic-offset summands, fp16 / bf16 output) and reject an output
with one element off by a few percent.
"""
import numpy as np
import pytest

from oracle import woq_oracle as O
from tests.parity_bound import check_elementwise, output_bound


def _case(seed=0, M=3, N=48, K=1024, bits=4, G=128, awq=True):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((M, K)).astype(np.float16)
    s = np.exp(rng.uniform(-1, 1, K)).astype(np.float32) if awq else None
    q = O.quantize(W, bits, G, True, s)
    w_hat = O.dequantize(q)
    y_ref = O.gemm(X.astype(np.float64), w_hat, s)
    return X, s, q, w_hat, y_ref


def _fp32_magic_sum(X, s, q):
    """A deliberately rough fp32 evaluation: x / s rounded to fp16, summands
    x' (1024 + u) added one at a time in fp32 over each group, then the offset
    (1024 + Z) sum x' removed and the group scaled, groups added in fp32."""
    G = q.group_size
    xs = (X.astype(np.float32) / s).astype(np.float16).astype(np.float32) if s is not None else X.astype(np.float32)
    M, K = xs.shape
    N = q.codes.shape[0]
    y = np.zeros((M, N), np.float32)
    for g in range(K // G):
        sl = slice(g * G, (g + 1) * G)
        part = np.zeros((M, N), np.float32)
        xsum = np.zeros((M, 1), np.float32)
        for k in range(sl.start, sl.stop):
            part = part + xs[:, k:k + 1] * (np.float32(1024) + q.codes[None, :, k].astype(np.float32))
            xsum = xsum + xs[:, k:k + 1]
        corr = part - (np.float32(1024) + q.zeros[:, g].astype(np.float32))[None, :] * xsum
        y = y + q.scales[:, g].astype(np.float32)[None, :] * corr
    return y


@pytest.mark.parametrize("out", ["f16", "bf16"])
def test_checker_accepts_kernel_like_roundings(out):
    X, s, q, w_hat, y_ref = _case()
    bound = output_bound(X.astype(np.float64), w_hat, q.scales, 4, 128, s, y_ref, out)
    y32 = _fp32_magic_sum(X, s, q)
    if out == "f16":
        y = y32.astype(np.float16).astype(np.float64)
    else:
        b = (y32.view(np.uint32) + 0x7FFF + ((y32.view(np.uint32) >> 16) & 1)) >> 16   # RNE to bf16
        y = O.bf16_bits_to_f64(b.astype(np.uint16))
    ok, worst, _ = check_elementwise(y, y_ref, bound)
    assert ok, worst
    # the exact result rounded once to the output type passes with room
    ok, worst, _ = check_elementwise(y_ref.astype(np.float32).astype(np.float16), y_ref, bound)
    assert ok and worst < 0.5


@pytest.mark.parametrize("rel", [0.03, 0.10, -0.10])
def test_checker_rejects_one_element_off_by_a_few_percent(rel):
    X, s, q, w_hat, y_ref = _case(seed=1, M=2, N=64, K=2048)
    bound = output_bound(X.astype(np.float64), w_hat, q.scales, 4, 128, s, y_ref, "f16")
    y = y_ref.astype(np.float16).astype(np.float64)
    # the output of largest magnitude, perturbed by rel
    i = np.unravel_index(int(np.argmax(np.abs(y_ref))), y_ref.shape)
    bad = y.copy()
    bad[i] = y_ref[i] * (1 + rel)
    ok, worst, where = check_elementwise(bad, y_ref, bound)
    assert not ok and where == i and worst > 1.0


def test_checker_rejects_a_wrong_row_the_l2_bar_misses():
    # N = 4096 outputs, one row scaled by 1.1 (the case the whole-output bar
    # lets through): relative L2 stays under 2e-3, the element bound trips
    X, s, q, w_hat, y_ref = _case(seed=2, M=1, N=4096, K=1024, awq=False)
    bound = output_bound(X.astype(np.float64), w_hat, q.scales, 4, 128, None, y_ref, "f16")
    n = int(np.argsort(np.abs(y_ref[0]))[len(y_ref[0]) // 2])   # a row of median magnitude
    bad = y_ref.astype(np.float16).astype(np.float64)
    bad[0, n] *= 1.1
    assert O.rel_l2(bad, y_ref) < 2e-3
    ok, _, where = check_elementwise(bad, y_ref, bound)
    assert not ok and where == (0, n)


def test_checker_rejects_non_finite_outputs():
    X, s, q, w_hat, y_ref = _case(seed=3, M=1, N=8)
    bound = output_bound(X.astype(np.float64), w_hat, q.scales, 4, 128, s, y_ref, "f16")
    bad = y_ref.copy()
    bad[0, 3] = np.nan
    assert not check_elementwise(bad, y_ref, bound)[0]
