"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print, exact rational arithmetic, brute force over every code, closed
forms and invariants.  None of these tests needs a GPU.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import woq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16(a):
    return np.asarray(a, dtype=np.float32).astype(np.float16)


def _random_groups(rng, N, K, std=0.02, outlier_frac=0.01):
    w = rng.standard_normal((N, K)).astype(np.float32) * np.float32(std)
    m = rng.random((N, K)) < outlier_frac
    w[m] = rng.standard_normal(int(m.sum())).astype(np.float32) * np.float32(0.5)
    return w.astype(np.float16)


# ---------------------------------------------------------------------------
# Worked example printed on "LLM Quantization: 160GB Model on a Laptop",
# section "Symmetric Quantization".
# ---------------------------------------------------------------------------

def test_worked_example_symmetric():
    g = _load("worked_example_symmetric.json")
    w = _f16(g["values"])[None, :]
    q = O.quantize(w, g["bits"], len(g["values"]), asymmetric=False)
    signed = q.codes.astype(int)[0] - 2 ** (g["bits"] - 1)
    assert signed.tolist() == g["quantized"]
    S = float(q.scales[0, 0])
    tol = 0.5 * 10 ** -g["print_decimals"]
    assert abs(S - g["scale_approx"]) <= tol
    w_hat = O.dequantize(q)[0]
    assert np.all(np.abs(w_hat - np.array(g["dequantized_approx"])) <= tol)
    err = np.mean(np.abs(w_hat - w[0].astype(np.float64)) / np.abs(w[0].astype(np.float64)))
    assert round(100 * err) == g["average_error_percent"]


def test_worked_example_in_a_zero_padded_group_of_128():
    # Zero padding changes neither the absmax nor the first six codes.
    g = _load("worked_example_symmetric.json")
    w = np.zeros((1, 128), np.float16)
    w[0, :6] = _f16(g["values"])
    q = O.quantize(w, 4, 128, asymmetric=False)
    assert (q.codes[0, :6].astype(int) - 8).tolist() == g["quantized"]
    assert np.all(q.codes[0, 6:] == 8)


def test_worked_example_asymmetric_error_in_page_range():
    # "LLM Quantization ...", section "Asymmetric Quantization": average error
    # drops to 5-10% (a loose claim; our zero-point form lands inside it).
    g = _load("worked_example_symmetric.json")
    w = _f16(g["values"])[None, :]
    q = O.quantize(w, 4, 6, asymmetric=True)
    w_hat = O.dequantize(q)[0]
    err = np.mean(np.abs(w_hat - w[0].astype(np.float64)) / np.abs(w[0].astype(np.float64)))
    assert 0.05 <= err <= 0.10
    assert q.codes.min() == 0  # the minimum lands on the bottom code


# ---------------------------------------------------------------------------
# Exact rational reference of the code decision (fp16 inputs, no fold).
# For an fp16 w and an fp16 S the exact quotient is never within one binary32
# rounding of a half-integer unless it is one, so rne(fl32(w/S)) equals the
# exactly rounded quotient.
# ---------------------------------------------------------------------------

def _round_half_even(fr: Fraction) -> int:
    return round(fr)  # Python rounds Fractions half-to-even


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("asym", [False, True])
def test_codes_equal_exact_rational_rounding(bits, asym):
    rng = np.random.default_rng(11 + bits + 10 * asym)
    W = _random_groups(rng, 6, 256)
    q = O.quantize(W, bits, 128, asym)
    for n in range(W.shape[0]):
        for gi in range(2):
            S = Fraction(float(q.scales[n, gi]))
            grp = [Fraction(float(v)) for v in W[n, 128 * gi:128 * (gi + 1)]]
            if asym:
                Z = _round_half_even(-min(grp) / S)
                Z = min(max(Z, 0), 2 ** bits - 1)
                assert float(q.zeros[n, gi]) == Z
                ref = [min(max(_round_half_even(v / S) + Z, 0), 2 ** bits - 1) for v in grp]
            else:
                h = 2 ** (bits - 1)
                ref = [min(max(_round_half_even(v / S), -h), h - 1) + h for v in grp]
            assert q.codes[n, 128 * gi:128 * (gi + 1)].tolist() == ref


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("asym", [False, True])
def test_scale_is_fp16_rounding_of_exact_ratio(bits, asym):
    rng = np.random.default_rng(5 + bits)
    W = _random_groups(rng, 8, 512)
    q = O.quantize(W, bits, 128, asym)
    g = W.astype(np.float64).reshape(8, 4, 128)
    if asym:
        exact = (g.max(2) - g.min(2)) / (2 ** bits - 1)
    else:
        exact = np.abs(g).max(2) / (2 ** (bits - 1) - 1)
    S = q.scales.astype(np.float64)
    # within half an fp16 ulp (plus the binary32 intermediate rounding)
    ulp = np.spacing(q.scales).astype(np.float64)
    assert np.all(np.abs(S - exact) <= 0.5 * ulp + exact * 2.0 ** -23)


# ---------------------------------------------------------------------------
# Brute force: every code is the grid point nearest to w (round-to-nearest).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("folded", [False, True])
def test_codes_are_nearest_grid_points(bits, asym, folded):
    rng = np.random.default_rng(100 + bits + 2 * asym + 4 * folded)
    N, K = 5, 384
    W = _random_groups(rng, N, K)
    s = (rng.random(K).astype(np.float32) * 3 + 0.25) if folded else None
    q = O.quantize(W, bits, 128, asym, s)
    w = O.fold_act_scale(W, s).astype(np.float64)
    S = np.repeat(q.scales.astype(np.float64), 128, axis=1)
    Z = np.repeat(q.zeros.astype(np.float64), 128, axis=1) if asym else 2.0 ** (bits - 1)
    Z = np.broadcast_to(Z, w.shape)
    cand = np.arange(2 ** bits, dtype=np.float64)
    grid = (cand[None, None, :] - Z[..., None]) * S[..., None]          # [N,K,codes]
    dist = np.abs(w[..., None] - grid)
    best = dist.min(axis=2)
    got = np.take_along_axis(dist, q.codes[..., None].astype(np.int64), axis=2)[..., 0]
    # the fp32 division can only move a decision when w/S is within one
    # binary32 rounding of a half-integer
    slack = np.abs(w) * 2.0 ** -22
    assert np.all(got <= best + slack)
    # exact ties (two grid points equally near) go to the even integer q = u - Z
    ties = np.sum(dist == best[..., None], axis=2) > 1
    if ties.any():
        assert np.all(((q.codes.astype(np.int64) - Z.astype(np.int64))[ties] % 2) == 0)


@pytest.mark.parametrize("bits", [3, 4])
def test_exact_ties_round_half_to_even(bits):
    # S is a power of two when absmax = qmax * 2^-6; values (j + 1/2) S are ties.
    qmax = 2 ** (bits - 1) - 1
    S = 2.0 ** -6
    vals = [qmax * S] + [(j + 0.5) * S for j in range(-qmax, qmax - 1)]
    vals += [0.0] * (128 - len(vals))
    W = np.array([vals], dtype=np.float16)
    assert np.all(W.astype(np.float64) == np.array([vals]))
    q = O.quantize(W, bits, 128, asymmetric=False)
    assert float(q.scales[0, 0]) == S
    signed = q.codes[0].astype(int) - 2 ** (bits - 1)
    for j, v in enumerate(vals[1:1 + 2 * qmax - 1], start=1):
        lo = int(np.floor(v / S))
        expect = lo if lo % 2 == 0 else lo + 1
        assert signed[j] == expect


# ---------------------------------------------------------------------------
# Range, clipping and the dequantization error bound.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("asym", [False, True])
def test_codes_in_range_and_extremes_on_end_codes(bits, asym):
    rng = np.random.default_rng(7 * bits + asym)
    W = _random_groups(rng, 16, 1024)
    q = O.quantize(W, bits, 128, asym)
    assert q.codes.min() >= 0 and q.codes.max() <= 2 ** bits - 1
    g = W.astype(np.float64).reshape(16, 8, 128)
    c = q.codes.reshape(16, 8, 128).astype(int)
    if asym:
        # the group minimum lands on code 0, the maximum within one of the top
        assert np.all(np.take_along_axis(c, g.argmin(2)[..., None], 2) == 0)
        assert np.all(np.take_along_axis(c, g.argmax(2)[..., None], 2) >= 2 ** bits - 2)
    else:
        qmax = 2 ** (bits - 1) - 1
        top = np.take_along_axis(c, np.abs(g).argmax(2)[..., None], 2)[..., 0] - 2 ** (bits - 1)
        assert np.all(np.abs(top) == qmax)
        assert c.min() >= 1  # -2^(b-1) is never produced by absmax scaling


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("folded", [False, True])
def test_dequant_error_bound(bits, asym, folded):
    rng = np.random.default_rng(31 + bits + 2 * asym + 4 * folded)
    N, K = 32, 1024
    W = _random_groups(rng, N, K)
    s = (rng.random(K).astype(np.float32) * 3 + 0.25) if folded else None
    q = O.quantize(W, bits, 128, asym, s)
    w = O.fold_act_scale(W, s).astype(np.float64)
    err = np.abs(w - O.dequantize(q))
    S = np.repeat(q.scales.astype(np.float64), 128, axis=1)
    if asym:
        bound = S * (0.5 + (2 ** bits - 1) * 2.0 ** -11 + 2.0 ** -20)
    else:
        bound = S * (0.5 + 2.0 ** -20)
    assert np.all(err <= bound)


def test_group_size_trend():
    # "Quantising ...", section "Post-training methods for 4-bit weights": a
    # N(0, 0.02) row of 4096 with two 0.8 outliers; smaller groups reduce the
    # mean absolute error (the page prints no values, only the trend).
    rng = np.random.default_rng(0)
    row = rng.normal(0, 0.02, 4096)
    row[[10, 500]] = 0.8
    W = row.astype(np.float16)[None, :]
    errs = []
    for G in (4096, 128, 32):
        q = O.quantize(W, 4, G, asymmetric=False)
        errs.append(np.abs(O.dequantize(q) - W.astype(np.float64)).mean())
    assert errs[0] > errs[1] > errs[2]
    assert errs[0] > 3 * errs[1]


# ---------------------------------------------------------------------------
# Degenerate groups.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [3, 4])
def test_zero_group(bits):
    W = np.zeros((2, 256), np.float16)
    W[1, 128:] = _f16(np.linspace(-0.1, 0.1, 128))
    qs = O.quantize(W, bits, 128, asymmetric=False)
    assert float(qs.scales[0, 0]) == 0.0 and np.all(qs.codes[0] == 2 ** (bits - 1))
    assert np.all(O.dequantize(qs)[0] == 0)
    qa = O.quantize(W, bits, 128, asymmetric=True)
    # zero range -> range 1 ("CMU 11-868 L19-L20", section "absmax and zero-point")
    assert float(qa.scales[0, 0]) == float(np.float16(np.float32(1) / np.float32(2 ** bits - 1)))
    assert float(qa.zeros[0, 0]) == 0 and np.all(qa.codes[0, :128] == 0)
    assert np.all(O.dequantize(qa)[0, :128] == 0)


@pytest.mark.parametrize("c", [0.3, -0.3, 0.01, 2.0])
def test_constant_group_asymmetric(c):
    bits = 4
    W = np.full((1, 128), c, np.float16)
    q = O.quantize(W, bits, 128, asymmetric=True)
    S = float(np.float16(np.float32(1) / np.float32(15)))
    assert float(q.scales[0, 0]) == S
    cv = float(W[0, 0])
    Z = min(max(round(Fraction(-cv) / Fraction(S)), 0), 15)
    u = min(max(round(Fraction(cv) / Fraction(S)) + Z, 0), 15)
    assert float(q.zeros[0, 0]) == Z and np.all(q.codes == u)


def test_underflowing_scale():
    # absmax below 7 * 2^-25: the fp16 scale rounds to 0
    W = np.zeros((1, 128), np.float16)
    W[0, 3] = np.float16(2.0 ** -24)
    W[0, 9] = -np.float16(2.0 ** -24)
    qs = O.quantize(W, 4, 128, asymmetric=False)
    assert float(qs.scales[0, 0]) == 0 and np.all(qs.codes == 8)
    qa = O.quantize(W, 4, 128, asymmetric=True)
    assert float(qa.scales[0, 0]) == 0 and float(qa.zeros[0, 0]) == 0 and np.all(qa.codes == 0)


# ---------------------------------------------------------------------------
# Packed layout v2 (3-bit pairs kept whole; 4-bit as in v1).
# ---------------------------------------------------------------------------

def test_layout_v2_fixed_words():
    g = _load("layout_v2_words.json")
    u4 = (np.arange(16) % 16).astype(np.uint8)[None, :]
    w4 = O.pack_v2(u4, 4).view("<u4")[0].tolist()
    assert w4 == [int(h, 16) for h in g["four_bit"]["words_hex"]]
    u3 = (np.arange(32) % 8).astype(np.uint8)[None, :]
    w3 = O.pack_v2(u3, 3).view("<u4")[0].tolist()
    assert w3 == [int(h, 16) for h in g["three_bit"]["words_hex"]]


@pytest.mark.parametrize("bits", [3, 4])
def test_layout_v2_round_trip_and_single_code(bits):
    rng = np.random.default_rng(bits)
    u = rng.integers(0, 2 ** bits, size=(7, 256), dtype=np.uint8)
    p = O.pack_v2(u, bits)
    assert p.shape == (7, 256 * bits // 8)
    assert np.array_equal(O.unpack_v2(p, bits, 256), u)
    # a lone code lands on exactly the bits the definition names
    for k in (0, 1, 2, 7, 13, 28, 29, 30, 31, 200, 255):
        for code in range(1, 2 ** bits):
            one = np.zeros((1, 256), np.uint8)
            one[0, k] = code
            words = O.pack_v2(one, bits).view("<u4")[0]
            if bits == 4:
                j, r = divmod(k, 8)
                t, h = divmod(r, 2)
                expect = {j: code << (16 * h + 4 * t)}
            else:
                j, i = divmod(k, 32)
                t, h = divmod(i, 2)
                if t < 15:
                    expect = {3 * j + t // 5: code << (16 * h + 3 * (t % 5))}
                else:
                    expect = {3 * j + b: 1 << (16 * h + 15) for b in range(3) if (code >> b) & 1}
            nz = {int(i): int(v) for i, v in enumerate(words) if v}
            assert nz == expect, (k, code)


def test_layout_v2_three_bit_pairs_decode_with_one_mask():
    # the property the layout is for: pair t < 15 of a unit is one 3-bit field
    # in each 16-bit half of its word, (w >> 3 (t % 5)) & 0x00070007
    rng = np.random.default_rng(9)
    u = rng.integers(0, 8, size=(3, 64), dtype=np.uint8)
    words = O.pack_v2(u, 3).view("<u4").reshape(3, 2, 3)
    for j in range(2):
        for t in range(15):
            f = (words[:, j, t // 5] >> (3 * (t % 5))) & 0x00070007
            assert np.array_equal(f & 0xFFFF, u[:, 32 * j + 2 * t])
            assert np.array_equal(f >> 16, u[:, 32 * j + 2 * t + 1])


# ---------------------------------------------------------------------------
# Dequantization and the GEMV/GEMM against exact rational arithmetic.
# ---------------------------------------------------------------------------

def test_dequant_exact():
    rng = np.random.default_rng(3)
    W = _random_groups(rng, 3, 256)
    q = O.quantize(W, 4, 128, asymmetric=True)
    w_hat = O.dequantize(q)
    for n in range(3):
        for k in range(0, 256, 17):
            g = k // 128
            ref = (Fraction(int(q.codes[n, k])) - Fraction(float(q.zeros[n, g]))) * Fraction(float(q.scales[n, g]))
            assert Fraction(float(w_hat[n, k])) == ref


@pytest.mark.parametrize("with_scale", [False, True])
def test_gemm_against_fractions(with_scale):
    rng = np.random.default_rng(17)
    M, N, K = 2, 3, 256
    W = _random_groups(rng, N, K)
    X = rng.standard_normal((M, K)).astype(np.float16)
    s = (rng.random(K).astype(np.float32) + 0.5) if with_scale else None
    q = O.quantize(W, 4, 128, asymmetric=True, act_scale=s)
    Y = O.gemm(X.astype(np.float64), O.dequantize(q), s)
    assert Y.shape == (M, N)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = k // 128
                wk = (Fraction(int(q.codes[n, k])) - Fraction(float(q.zeros[n, g]))) * Fraction(float(q.scales[n, g]))
                xk = Fraction(float(X[m, k]))
                if s is not None:
                    xk /= Fraction(float(s[k]))
                acc += xk * wk
            assert abs(float(Y[m, n]) - float(acc)) <= 1e-12 * max(1.0, abs(float(acc)))


def test_gemm_constant_codes_closed_form():
    # constant u, S, Z -> y_m = S (u - Z) sum_k x_mk
    K = 512
    q = O.Quantized(np.full((4, K), 11, np.uint8), np.full((4, K // 128), 0.0625, np.float16),
                    np.full((4, K // 128), 3, np.float16), 4, 128, True)
    X = np.random.default_rng(2).standard_normal((3, K)).astype(np.float16).astype(np.float64)
    Y = O.gemm(X, O.dequantize(q))
    assert np.allclose(Y, (0.0625 * 8 * X.sum(1))[:, None] * np.ones((1, 4)), rtol=1e-14, atol=0)


def test_bf16_bits_exact():
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x0000, 0x8000, 0x7F7F], np.uint16)
    vals = O.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -2.0 and vals[3] == 0.0
    assert vals[2] == 3.140625
    assert vals[5] == 255 * 2.0 ** 120   # exponent 254, mantissa 127/128


# ---------------------------------------------------------------------------
# The AWQ fold.
# ---------------------------------------------------------------------------

def test_awq_fold_identity_without_quantization():
    # (X diag(s)^-1)(diag(s) W) = X W ("Quantising ...", section "Why LLMs are
    # hard to quantise"), to fp64 rounding, with quantization bypassed.
    rng = np.random.default_rng(4)
    W = _random_groups(rng, 8, 256)
    X = rng.standard_normal((3, 256)).astype(np.float16)
    s = rng.random(256).astype(np.float32) * 4 + 0.1
    Wf = O.fold_act_scale(W, s).astype(np.float64)
    Y = O.gemm(X.astype(np.float64), Wf, s)
    Yref = X.astype(np.float64) @ W.astype(np.float64).T
    assert O.rel_l2(Y, Yref) < 1e-6


def test_awq_scaling_a_non_max_channel_shrinks_its_error():
    # Lab 4 Question 2 of "MIT 6.5940 Lab 4 + Lab 5": scaling a salient channel
    # by s while the group max stays put divides that weight's error by ~s.
    rng = np.random.default_rng(9)
    e1s, e2s = [], []
    for trial in range(50):
        w = (rng.standard_normal(128) * 0.02).astype(np.float16)
        w[0] = np.float16(0.1)            # the group max, unchanged by scaling
        j = 5
        w[j] = np.float16(0.013 + 0.0005 * trial)
        W = w[None, :]
        s = np.ones(128, np.float32)
        s[j] = 2.0
        q1 = O.quantize(W, 3, 128, asymmetric=False)
        q2 = O.quantize(W, 3, 128, asymmetric=False, act_scale=s)
        assert q1.scales[0, 0] == q2.scales[0, 0]
        S = float(q1.scales[0, 0])
        e2 = abs(O.dequantize(q2)[0, j] / 2.0 - float(w[j]))
        assert e2 <= S / 4 * (1 + 1e-6)
        e1s.append(abs(O.dequantize(q1)[0, j] - float(w[j])))
        e2s.append(e2)
    # on average the error roughly halves (about S/4 unscaled, S/8 scaled)
    assert np.mean(e2s) < 0.75 * np.mean(e1s)


# ---------------------------------------------------------------------------
# AWQ exponent search ("MIT 6.5940 Lab 4 + Lab 5", Question 2; the layer-wise
# reconstruction objective of "Quantising Large Language Models ...").
# ---------------------------------------------------------------------------
def _awq_case(seed, T=48, K=256, N=24, outliers=8):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, K)).astype(np.float32)
    ch = rng.choice(K, outliers, replace=False)
    X[:, ch] *= 50.0
    W = (rng.standard_normal((N, K)).astype(np.float32) * 0.02).astype(np.float16)
    return X.astype(np.float16).astype(np.float64), W


def test_awq_scale_closed_forms():
    X, _ = _awq_case(1)
    m = O.awq_channel_mean(X)
    # alpha = 0 is plain RTN: every scale is exactly 1
    assert np.all(O.awq_scale_for(m, 0.0) == np.float32(1))
    # alpha = 1 is the mean |x| itself (rounded once to fp32)
    brute = np.array([sum(abs(float(X[t, k])) for t in range(X.shape[0])) / X.shape[0] for k in range(X.shape[1])])
    assert np.array_equal(O.awq_scale_for(m, 1.0), brute.astype(np.float32))
    # alpha = 1/2 is the square-root scale the LLaMA-shaped workload uses as its
    # input AWQ scale (written independently in the input generator)
    from weight_only_quantization_quantize_amd import synth
    ch = synth.outlier_channels(512, 3100)
    s_gen = synth.awq_scale(512, 3200, ch)
    x_cal = synth.to_f16(synth.activations_f32(synth.CALIBRATION_TOKENS, 512, 3200, ch)).astype(np.float64)
    s_half = O.awq_scale_for(O.awq_channel_mean(x_cal), 0.5)
    assert np.max(np.abs(s_half.astype(np.float64) / s_gen.astype(np.float64) - 1)) < 2 ** -22


def test_awq_loss_against_exact_rationals():
    # The loss, term by term in exact rational arithmetic, from the oracle's own
    # codes / scales / zeros: X W^T and (X / s) w_hat^T, differenced and squared.
    X, W = _awq_case(2, T=3, K=64, N=2, outliers=2)
    m = O.awq_channel_mean(X)
    for alpha in (0.0, 0.5):
        s = O.awq_scale_for(m, alpha)
        q = O.quantize(W, 4, 32, True, s)
        total = Fraction(0)
        for t in range(3):
            for n in range(2):
                y_ref = sum(Fraction(float(X[t, k])) * Fraction(float(W[n, k])) for k in range(64))
                y_q = Fraction(0)
                for k in range(64):
                    g = k // 32
                    w_hat = (Fraction(int(q.codes[n, k])) - Fraction(float(q.zeros[n, g]))) * Fraction(float(q.scales[n, g]))
                    y_q += Fraction(float(X[t, k])) / Fraction(float(s[k])) * w_hat
                total += (y_ref - y_q) ** 2
        got = O.awq_loss(X, W, s, 4, 32, True)
        assert abs(got - float(total)) <= 1e-9 * float(total)


def test_awq_loss_scales_with_the_square_of_a_power_of_two():
    # Doubling W doubles every scale exactly and leaves the codes alone, so the
    # output error doubles and the loss is multiplied by exactly 4.
    X, W = _awq_case(3)
    m = O.awq_channel_mean(X)
    s = O.awq_scale_for(m, 0.35)
    W2 = (W.astype(np.float32) * 2).astype(np.float16)
    for bits, asym in ((4, True), (3, False)):
        assert O.awq_loss(X, W2, s, bits, 128, asym) == 4 * O.awq_loss(X, W, s, bits, 128, asym)


def test_awq_search_on_outlier_channels_falls_then_rises():
    # Scaling the channels that carry large activations lowers the error, and
    # too large an exponent inflates the group maxima again (Lab 4 Q2.2).
    X, W = _awq_case(4, T=64, K=512, N=32, outliers=8)
    losses, best, s = O.awq_search(X, W, 4, 128, True, 20)
    assert 0 < best < 19
    assert losses[best] < 0.5 * losses[0]
    assert losses[-1] > 2 * losses[best]
    assert np.array_equal(s, O.awq_scale_for(O.awq_channel_mean(X), best / 20))


def test_awq_search_equal_channel_means_keep_alpha_zero():
    # Every channel with mean |x| = 1 gives s = 1 for every exponent: all
    # errors are equal and the first exponent (plain RTN) is kept.
    rng = np.random.default_rng(6)
    X = np.where(rng.random((16, 256)) < 0.5, -1.0, 1.0)
    W = (rng.standard_normal((8, 256)) * 0.02).astype(np.float16)
    losses, best, s = O.awq_search(X, W, 4, 128, True, 10)
    assert np.all(losses == losses[0]) and best == 0 and np.all(s == 1)


# ---------------------------------------------------------------------------
# GPTQ ("CMU 11-868 L19-L20", section "The algorithm in four steps")
# ---------------------------------------------------------------------------
def _correlated_inputs(seed, T=192, K=256, rank=8):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, rank)) @ rng.standard_normal((rank, K)) + 0.3 * rng.standard_normal((T, K))
    return X.astype(np.float16).astype(np.float64)


def test_gptq_upper_factor_inverts_the_damped_hessian():
    X = _correlated_inputs(1)
    U, dead = O.gptq_upper_factor(X)
    H = 2 * X.T @ X
    H = H + 0.01 * np.mean(np.diag(H)) * np.eye(H.shape[0])
    assert not dead.any()
    assert np.allclose(np.tril(U, -1), 0) and np.all(np.diag(U) > 0)
    assert np.abs(U.T @ U @ H - np.eye(H.shape[0])).max() < 1e-8


@pytest.mark.parametrize("bits,asym,G", [(4, True, 128), (3, False, 32), (4, False, 64)])
def test_gptq_with_a_diagonal_hessian_is_rtn(bits, asym, G):
    # Uncorrelated input channels make (2 X^T X + lambda I)^-1 diagonal: no
    # error is pushed anywhere, and GPTQ must return the RTN codes exactly.
    rng = np.random.default_rng(bits + G)
    K, N = 256, 16
    X = np.diag(rng.uniform(0.5, 3.0, K)).astype(np.float16).astype(np.float64)
    W = _random_groups(rng, N, K)
    q = O.gptq(X, W, bits, G, asym)
    r = O.quantize(W, bits, G, asym)
    assert np.array_equal(q.codes, r.codes)
    assert np.array_equal(q.scales.view(np.uint16), r.scales.view(np.uint16))
    if asym:
        assert np.array_equal(q.zeros.view(np.uint16), r.zeros.view(np.uint16))


def test_gptq_errors_satisfy_w_minus_w_hat_equals_e_u():
    # Unrolling the column updates: W - w_hat = E U with E the scaled errors.
    X = _correlated_inputs(2)
    W = _random_groups(np.random.default_rng(2), 12, 256)
    q, E = O.gptq(X, W, 4, 128, True, return_errors=True)
    U, _ = O.gptq_upper_factor(X)
    D = W.astype(np.float64) - O.dequantize(q)
    assert np.abs(D - E @ U).max() < 1e-12


def test_gptq_beats_rtn_on_correlated_inputs():
    X = _correlated_inputs(3)
    W = _random_groups(np.random.default_rng(3), 32, 256)
    for bits, asym in ((4, True), (3, False)):
        lg = O.reconstruction_loss(X, W, O.gptq(X, W, bits, 128, asym))
        lr = O.reconstruction_loss(X, W, O.quantize(W, bits, 128, asym))
        assert lg < 0.5 * lr


def test_gptq_dead_channel_is_zeroed():
    X = _correlated_inputs(4)
    X[:, 7] = 0.0
    W = _random_groups(np.random.default_rng(4), 8, 256)
    U, dead = O.gptq_upper_factor(X)
    assert dead[7] and dead.sum() == 1
    for asym in (True, False):
        assert np.all(O.dequantize(O.gptq(X, W, 4, 128, asym))[:, 7] == 0)


def test_codes_with_params_matches_quantize():
    rng = np.random.default_rng(5)
    W = _random_groups(rng, 16, 128)
    for bits, asym in ((4, True), (3, False), (4, False)):
        q = O.quantize(W, bits, 128, asym)
        for k in (0, 5, 127):
            u = O.codes_with_params(W[:, k].astype(np.float32), q.scales[:, 0], None if q.zeros is None else q.zeros[:, 0],
                                    bits, asym)
            assert np.array_equal(u, q.codes[:, k])


# ---------------------------------------------------------------------------
# GPTQ worked in exact rational arithmetic on a tiny layer ("CMU 11-868
# L19-L20", section "The algorithm in four steps").  The factor is never
# formed: with A = (2 X^T X + lambda I)^-1 = Lt D Lt^T (Lt unit lower
# triangular, D diagonal), the Cholesky factor is L = Lt D^(1/2), so the
# update ratio U[k, j] / U[k, k] of the column step is exactly Lt[j, k], a
# rational number.  Every rounding decision is replayed by exact rounding to
# binary32 / binary16.  The case is chosen so that taking a group's
# parameters from the original weights instead of the updated ones changes
# the scales and the codes.
# ---------------------------------------------------------------------------

def _round_binary(v: Fraction, sig_bits: int, emin: int) -> Fraction:
    """v rounded to the nearest binary float with sig_bits significant bits
    (half to even), subnormals below 2^emin."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, emin) - (sig_bits - 1))
    r = round(a / ulp) * ulp
    return r if v > 0 else -r


def _fl32(v):
    return _round_binary(v, 24, -126)


def _f16r(v):
    return _round_binary(v, 11, -14)


def _rtn_params_exact(vals, bits, asym):
    vals = [_fl32(v) for v in vals]
    if asym:
        qu = 2 ** bits - 1
        r = _fl32(max(vals) - min(vals))
        S = _f16r(_fl32((r if r != 0 else Fraction(1)) / qu))
        Z = min(max(round(_fl32(-min(vals) / S)), 0), qu) if S != 0 else 0
        return S, Fraction(Z)
    h = 2 ** (bits - 1)
    return _f16r(_fl32(max(abs(v) for v in vals) / (h - 1))), Fraction(h)


def _code_exact(v, S, Z, bits, asym):
    q = round(_fl32(_fl32(v) / S))
    if asym:
        return min(max(q + int(Z), 0), 2 ** bits - 1)
    h = 2 ** (bits - 1)
    return min(max(q, -h), h - 1) + h


def _inverse_exact(A):
    n = len(A)
    M = [list(r) + [Fraction(int(i == j)) for j in range(n)] for i, r in enumerate(A)]
    for c in range(n):
        p = next(r for r in range(c, n) if M[r][c] != 0)
        M[c], M[p] = M[p], M[c]
        M[c] = [v / M[c][c] for v in M[c]]
        for r in range(n):
            if r != c and M[r][c] != 0:
                f = M[r][c]
                M[r] = [a - f * b for a, b in zip(M[r], M[c])]
    return [r[n:] for r in M]


def _unit_lower_of_ldl(A):
    n = len(A)
    L = [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]
    D = [Fraction(0)] * n
    for j in range(n):
        D[j] = A[j][j] - sum(L[j][k] ** 2 * D[k] for k in range(j))
        for i in range(j + 1, n):
            L[i][j] = (A[i][j] - sum(L[i][k] * L[j][k] * D[k] for k in range(j))) / D[j]
    return L


def _gptq_exact(X, W, bits, G, asym, params_from_original=False):
    T, K, N = len(X), len(X[0]), len(W)
    H = [[2 * sum(X[t][i] * X[t][j] for t in range(T)) for j in range(K)] for i in range(K)]
    lam = Fraction(1, 100) * sum(H[i][i] for i in range(K)) / K
    for i in range(K):
        H[i][i] += lam
    Lt = _unit_lower_of_ldl(_inverse_exact(H))
    w = [list(r) for r in W]
    codes = [[0] * K for _ in range(N)]
    S = [[None] * (K // G) for _ in range(N)]
    Z = [[None] * (K // G) for _ in range(N)]
    for k in range(K):
        g = k // G
        for n in range(N):
            if k % G == 0:
                src = W[n] if params_from_original else w[n]
                S[n][g], Z[n][g] = _rtn_params_exact(src[k:k + G], bits, asym)
            u = _code_exact(w[n][k], S[n][g], Z[n][g], bits, asym)
            codes[n][k] = u
            e = w[n][k] - (u - Z[n][g]) * S[n][g]
            for j in range(k + 1, K):
                w[n][j] -= e * Lt[j][k]
    return codes, S, Z


_GPTQ_TINY_X = [[-1.0, 1.5, 1.0, -2.0], [-0.5, 1.5, 0.0, -2.0], [1.0, 1.0, 1.5, -1.5]]
_GPTQ_TINY_W = [[-0.875, 0.75, -1.0, 0.0625], [-0.875, -0.4375, -0.0625, -0.1875]]
# (bits, asym) -> codes, scales, zeros that the exact computation gives
_GPTQ_TINY_EXPECT = {
    (4, True): ([[0, 15, 0, 15], [0, 15, 0, 13]],
                [[0.10833740234375, 0.07135009765625], [0.0291595458984375, 0.019989013671875]],
                [[8, 14], [15, 15]]),
    (3, False): ([[1, 7, 1, 4], [1, 2, 3, 1]],
                 [[0.291748046875, 0.330810546875], [0.291748046875, 0.09912109375]],
                 None),
}


@pytest.mark.parametrize("bits,asym", [(4, True), (3, False)])
def test_gptq_tiny_layer_against_exact_rationals(bits, asym):
    X = np.array(_GPTQ_TINY_X, np.float16)
    W = np.array(_GPTQ_TINY_W, np.float16)
    Xq = [[Fraction(float(v)) for v in r] for r in X]
    Wq = [[Fraction(float(v)) for v in r] for r in W]
    codes, S, Z = _gptq_exact(Xq, Wq, bits, 2, asym)
    e_codes, e_S, e_Z = _GPTQ_TINY_EXPECT[(bits, asym)]
    assert codes == e_codes
    assert [[float(s) for s in r] for r in S] == e_S
    if asym:
        assert [[int(z) for z in r] for r in Z] == e_Z
    # the case separates the readings: parameters from the original weights
    # give other scales and other codes
    codes_o, S_o, _ = _gptq_exact(Xq, Wq, bits, 2, asym, params_from_original=True)
    assert S_o != S and codes_o != codes
    q = O.gptq(X.astype(np.float64), W, bits, 2, asym)
    assert q.codes.tolist() == e_codes
    assert q.scales.astype(np.float64).tolist() == e_S
    if asym:
        assert q.zeros.astype(np.float64).tolist() == [[float(z) for z in r] for r in e_Z]
    else:
        assert q.zeros is None


# ---------------------------------------------------------------------------
# The parity checker, the layer objective, activation decoding and the AWQ
# scale floor, each against closed forms or exact arithmetic.
# ---------------------------------------------------------------------------

def test_rel_l2_closed_forms():
    ref = np.array([3.0, 4.0])                         # ||ref|| = 5
    assert O.rel_l2(ref, ref) == 0.0
    assert O.rel_l2(np.array([4.0, 4.0]), ref) == 0.2   # ||(1, 0)|| / 5
    assert abs(O.rel_l2(ref * 1.1, ref) - 0.1) < 1e-15
    assert abs(O.rel_l2(np.array([[3.0, 4.0], [5.0, 12.0]]), np.array([[0.0, 0.0], [5.0, 12.0]])) - 5.0 / 13.0) < 1e-15
    assert O.rel_l2(np.array([0.0, 2.0]), np.zeros(2)) == 2.0   # zero reference: the plain norm


def test_reconstruction_loss_against_fractions():
    rng = np.random.default_rng(12)
    T, N, K = 3, 2, 64
    X = rng.standard_normal((T, K)).astype(np.float16).astype(np.float64)
    W = _random_groups(rng, N, K)
    q = O.quantize(W, 3, 32, True)
    total = Fraction(0)
    for t in range(T):
        for n in range(N):
            d = Fraction(0)
            for k in range(K):
                g = k // 32
                w_hat = (Fraction(int(q.codes[n, k])) - Fraction(float(q.zeros[n, g]))) * Fraction(float(q.scales[n, g]))
                d += Fraction(float(X[t, k])) * (Fraction(float(W[n, k])) - w_hat)
            total += d * d
    got = O.reconstruction_loss(X, W, q)
    assert abs(got - float(total)) <= 1e-12 * float(total)


def test_activations_f64_decodes_bf16_bits_and_fp16_values():
    bits = np.array([[0x3F80, 0xC000, 0x4049, 0x0000], [0x8000, 0x7F7F, 0x0001, 0xBF00]], np.uint16)
    vals = O.activations_f64(bits, "bf16")
    assert vals.dtype == np.float64 and vals.shape == (2, 4)
    assert vals.tolist() == [[1.0, -2.0, 3.140625, 0.0], [0.0, 255 * 2.0 ** 120, 2.0 ** -133, -0.5]]
    h = np.array([[1.0, -2.5, 65504.0, 2.0 ** -24]], np.float16)
    assert O.activations_f64(h, "f16").tolist() == [[1.0, -2.5, 65504.0, 2.0 ** -24]]


def test_awq_scale_floor_for_quiet_channels():
    # channels whose mean |x| is below the floor 1e-4 are scaled as if it were
    # 1e-4 (alpha = 1 returns the floored means themselves, rounded to fp32)
    m = np.array([0.0, 5e-5, 1e-4, 2e-4, 1.0])
    assert np.array_equal(O.awq_scale_for(m, 1.0), np.array([1e-4, 1e-4, 1e-4, 2e-4, 1.0], np.float32))
    s = O.awq_scale_for(m, 0.5)
    assert np.all(np.abs(s[:3].astype(np.float64) - 1e-2) <= 1e-2 * 2.0 ** -23)
    # a channel that never fires still gets a finite, positive scale in the search
    X = np.ones((4, 128))
    X[:, 3] = 0.0
    W = np.full((2, 128), 0.01, np.float16)
    _, _, best_s = O.awq_search(X, W, 4, 128, True, 4)
    assert np.all(np.isfinite(best_s)) and np.all(best_s > 0)
