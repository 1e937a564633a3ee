"""The premise behind the quantize kernel's one-step quotient for fp16 weights.

Without an AWQ fold both w and S are fp16 values, and the kernel rounds
w * fl32(1/S) after a single Markstein correction instead of the IEEE
quotient (rtn_rules.h, div_by_scale_f16).  That decides the same code because
w / S is either exactly a half-integer or at least 2^-12 from every
half-integer wherever a code is not clipped (|w / S| < 16).  This checks that
gap over every finite fp16 w against fp16 scales from every binade (normal
and subnormal), in exact arithmetic: fp16 values are dyadic rationals, so
2w - (2k+1)S is computed exactly in float64 scaled by 2^25.
"""
import numpy as np
import pytest


def _all_finite_f16():
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    return v[np.isfinite(v)].astype(np.float64)


def _scales():
    # every binade: a spread of significands in each, plus all subnormals
    rng = np.random.default_rng(12)
    pos = np.arange(1, 0x7C00, dtype=np.uint16)  # positive finite fp16 bit patterns
    sub = pos[pos < 0x0400]
    normal = pos[pos >= 0x0400]
    picks = [sub]
    for e in range(1, 31):
        binade = normal[(normal >> 10) == e]
        picks.append(binade[[0, 1, 2, len(binade) - 1]])
        picks.append(rng.choice(binade, 28, replace=False))
    return np.concatenate(picks).view(np.float16).astype(np.float64)


@pytest.mark.parametrize("part", range(4))
def test_fp16_quotients_are_ties_or_far_from_them(part):
    w = _all_finite_f16()
    S = _scales()[part::4]
    two25 = 2.0 ** 25
    W2 = np.round(w * two25 * 2)          # 2w in units of 2^-25: exact integers below 2^53
    worst = np.inf
    for s in S:
        q = w / s
        keep = np.abs(q) < 16
        qk = q[keep]
        k = np.floor(qk)                   # nearest half-integer candidate: k + 1/2
        num = W2[keep] - (2 * k + 1) * np.round(s * two25)   # 2^25 (2w - (2k+1) S), exact
        tie = num == 0
        gap = np.abs(num[~tie]) / (2 * s * two25)             # |w/S - (k + 1/2)|
        if gap.size:
            worst = min(worst, float(gap.min()))
        # a tie is an exactly representable half-integer quotient
        assert np.all(qk[tie] == k[tie] + 0.5)
    assert worst >= 2.0 ** -12, worst
