// Round-to-nearest rules shared by every kernel that decides codes: the
// group scale / zero point and the code of one weight, each decision one
// correctly rounded binary32 operation (IEEE division or its exact
// equivalent, rintf = round half to even, fp32 -> fp16 round-to-nearest-even
// with subnormals), and the layout-v2 store of a 32-code chunk.
//
//   symmetric : S = f16(max|w| / (2^(b-1)-1)), u = clip(rne(w/S), -2^(b-1), 2^(b-1)-1) + 2^(b-1)
//   asymmetric: r = max-min (1 if 0), S = f16(r / (2^b-1)),
//               Z = clip(rne(-min/S), 0, 2^b-1), u = clip(rne(w/S) + Z, 0, 2^b-1)
//
// ("Quantising Large Language Models for Efficient Inference", section
// "Post-training methods for 4-bit weights"; "CMU 11-868 L19-L20 Model
// Quantization", section "absmax and zero-point"; "LLM Quantization: 160GB
// Model on a Laptop", sections "Symmetric Quantization" and "Asymmetric
// Quantization".)  None of these has a multiply-add for the compiler to
// contract.
#pragma once

#include "woq_device.h"

namespace woq {

__device__ inline uint16_t f32_to_half_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// Scale (and zero point) of one group from its statistic.  For the
// symmetric form `lo` is unused and `hi` is max|w|.
template <int BITS, bool ASYM>
struct GroupParams {
  float S;        // the stored fp16 scale, widened exactly
  float R;        // fl32(1 / S), IEEE division (0 when S == 0)
  int Z;          // zero point (symmetric: 2^(b-1))
  uint16_t S16;   // fp16 bits of S
  bool zero;      // S == 0: every code is Z
};

// fl32(w / S) from R = fl32(1 / S) without a division: q0 = w R is within
// about one ulp of w / S, each residual w - q S is exact in an fma, and two
// correction steps give the correctly rounded quotient (Markstein's
// division with a correctly rounded reciprocal).  Checked on the GPU against
// IEEE division for every finite fp16 w and positive fp16 S, and for 2^34
// random fp32 w: equal everywhere except the sign of a zero quotient, which
// the rounding to an integer code ignores.
__device__ inline float div_by_scale(float w, float S, float R) {
  const float q0 = w * R;
  const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, S, w), R, q0);
  return __builtin_fmaf(__builtin_fmaf(-q1, S, w), R, q1);
}

// The same code with one correction step, for fp16 w (no AWQ fold) and
// fp16 S.  Only |w / S| < 16 can give a code that is not clipped, and there
// w / S is either
//  * exactly a half-integer h: q0 = h (1 + e) with |e| <= 2^-23, the residual
//    w - q0 S = -h e S is exact, and q0 + R (-h e S) = h up to h 2^-46, so
//    the corrected quotient is h itself, as the IEEE quotient is; or
//  * at least 2^-12 away from every half-integer: 2 w - (2k + 1) S is a
//    nonzero integer multiple of 2^min(e_w + 1, e_S), e_w and e_S being the
//    weights of the last significand bits of w and S, and S < 2^(e_S + 11);
//    the corrected quotient is within an ulp (2^-19 below 16) of w / S, so it
//    rounds to the same integer as the IEEE quotient.
// tests/test_quantize_rounding.py checks the gap on every fp16 w against
// fp16 scales of every binade.
__device__ inline float div_by_scale_f16(float w, float S, float R) {
  const float q0 = w * R;
  return __builtin_fmaf(__builtin_fmaf(-q0, S, w), R, q0);
}

template <int BITS, bool ASYM>
__device__ inline void set_reciprocal(GroupParams<BITS, ASYM>& p) {
  p.R = p.zero ? 0.0f : 1.0f / p.S;
}

template <int BITS, bool ASYM>
__device__ inline GroupParams<BITS, ASYM> group_params(float lo, float hi) {
  GroupParams<BITS, ASYM> p;
  if (!ASYM) {
    const float qmax = (float)((1 << (BITS - 1)) - 1);
    p.S16 = f32_to_half_bits(hi / qmax);
    p.S = half_bits_to_f32(p.S16);
    p.Z = 1 << (BITS - 1);
    p.zero = (p.S == 0.0f);
  } else {
    const float qu = (float)((1 << BITS) - 1);
    float r = hi - lo;
    if (r == 0.0f) r = 1.0f;
    p.S16 = f32_to_half_bits(r / qu);
    p.S = half_bits_to_f32(p.S16);
    p.zero = (p.S == 0.0f);
    if (p.zero) {
      p.Z = 0;
    } else {
      int z = (int)__builtin_rintf(-lo / p.S);
      p.Z = z < 0 ? 0 : (z > (1 << BITS) - 1 ? (1 << BITS) - 1 : z);
    }
  }
  set_reciprocal(p);
  return p;
}

// Code of one weight: u = clip(rne(w / S) + Z, 0, 2^b - 1) (symmetric:
// Z = 2^(b-1), the same as clipping rne(w / S) to [-2^(b-1), 2^(b-1) - 1]
// and adding 2^(b-1)).  S == 0 needs no branch: R = 0 makes the quotient 0
// for finite w, so u = clip(Z) = Z, the definition's code for that group.
// (A branch per weight compiled to an exec-mask change around each of a
// chunk's 32 codes.)  The float -> int conversion saturates, so quotients
// of any size clip as the definition says.
// F16W: w is an fp16 value (no fold), so one correction step decides the
// same code (div_by_scale_f16).
template <int BITS, bool ASYM, bool F16W = false>
__device__ inline uint32_t code_of(float w, const GroupParams<BITS, ASYM>& p) {
  const float q = F16W ? div_by_scale_f16(w, p.S, p.R) : div_by_scale(w, p.S, p.R);
  const int v = (int)__builtin_rintf(q) + p.Z;
  const int top = (1 << BITS) - 1;
  return (uint32_t)(v < 0 ? 0 : (v > top ? top : v));
}

template <int BITS, bool ASYM, bool F16W = false>
__device__ inline void codes_of_chunk(const float (&w)[32], const GroupParams<BITS, ASYM>& p, uint32_t (&u)[32]) {
#pragma unroll
  for (int i = 0; i < 32; ++i) u[i] = code_of<BITS, ASYM, F16W>(w[i], p);
}

template <int BITS>
__device__ inline void store_chunk(uint8_t* __restrict__ packed, int64_t n, int K, int kc, const uint32_t (&u)[32]) {
  if (BITS == 4) {
    u32x4_t out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t word = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) word |= u[8 * j + 2 * t + h] << (16 * h + 4 * t);
      out[j] = word;
    }
    *reinterpret_cast<u32x4_t*>(packed + n * (int64_t)(K / 2) + (int64_t)kc * 16) = out;
  } else {
    // layout v2: pair t < 15 whole at bits 16 h + 3 (t % 5) of word t / 5;
    // pair 15's bit b at bit 16 h + 15 of word b
    uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int t = i >> 1, h = i & 1;
      if (t < 15) {
        w[t / 5] |= (u[i] & 7u) << (16 * h + 3 * (t % 5));
      } else {
#pragma unroll
        for (int b = 0; b < 3; ++b) w[b] |= ((u[i] >> b) & 1u) << (16 * h + 15);
      }
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(packed + n * (int64_t)(3 * K / 8) + (int64_t)kc * 12);
    dst[0] = w[0];
    dst[1] = w[1];
    dst[2] = w[2];
  }
}


}  // namespace woq
