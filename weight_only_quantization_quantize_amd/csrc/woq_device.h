// Device-side helpers shared by the gfx950 kernels: packed-code decode into
// 16-bit float pairs, activation type traits, and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace woq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Activation types.  A packed code u is turned into a 16-bit float of value
// MAGIC + u by OR-ing it into the low mantissa bits of MAGIC's bit pattern:
//   fp16 0x6400 = 1024 (10 mantissa bits, spacing 1 on [1024, 2048))
//   bf16 0x4300 =  128 ( 7 mantissa bits, spacing 1 on [128, 256))
// Both hold every code 0..15 exactly.  The kernels multiply x by (MAGIC + u)
// and remove MAGIC + Z with the per-chunk activation sum:
//   sum x (u - Z) = sum x (MAGIC + u) - (MAGIC + Z) sum x.
// ---------------------------------------------------------------------------
struct F16 {
  static constexpr uint32_t kMagic2 = 0x64006400u;
  static constexpr float kMagic = 1024.0f;
  __device__ static inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
  }
  __device__ static inline float to_f32(uint16_t v) {
    return (float)__builtin_bit_cast(_Float16, v);
  }
  __device__ static inline uint16_t from_f32(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  }
  __device__ static inline float4_t mfma16x16x32(u32x4_t a, u32x4_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b),
                                                  c, 0, 0, 0);
  }
};

struct BF16 {
  static constexpr uint32_t kMagic2 = 0x43004300u;
  static constexpr float kMagic = 128.0f;
  __device__ static inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a), __builtin_bit_cast(bf162_t, b), c,
                                           false);
  }
  __device__ static inline float to_f32(uint16_t v) {
    return __builtin_bit_cast(float, (uint32_t)v << 16);
  }
  __device__ static inline uint16_t from_f32(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
  }
  __device__ static inline float4_t mfma16x16x32(u32x4_t a, u32x4_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, a),
                                                   __builtin_bit_cast(bf168_t, b), c, 0, 0, 0);
  }
};

// Word 3 of a raw (stride 0) buffer resource on gfx9-family GPUs, gfx950
// included: 32-bit data format, no swizzle.  Loads past the resource's byte
// count return zero.
constexpr int kBufferWord3 = 0x00020000;

// ---------------------------------------------------------------------------
// Packed-code decode.  Each helper returns the code pair (k, k+1) of pair index
// t in the two 16-bit halves, OR-ed with the magic pattern.
// ---------------------------------------------------------------------------

// 4-bit word holding k in [8j, 8j+8): pair t (k = 8j+2t, 8j+2t+1) at bits
// [4t, 4t+4) and [16+4t, 16+4t+4).
// A constant the compiler cannot fold: keeps MAGIC in a VGPR so that
// (w & mask) | MAGIC becomes one v_and_or_b32 with the mask in an SGPR.
__device__ inline uint32_t vgpr_const(uint32_t v) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

__device__ inline uint32_t pair4(uint32_t w, int t, uint32_t magic2) {
  return ((w >> (4 * t)) & 0x000F000Fu) | magic2;
}

// 3-bit unit (w0, w1, w2) holding 32 k, layout v2: pair t < 15 is the 3-bit
// field at bits [3 (t % 5), +3) and [16 + 3 (t % 5), +3) of word w_(t / 5);
// pair 15 keeps bit b of each half's code at bit 15 / 31 of word w_b.
__device__ inline uint32_t pair3(uint32_t w0, uint32_t w1, uint32_t w2, int t, uint32_t magic2) {
  if (t < 15) {
    const uint32_t w = t < 5 ? w0 : (t < 10 ? w1 : w2);
    return ((w >> (3 * (t % 5))) & 0x00070007u) | magic2;
  }
  return ((w0 >> 15) & 0x00010001u) | ((w1 >> 14) & 0x00020002u) | ((w2 >> 13) & 0x00040004u) | magic2;
}

// Sum over a team of `team` consecutive lanes (team a power of two <= 64);
// every lane of the team ends with the total.
__device__ inline float team_sum(float v, int team) {
  for (int off = team >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ inline float team_max(float v, int team) {
  for (int off = team >> 1; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ inline float team_min(float v, int team) {
  for (int off = team >> 1; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ inline float half_bits_to_f32(uint16_t v) { return (float)__builtin_bit_cast(_Float16, v); }

// 1 / s for an activation scale: the hardware reciprocal v_rcp_f32, within
// 1 ulp of the quotient.  Activations x * (1 / s) are rounded to a 16-bit
// float (relative error 2^-11 or 2^-8) before use, so the reciprocal's 2^-23
// does not show; an IEEE division costs about ten VALU instead of one.
__device__ inline float act_recip(float s) { return __builtin_amdgcn_rcpf(s); }

}  // namespace woq
