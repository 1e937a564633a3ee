// Group-wise RTN quantization of fp16 weights into layout-v2 codes plus fp16
// scales / zero points, bit-exact with the reference definition:
//
//   w = fl32(W * s)                       (optional AWQ fold, one multiply)
//   symmetric : S = f16(max|w| / (2^(b-1)-1)), u = clip(rne(w/S), -2^(b-1), 2^(b-1)-1) + 2^(b-1)
//   asymmetric: r = max-min (1 if 0), S = f16(r / (2^b-1)),
//               Z = clip(rne(-min/S), 0, 2^b-1), u = clip(rne(w/S) + Z, 0, 2^b-1)
//
// ("Quantising Large Language Models for Efficient Inference", section
// "Post-training methods for 4-bit weights"; "CMU 11-868 L19-L20 Model
// Quantization", section "absmax and zero-point"; "LLM Quantization: 160GB
// Model on a Laptop", sections "Symmetric Quantization" and "Asymmetric
// Quantization".)
//
// Every decision is one correctly rounded binary32 operation: the quotient
// of IEEE division (the group's S / qmax and -min / S divide; a weight's w / S
// comes from the group's reciprocal with two exact fma corrections, equal to
// the IEEE quotient, or with one when w is an unfolded fp16 weight, which
// rounds to the same integer; rtn_rules.h), rintf = round half to even,
// fp32 -> fp16 conversion round-to-nearest-even with subnormals, and no FMA
// contraction in this file.
//
// Work split: one thread owns one 32-weight chunk of a row (64 B of fp16 in,
// 16 B (4-bit) or 12 B (3-bit) of codes out).  For group sizes whose chunk
// count divides the 64-lane wave, the chunk threads of a group reduce the
// group statistic with lane shuffles; other group sizes use one workgroup per
// group with an LDS reduction.  The pass moves 2 B in and b/8 B out per
// weight and issues about 16 VALU per weight, so it sits near both the HBM
// and the VALU limit.
#include "rtn_rules.h"
#include "woq_device.h"
#include "woq_internal.h"

#pragma clang fp contract(off)

namespace woq {
namespace {

constexpr int kThreads = 256;

template <bool FOLD>
__device__ inline void load_chunk(const uint16_t* __restrict__ W, const float* __restrict__ s, int64_t row_off,
                                  int k0, float (&w)[32]) {
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(W + row_off + k0);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4_t v = src[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[8 * q + 2 * e] = half_bits_to_f32((uint16_t)(v[e] & 0xFFFFu));
      w[8 * q + 2 * e + 1] = half_bits_to_f32((uint16_t)(v[e] >> 16));
    }
  }
  if (FOLD) {
    const float4_t* sp = reinterpret_cast<const float4_t*>(s + k0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4_t sv = sp[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[4 * q + e] = w[4 * q + e] * sv[e];
    }
  }
}

// Chunk c of a matrix, in a group of `team` consecutive chunk threads
// (team = G/32 divides 64).
template <int BITS, bool ASYM, bool FOLD>
__device__ __attribute__((always_inline)) inline void team_chunk(const uint16_t* __restrict__ W,
                                                                 const float* __restrict__ s, int64_t c,
                                                                 int64_t total_chunks, int K, int G, int team,
                                                                 uint8_t* __restrict__ packed,
                                                                 uint16_t* __restrict__ scales,
                                                                 uint16_t* __restrict__ zeros) {
  const bool valid = c < total_chunks;
  const int cpr = K >> 5;
  // Row and chunk within the row: a 32-bit division whenever the matrix has
  // fewer than 2^32 chunks (the 64-bit one cost about 60 VALU and as many
  // scalar instructions per thread, two per weight).
  int64_t n = 0;
  int kc = 0;
  if (valid) {
    if (total_chunks <= 0xFFFFFFFFll) {
      const uint32_t c32 = (uint32_t)c, n32 = c32 / (uint32_t)cpr;
      n = n32;
      kc = (int)(c32 - n32 * (uint32_t)cpr);
    } else {
      n = c / cpr;
      kc = (int)(c - n * cpr);
    }
  }
  float w[32];
  if (valid) {
    load_chunk<FOLD>(W, s, n * (int64_t)K, kc * 32, w);
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i] = 0.0f;
  }
  float lo = 0.0f, hi = 0.0f;
  if (!ASYM) {
#pragma unroll
    for (int i = 0; i < 32; ++i) hi = fmaxf(hi, fabsf(w[i]));
    hi = team_max(hi, team);
  } else {
    lo = w[0];
    hi = w[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) {
      lo = fminf(lo, w[i]);
      hi = fmaxf(hi, w[i]);
    }
    lo = team_min(lo, team);
    hi = team_max(hi, team);
  }
  if (!valid) return;
  const GroupParams<BITS, ASYM> p = group_params<BITS, ASYM>(lo, hi);
  uint32_t u[32];
  codes_of_chunk<BITS, ASYM, !FOLD>(w, p, u);
  store_chunk<BITS>(packed, n, K, kc, u);
  if ((kc & (team - 1)) == 0) {
    const int64_t gi = n * (int64_t)(K / G) + (kc * 32) / G;
    scales[gi] = p.S16;
    if (ASYM) zeros[gi] = f32_to_half_bits((float)p.Z);
  }
}

template <int BITS, bool ASYM, bool FOLD>
__global__ __launch_bounds__(kThreads) void quantize_pack_team_kernel(
    const uint16_t* __restrict__ W, const float* __restrict__ s, int64_t total_chunks, int K, int G, int team,
    uint8_t* __restrict__ packed, uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros) {
  team_chunk<BITS, ASYM, FOLD>(W, s, (int64_t)blockIdx.x * kThreads + threadIdx.x, total_chunks, K, G, team,
                               packed, scales, zeros);
}

// Several matrices in one launch: workgroups [block0[i], block0[i + 1]) run
// matrix i's chunks exactly as quantize_pack_team_kernel would, so matrix
// i + 1 starts streaming while matrix i's last workgroups finish instead of
// behind a launch boundary.  The descriptors travel in the kernel arguments
// (indexed in place, no copy).
struct QpManyArgs {
  const uint16_t* W[kQpManyMax];
  const float* s[kQpManyMax];
  uint8_t* packed[kQpManyMax];
  uint16_t* scales[kQpManyMax];
  uint16_t* zeros[kQpManyMax];
  int64_t chunks[kQpManyMax];
  int K[kQpManyMax];
  unsigned block0[kQpManyMax + 1];
  int count;
};

template <int BITS, bool ASYM>
__global__ __launch_bounds__(kThreads) void quantize_pack_many_kernel(const QpManyArgs a, int G, int team) {
  const unsigned b = blockIdx.x;
  int i = 0;  // the last matrix whose first workgroup is at or before b (wave-uniform)
  for (int j = 1; j < a.count; ++j) i = a.block0[j] <= b ? j : i;
  const int64_t c = (int64_t)(b - a.block0[i]) * kThreads + threadIdx.x;
  if (a.s[i])
    team_chunk<BITS, ASYM, true>(a.W[i], a.s[i], c, a.chunks[i], a.K[i], G, team, a.packed[i], a.scales[i],
                                 a.zeros[i]);
  else
    team_chunk<BITS, ASYM, false>(a.W[i], nullptr, c, a.chunks[i], a.K[i], G, team, a.packed[i], a.scales[i],
                                  a.zeros[i]);
}

template <int BITS, bool ASYM>
hipError_t launch_many_typed(const QpMatrix* mats, int count, int G, hipStream_t stream) {
  const int team = G / 32;
  for (int first = 0; first < count; first += kQpManyMax) {
    QpManyArgs a{};
    a.count = count - first < kQpManyMax ? count - first : kQpManyMax;
    int64_t blocks = 0;
    for (int i = 0; i < a.count; ++i) {
      const QpMatrix& m = mats[first + i];
      a.W[i] = static_cast<const uint16_t*>(m.W);
      a.s[i] = m.s;
      a.packed[i] = static_cast<uint8_t*>(m.packed);
      a.scales[i] = static_cast<uint16_t*>(m.scales);
      a.zeros[i] = static_cast<uint16_t*>(m.zeros);
      a.chunks[i] = m.N * (m.K / 32);
      a.K[i] = (int)m.K;
      a.block0[i] = (unsigned)blocks;
      blocks += (a.chunks[i] + kThreads - 1) / kThreads;
      if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    }
    a.block0[a.count] = (unsigned)blocks;
    hipLaunchKernelGGL((quantize_pack_many_kernel<BITS, ASYM>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a,
                       G, team);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// One workgroup per group (any G that is a multiple of 32).
template <int BITS, bool ASYM, bool FOLD>
__global__ __launch_bounds__(kThreads) void quantize_pack_block_kernel(
    const uint16_t* __restrict__ W, const float* __restrict__ s, int K, int G, uint8_t* __restrict__ packed,
    uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros) {
  __shared__ float red_lo[kThreads / 64], red_hi[kThreads / 64];
  const int groups_per_row = K / G;
  const int64_t gid = blockIdx.x;
  const int64_t n = gid / groups_per_row;
  const int g = (int)(gid - n * groups_per_row);
  const int chunks = G >> 5;
  const int c0 = g * chunks;  // first chunk of the group within the row
  float lo = 0.0f, hi = 0.0f;
  bool first = true;
  for (int c = threadIdx.x; c < chunks; c += kThreads) {
    float w[32];
    load_chunk<FOLD>(W, s, n * (int64_t)K, (c0 + c) * 32, w);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (!ASYM) {
        hi = fmaxf(hi, fabsf(w[i]));
      } else if (first && i == 0) {
        lo = w[0];
        hi = w[0];
      } else {
        lo = fminf(lo, w[i]);
        hi = fmaxf(hi, w[i]);
      }
    }
    first = false;
  }
  // Threads that own no chunk must not disturb the asymmetric min / max.
  if (ASYM && first) {
    lo = __builtin_huge_valf();
    hi = -__builtin_huge_valf();
  }
  lo = team_min(lo, 64);
  hi = team_max(hi, 64);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red_lo[wave] = lo;
    red_hi[wave] = hi;
  }
  __syncthreads();
  lo = red_lo[0];
  hi = red_hi[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) {
    lo = fminf(lo, red_lo[i]);
    hi = fmaxf(hi, red_hi[i]);
  }
  const GroupParams<BITS, ASYM> p = group_params<BITS, ASYM>(lo, hi);
  for (int c = threadIdx.x; c < chunks; c += kThreads) {
    float w[32];
    load_chunk<FOLD>(W, s, n * (int64_t)K, (c0 + c) * 32, w);
    uint32_t u[32];
    codes_of_chunk<BITS, ASYM, !FOLD>(w, p, u);
    store_chunk<BITS>(packed, n, K, c0 + c, u);
  }
  if (threadIdx.x == 0) {
    scales[gid] = p.S16;
    if (ASYM) zeros[gid] = f32_to_half_bits((float)p.Z);
  }
}

template <int BITS, bool ASYM, bool FOLD>
hipError_t launch_typed(const void* W, const float* s, int64_t N, int64_t K, int G, void* packed, void* scales,
                        void* zeros, hipStream_t stream) {
  const int team = G / 32;
  if (team <= 64 && (64 % team) == 0) {
    const int64_t total = N * (K / 32);
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    hipLaunchKernelGGL((quantize_pack_team_kernel<BITS, ASYM, FOLD>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, static_cast<const uint16_t*>(W), s, total, (int)K, G, team,
                       static_cast<uint8_t*>(packed), static_cast<uint16_t*>(scales),
                       static_cast<uint16_t*>(zeros));
  } else {
    const int64_t groups = N * (K / G);
    hipLaunchKernelGGL((quantize_pack_block_kernel<BITS, ASYM, FOLD>), dim3((unsigned)groups), dim3(kThreads), 0,
                       stream, static_cast<const uint16_t*>(W), s, (int)K, G, static_cast<uint8_t*>(packed),
                       static_cast<uint16_t*>(scales), static_cast<uint16_t*>(zeros));
  }
  return hipGetLastError();
}

template <int BITS, bool ASYM>
hipError_t launch_fold(const void* W, const float* s, int64_t N, int64_t K, int G, void* packed, void* scales,
                       void* zeros, hipStream_t stream) {
  return s ? launch_typed<BITS, ASYM, true>(W, s, N, K, G, packed, scales, zeros, stream)
           : launch_typed<BITS, ASYM, false>(W, s, N, K, G, packed, scales, zeros, stream);
}

}  // namespace

bool quantize_pack_many_batched(int group_size) {
  const int team = group_size / 32;
  return team <= 64 && 64 % team == 0;
}

hipError_t launch_quantize_pack_many(const QpMatrix* mats, int count, int bits, int group_size, bool asymmetric,
                                     hipStream_t stream) {
  if (!quantize_pack_many_batched(group_size)) {
    // group sizes of the one-workgroup-per-group kernel: one launch each
    for (int i = 0; i < count; ++i) {
      const QpMatrix& m = mats[i];
      const hipError_t e =
          launch_quantize_pack(m.W, m.s, m.N, m.K, bits, group_size, asymmetric, m.packed, m.scales, m.zeros, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (bits == 4)
    return asymmetric ? launch_many_typed<4, true>(mats, count, group_size, stream)
                      : launch_many_typed<4, false>(mats, count, group_size, stream);
  return asymmetric ? launch_many_typed<3, true>(mats, count, group_size, stream)
                    : launch_many_typed<3, false>(mats, count, group_size, stream);
}

hipError_t launch_quantize_pack(const void* W, const float* act_scale, int64_t N, int64_t K, int bits,
                                int group_size, bool asymmetric, void* packed, void* scales, void* zeros,
                                hipStream_t stream) {
  if (bits == 4) {
    return asymmetric ? launch_fold<4, true>(W, act_scale, N, K, group_size, packed, scales, zeros, stream)
                      : launch_fold<4, false>(W, act_scale, N, K, group_size, packed, scales, zeros, stream);
  }
  return asymmetric ? launch_fold<3, true>(W, act_scale, N, K, group_size, packed, scales, zeros, stream)
                    : launch_fold<3, false>(W, act_scale, N, K, group_size, packed, scales, zeros, stream);
}

}  // namespace woq
