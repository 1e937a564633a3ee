// Fused dequantize + GEMV for M = 1 decode: y[n] = sum_k x'[k] (u[n,k] - Z) S.
//
// Decode is memory-bound: a [1, K] x [K, N] GEMV does about one flop per byte
// of weights ("MIT 6.5940 Lab 4 + Lab 5", Lab 4 "Starting point and setup";
// "CMU 11-868 L19-L20", section "Back to the question: where does the speed
// come from?"), so the kernel is built to stream the packed codes from HBM
// exactly once and dequantize them in registers ("Quantising Large Language
// Models ...", section "Weight-only vs weight-and-activation quantisation").
//
// Mapping (one 64-lane wave per output row, or per 64/team rows when a row
// has fewer than 64 chunks of 32 weights):
//  * a team of `team` lanes covers one row; lane p of the team owns chunks
//    c = i*team + p (i < CPL) of every row, i.e. a fixed slice of K;
//  * that slice of x (divided by the AWQ scale when given, rounded once to
//    the activation type) lives in registers for the whole kernel, together
//    with the fp32 sum of each chunk's 32 activations;
//  * per row the team issues CPL lane-contiguous loads (16 B per lane for
//    4-bit, 12 B for 3-bit: a team reads a contiguous stretch of the row) plus
//    the fp16 scale / zero of each chunk's group;
//  * a code pair is turned into the 16-bit float pair (MAGIC + u) by one
//    shift / mask / OR, multiplied into fp32 with v_dot2 against the matching
//    activation pair, and the chunk total is corrected and scaled in fp32:
//      S * (sum x (MAGIC + u) - (MAGIC + Z) * sum x) = S * sum x (u - Z);
//  * the team reduces its partial sums with lane shuffles and one lane writes
//    y[n] rounded to the activation type.
#include "woq_device.h"
#include "woq_internal.h"

namespace woq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <int BITS>
struct ChunkCodes;
template <>
struct ChunkCodes<4> {
  uint32_t w[4];
};
template <>
struct ChunkCodes<3> {
  uint32_t w[3];
};

template <int BITS>
__device__ inline void load_codes(const uint8_t* __restrict__ packed, int64_t n, int K, int c, ChunkCodes<BITS>& cc) {
  if (BITS == 4) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(packed + n * (int64_t)(K / 2) + (int64_t)c * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) cc.w[j] = v[j];
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(packed + n * (int64_t)(3 * K / 8) + (int64_t)c * 12);
#pragma unroll
    for (int j = 0; j < 3; ++j) cc.w[j] = p[j];
  }
}

// sum over the chunk of x (MAGIC + u), accumulated in fp32 by v_dot2.
template <int BITS, class XT>
__device__ inline float chunk_dot(const ChunkCodes<BITS>& cc, const uint32_t (&xr)[16]) {
  float a = 0.0f;
  if (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) a = XT::dot2(pair4(cc.w[j], t, XT::kMagic2), xr[4 * j + t], a);
  } else {
#pragma unroll
    for (int t = 0; t < 16; ++t) a = XT::dot2(pair3(cc.w[0], cc.w[1], cc.w[2], t, XT::kMagic2), xr[t], a);
  }
  return a;
}

template <int BITS, bool ASYM, class XT, int CPL, bool SCALE, int ROWS>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const uint16_t* __restrict__ x, const float* __restrict__ s,
                                                        const uint8_t* __restrict__ packed,
                                                        const uint16_t* __restrict__ scales,
                                                        const uint16_t* __restrict__ zeros, int N, int K, int G,
                                                        int team_log2, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int team = 1 << team_log2;
  const int p = lane & (team - 1);
  const int r = lane >> team_log2;
  const int rps = 64 >> team_log2;  // rows per wave step
  const int cpr = K >> 5;           // chunks per row
  const int gpr = K / G;            // groups per row
  const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int waves = gridDim.x * kWaves;

  // Activation slice of this lane, resident for the whole kernel.
  uint32_t xr[CPL][16];
  float xsum[CPL];
  const uint32_t ones2 = XT::kMagic2 == F16::kMagic2 ? 0x3C003C00u : 0x3F803F80u;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = i * team + p;
    if (c < cpr) {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + 32 * c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4_t v = src[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) xr[i][4 * q + e] = v[e];
      }
      if (SCALE) {
        const float4_t* sp = reinterpret_cast<const float4_t*>(s + 32 * c);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float4_t sv = sp[q];
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const uint32_t pr = xr[i][2 * q + e / 2];
            const float a0 = XT::to_f32((uint16_t)(pr & 0xFFFFu)) / sv[e];
            const float a1 = XT::to_f32((uint16_t)(pr >> 16)) / sv[e + 1];
            xr[i][2 * q + e / 2] = (uint32_t)XT::from_f32(a0) | ((uint32_t)XT::from_f32(a1) << 16);
          }
        }
      }
      float t = 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) t = XT::dot2(xr[i][q], ones2, t);
      xsum[i] = t;
    } else {
#pragma unroll
      for (int q = 0; q < 16; ++q) xr[i][q] = 0u;
      xsum[i] = 0.0f;
    }
  }

  const float zsym = (float)(1 << (BITS - 1));
  for (int row0 = wave * rps * ROWS; row0 < N; row0 += waves * rps * ROWS) {
    ChunkCodes<BITS> cc[ROWS][CPL];
    float sc[ROWS][CPL], zc[ROWS][CPL];
    // Issue every load of the ROWS rows before any arithmetic.
#pragma unroll
    for (int rr = 0; rr < ROWS; ++rr) {
      const int n = row0 + rr * rps + r;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = i * team + p;
        if (n < N && c < cpr) {
          load_codes<BITS>(packed, n, K, c, cc[rr][i]);
          const int64_t gi = (int64_t)n * gpr + (32 * c) / G;
          sc[rr][i] = half_bits_to_f32(scales[gi]);
          zc[rr][i] = ASYM ? half_bits_to_f32(zeros[gi]) : zsym;
        } else {
#pragma unroll
          for (int j = 0; j < (BITS == 4 ? 4 : 3); ++j) cc[rr][i].w[j] = 0u;
          sc[rr][i] = 0.0f;
          zc[rr][i] = 0.0f;
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < ROWS; ++rr) {
      const int n = row0 + rr * rps + r;
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const float a = chunk_dot<BITS, XT>(cc[rr][i], xr[i]);
        acc += sc[rr][i] * (a - (XT::kMagic + zc[rr][i]) * xsum[i]);
      }
      acc = team_sum(acc, team);
      if (p == 0 && n < N) y[n] = XT::from_f32(acc);
    }
  }
}

template <int BITS, bool ASYM, class XT, int CPL, bool SCALE>
hipError_t launch_cpl(const void* x, const float* s, const void* packed, const void* scales, const void* zeros,
                      int64_t N, int64_t K, int G, int team_log2, void* y, hipStream_t stream) {
  constexpr int ROWS = 2;
  const int rps = 64 >> team_log2;
  const int64_t waves_needed = (N + (int64_t)rps * ROWS - 1) / ((int64_t)rps * ROWS);
  int64_t blocks = (waves_needed + kWaves - 1) / kWaves;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL((gemv_kernel<BITS, ASYM, XT, CPL, SCALE, ROWS>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(x), s, static_cast<const uint8_t*>(packed),
                     static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), (int)N, (int)K, G,
                     team_log2, static_cast<uint16_t*>(y));
  return hipGetLastError();
}

template <int BITS, bool ASYM, class XT, bool SCALE>
hipError_t launch_scale(const void* x, const float* s, const void* packed, const void* scales, const void* zeros,
                        int64_t N, int64_t K, int G, void* y, hipStream_t stream) {
  const int cpr = (int)(K / 32);
  int team_log2 = 0;
  while ((1 << team_log2) < cpr && team_log2 < 6) ++team_log2;
  const int team = 1 << team_log2;
  const int cpl = (cpr + team - 1) / team;
#define WOQ_CPL_CASE(C) \
  case C:               \
    return launch_cpl<BITS, ASYM, XT, C, SCALE>(x, s, packed, scales, zeros, N, K, G, team_log2, y, stream);
  switch (cpl) {
    WOQ_CPL_CASE(1)
    WOQ_CPL_CASE(2)
    WOQ_CPL_CASE(3)
    WOQ_CPL_CASE(4)
    WOQ_CPL_CASE(5)
    WOQ_CPL_CASE(6)
    WOQ_CPL_CASE(7)
    WOQ_CPL_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef WOQ_CPL_CASE
}

template <int BITS, bool ASYM, class XT>
hipError_t launch_xt(const void* x, const float* s, const void* packed, const void* scales, const void* zeros,
                     int64_t N, int64_t K, int G, void* y, hipStream_t stream) {
  return s ? launch_scale<BITS, ASYM, XT, true>(x, s, packed, scales, zeros, N, K, G, y, stream)
           : launch_scale<BITS, ASYM, XT, false>(x, s, packed, scales, zeros, N, K, G, y, stream);
}

template <int BITS, bool ASYM>
hipError_t launch_asym(const void* x, int xdtype, const float* s, const void* packed, const void* scales,
                       const void* zeros, int64_t N, int64_t K, int G, void* y, hipStream_t stream) {
  return xdtype == 0 ? launch_xt<BITS, ASYM, F16>(x, s, packed, scales, zeros, N, K, G, y, stream)
                     : launch_xt<BITS, ASYM, BF16>(x, s, packed, scales, zeros, N, K, G, y, stream);
}

}  // namespace

// Largest K the register-resident GEMV handles (8 chunks of 32 per lane).
int gemv_max_k() { return 64 * 8 * 32; }

hipError_t launch_gemv(const void* x, int xdtype, const float* act_scale, const void* packed, const void* scales,
                       const void* zeros, int64_t N, int64_t K, int bits, int group_size, bool asymmetric, void* y,
                       hipStream_t stream) {
  if (bits == 4)
    return asymmetric ? launch_asym<4, true>(x, xdtype, act_scale, packed, scales, zeros, N, K, group_size, y, stream)
                      : launch_asym<4, false>(x, xdtype, act_scale, packed, scales, zeros, N, K, group_size, y, stream);
  return asymmetric ? launch_asym<3, true>(x, xdtype, act_scale, packed, scales, zeros, N, K, group_size, y, stream)
                    : launch_asym<3, false>(x, xdtype, act_scale, packed, scales, zeros, N, K, group_size, y, stream);
}

}  // namespace woq
