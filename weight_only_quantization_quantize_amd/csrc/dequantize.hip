// Dequantization w_hat = (u - Z) * S to fp32, one thread per 32-weight chunk.
// The second half of pseudo-quantization ("MIT 6.5940 Lab 4 + Lab 5", Lab 4
// "Starting point and setup"); exact because |u - Z| < 16 and S carries 11
// significant bits.  Used to check the decode of layout v2 in isolation.
#include "woq_device.h"
#include "woq_internal.h"

namespace woq {
namespace {

constexpr int kThreads = 256;

template <int BITS, bool ASYM>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(const uint8_t* __restrict__ packed,
                                                              const uint16_t* __restrict__ scales,
                                                              const uint16_t* __restrict__ zeros,
                                                              int64_t total_chunks, int K, int G,
                                                              float* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= total_chunks) return;
  const int cpr = K >> 5;
  const int64_t n = c / cpr;
  const int kc = (int)(c - n * cpr);
  const int64_t gi = n * (K / G) + (kc * 32) / G;
  const float S = half_bits_to_f32(scales[gi]);
  const float Z = ASYM ? half_bits_to_f32(zeros[gi]) : (float)(1 << (BITS - 1));
  uint32_t u[32];
  if (BITS == 4) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(packed + n * (int64_t)(K / 2) + (int64_t)kc * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t pr = pair4(v[j], t, 0u);
        u[8 * j + 2 * t] = pr & 0xFFFFu;
        u[8 * j + 2 * t + 1] = pr >> 16;
      }
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(packed + n * (int64_t)(3 * K / 8) + (int64_t)kc * 12);
    const uint32_t w0 = p[0], w1 = p[1], w2 = p[2];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint32_t pr = pair3(w0, w1, w2, t, 0u);
      u[2 * t] = pr & 0xFFFFu;
      u[2 * t + 1] = pr >> 16;
    }
  }
  float4_t* dst = reinterpret_cast<float4_t*>(out + n * (int64_t)K + (int64_t)kc * 32);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    float4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = ((float)u[4 * q + e] - Z) * S;
    dst[q] = o;
  }
}

template <int BITS, bool ASYM>
hipError_t launch_typed(const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K, int G,
                        float* out, hipStream_t stream) {
  const int64_t total = N * (K / 32);
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((dequantize_kernel<BITS, ASYM>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint8_t*>(packed), static_cast<const uint16_t*>(scales),
                     static_cast<const uint16_t*>(zeros), total, (int)K, G, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize(const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K,
                             int bits, int group_size, bool asymmetric, float* out, hipStream_t stream) {
  if (bits == 4)
    return asymmetric ? launch_typed<4, true>(packed, scales, zeros, N, K, group_size, out, stream)
                      : launch_typed<4, false>(packed, scales, zeros, N, K, group_size, out, stream);
  return asymmetric ? launch_typed<3, true>(packed, scales, zeros, N, K, group_size, out, stream)
                    : launch_typed<3, false>(packed, scales, zeros, N, K, group_size, out, stream);
}

}  // namespace woq
