// Fused dequantize + GEMM for M >= 1 on gfx950 matrix cores:
//   Y[m, n] = sum_g S[n,g] * sum_{k in g} x'[m,k] (u[n,k] - Z[n,g]),  x' = X / s.
//
// The pages note that large batches are compute-bound, so weight-only
// quantization saves memory there but not time, and that the W4A16 path uses
// no 4-bit matrix instruction ("CMU 11-868 L19-L20", section "Back to the
// question: where does the speed come from?"; TinyChat record, hardware
// caveats).  Here the codes are widened to 16-bit floats and fed to
// v_mfma_f32_16x16x32_{f16,bf16}.
//
// Direct-decode kernel (this file): a workgroup of 4 waves owns a tile of
// 16*MT rows of X and 4 * 16*NT columns of W.  Per K-block of KB (32, 64 or
// 128, never crossing a group):
//  * X[m0:m0+16MT, kb:kb+KB] is staged through LDS once for the 4 waves
//    (divided by the AWQ scale and rounded when one is given), together with
//    each row's sum over the block;
//  * every lane loads the codes of its own B fragment straight from HBM (one
//    16-byte load per column tile for KB = 128), turns each code into the
//    16-bit float MAGIC + u (exact) and issues KB/32 MFMAs per (mt, nt);
//  * at the end of a group the fp32 partial sums are corrected and scaled,
//    acc += S (part - (MAGIC + Z) * sum x), so the only roundings are the
//    MFMA's fp32 accumulation and the final conversion of Y.
//
// MFMA operand slots: lane l of a 16x16x32 MFMA supplies A[m = l%16][slot
// 8*(l/16) + j] and B[slot 8*(l/16) + j][n = l%16], j = 0..7, and receives
// C[m = 4*(l/16) + i][n = l%16], i = 0..3.  Any assignment of K indices to
// slots that is the same for A and B gives the same product; the kernel gives
// lane group lg = l/16 the contiguous K range kb + lg*KB/4 + [0, KB/4) so its
// codes arrive in one load.
#include "woq_device.h"
#include "woq_internal.h"

namespace woq {
namespace {

constexpr int kThreads = 256;

template <int BITS, int KB>
struct BCodes;
template <int KB>
struct BCodes<4, KB> {
  uint32_t w[KB / 32];  // words of this lane's K range (8 codes each)
};
template <int KB>
struct BCodes<3, KB> {
  uint32_t w[3];  // the 32-weight unit holding this lane's K range
};

template <int BITS, int KB>
__device__ inline void load_b(const uint8_t* __restrict__ packed, int64_t n, int K, int kbeg, BCodes<BITS, KB>& b) {
  if (BITS == 4) {
    const uint8_t* p = packed + n * (int64_t)(K / 2) + kbeg / 2;
    if (KB == 128) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
      for (int j = 0; j < 4; ++j) b.w[j] = v[j];
    } else if (KB == 64) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      b.w[0] = v.x;
      b.w[KB / 32 - 1] = v.y;
    } else {
      b.w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
  } else {
    const uint32_t* p =
        reinterpret_cast<const uint32_t*>(packed + n * (int64_t)(3 * K / 8) + (int64_t)(kbeg / 32) * 12);
    b.w[0] = p[0];
    b.w[1] = p[1];
    b.w[2] = p[2];
  }
}

// B fragment (8 consecutive K of one column) for MFMA q of the K-block.
template <int BITS, int KB, class XT>
__device__ inline u32x4_t b_fragment(const BCodes<BITS, KB>& b, int q, int t0) {
  u32x4_t f;
  if (BITS == 4) {
#pragma unroll
    for (int t = 0; t < 4; ++t) f[t] = pair4(b.w[q], t, XT::kMagic2);
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) f[t] = pair3(b.w[0], b.w[1], b.w[2], t0 + 4 * q + t, XT::kMagic2);
  }
  return f;
}

template <int BITS, bool ASYM, class XT, int MT, int NT, int KB, bool SCALE>
__global__ __launch_bounds__(kThreads) void gemm_direct_kernel(
    const uint16_t* __restrict__ X, const float* __restrict__ s, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int M, int N, int K, int G,
    uint16_t* __restrict__ Y) {
  constexpr int BM = 16 * MT;
  constexpr int BN = 4 * 16 * NT;
  constexpr int XP = KB + 8;  // LDS row pitch in halves (16 B pad against bank conflicts)
  constexpr int SEG = KB / 8; // 16-byte segments per staged row
  // bf16 with an AWQ scale: x / s is staged as a bf16 pair hi + lo (about 16
  // significant bits) and each MFMA is issued for both halves.
  constexpr bool kSplitX = SCALE && XT::kMagic2 == BF16::kMagic2;
  __shared__ __attribute__((aligned(16))) uint16_t xs[BM * XP];
  __shared__ __attribute__((aligned(16))) uint16_t xl[kSplitX ? BM * XP : 8];
  __shared__ float xsum_s[BM];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int m0 = blockIdx.y * BM;
  const int nw = blockIdx.x * BN + wave * 16 * NT;
  const int gpr = K / G;
  const float zsym = (float)(1 << (BITS - 1));

  float4_t acc[MT][NT], part[MT][NT];
  float xg[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc[mt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
      part[mt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) xg[mt][i] = 0.f;
  }
  const uint32_t ones2 = XT::kMagic2 == F16::kMagic2 ? 0x3C003C00u : 0x3F803F80u;

  for (int kb = 0; kb < K; kb += KB) {
    // Codes of this K-block for every column tile (issued first: HBM latency).
    BCodes<BITS, KB> bc[NT];
    const int kbeg = kb + lg * (KB / 4);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // columns past N load row N-1 (always valid); their results are never stored
      const int n = nw + 16 * nt + lr;
      load_b<BITS, KB>(packed, n < N ? n : N - 1, K, kbeg, bc[nt]);
    }

    __syncthreads();  // previous block's LDS readers are done
    for (int it = threadIdx.x; it < BM * SEG; it += kThreads) {
      const int m = it / SEG, seg = it - m * SEG;
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u}, vl = v;
      if (m0 + m < M) v = *reinterpret_cast<const u32x4_t*>(X + (int64_t)(m0 + m) * K + kb + 8 * seg);
      if (SCALE) {
        const float4_t s0 = *reinterpret_cast<const float4_t*>(s + kb + 8 * seg);
        const float4_t s1 = *reinterpret_cast<const float4_t*>(s + kb + 8 * seg + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float d0 = e < 2 ? s0[2 * e] : s1[2 * e - 4];
          const float d1 = e < 2 ? s0[2 * e + 1] : s1[2 * e - 3];
          const float a0 = XT::to_f32((uint16_t)(v[e] & 0xFFFFu)) / d0;
          const float a1 = XT::to_f32((uint16_t)(v[e] >> 16)) / d1;
          const uint16_t h0 = XT::from_f32(a0), h1 = XT::from_f32(a1);
          v[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
          if (kSplitX)
            vl[e] = (uint32_t)XT::from_f32(a0 - XT::to_f32(h0)) | ((uint32_t)XT::from_f32(a1 - XT::to_f32(h1)) << 16);
        }
      }
      *reinterpret_cast<u32x4_t*>(&xs[m * XP + 8 * seg]) = v;
      if (kSplitX) *reinterpret_cast<u32x4_t*>(&xl[m * XP + 8 * seg]) = vl;
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) ps = XT::dot2(v[e], ones2, ps);
      if (kSplitX) {
#pragma unroll
        for (int e = 0; e < 4; ++e) ps = XT::dot2(vl[e], ones2, ps);
      }
      ps = team_sum(ps, SEG);
      if (seg == 0) xsum_s[m] = ps;
    }
    __syncthreads();

    const int t0 = BITS == 3 ? ((kbeg & 31) >> 1) : 0;
#pragma unroll
    for (int q = 0; q < KB / 32; ++q) {
      u32x4_t a[MT], al[kSplitX ? MT : 1];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        a[mt] = *reinterpret_cast<const u32x4_t*>(&xs[(16 * mt + lr) * XP + lg * (KB / 4) + 8 * q]);
        if constexpr (kSplitX)
          al[mt] = *reinterpret_cast<const u32x4_t*>(&xl[(16 * mt + lr) * XP + lg * (KB / 4) + 8 * q]);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const u32x4_t b = b_fragment<BITS, KB, XT>(bc[nt], q, t0);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          part[mt][nt] = XT::mfma16x16x32(a[mt], b, part[mt][nt]);
          if constexpr (kSplitX) part[mt][nt] = XT::mfma16x16x32(al[mt], b, part[mt][nt]);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) xg[mt][i] += xsum_s[16 * mt + 4 * lg + i];

    if ((kb + KB) % G == 0) {
      const int g = kb / G;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = nw + 16 * nt + lr;
        float S = 0.f, Z = zsym;
        if (n < N) {
          S = half_bits_to_f32(scales[(int64_t)n * gpr + g]);
          if (ASYM) Z = half_bits_to_f32(zeros[(int64_t)n * gpr + g]);
        }
        const float c = XT::kMagic + Z;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][nt][i] += S * (part[mt][nt][i] - c * xg[mt][i]);
          part[mt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) xg[mt][i] = 0.f;
    }
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = nw + 16 * nt + lr;
    if (n >= N) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 16 * mt + 4 * lg + i;
        if (m < M) Y[(int64_t)m * N + n] = XT::from_f32(acc[mt][nt][i]);
      }
  }
}

template <int BITS, bool ASYM, class XT, int MT, int NT, int KB>
hipError_t launch_tile(const void* X, const float* s, const void* packed, const void* scales, const void* zeros,
                       int64_t M, int64_t N, int64_t K, int G, void* Y, hipStream_t stream) {
  const dim3 grid((unsigned)((N + 64 * NT - 1) / (64 * NT)), (unsigned)((M + 16 * MT - 1) / (16 * MT)));
  if (s) {
    hipLaunchKernelGGL((gemm_direct_kernel<BITS, ASYM, XT, MT, NT, KB, true>), grid, dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(X), s, static_cast<const uint8_t*>(packed),
                       static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), (int)M, (int)N,
                       (int)K, G, static_cast<uint16_t*>(Y));
  } else {
    hipLaunchKernelGGL((gemm_direct_kernel<BITS, ASYM, XT, MT, NT, KB, false>), grid, dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(X), s, static_cast<const uint8_t*>(packed),
                       static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), (int)M, (int)N,
                       (int)K, G, static_cast<uint16_t*>(Y));
  }
  return hipGetLastError();
}

template <int BITS, bool ASYM, class XT, int KB>
hipError_t launch_kb(const void* X, const float* s, const void* packed, const void* scales, const void* zeros,
                     int64_t M, int64_t N, int64_t K, int G, void* Y, hipStream_t stream) {
  if (M <= 16) return launch_tile<BITS, ASYM, XT, 1, 1, KB>(X, s, packed, scales, zeros, M, N, K, G, Y, stream);
  if (M <= 32) return launch_tile<BITS, ASYM, XT, 2, 1, KB>(X, s, packed, scales, zeros, M, N, K, G, Y, stream);
  if (M <= 64) return launch_tile<BITS, ASYM, XT, 4, 1, KB>(X, s, packed, scales, zeros, M, N, K, G, Y, stream);
  return launch_tile<BITS, ASYM, XT, 4, 4, KB>(X, s, packed, scales, zeros, M, N, K, G, Y, stream);
}

template <int BITS, bool ASYM, class XT>
hipError_t launch_xt(const void* X, const float* s, const void* packed, const void* scales, const void* zeros,
                     int64_t M, int64_t N, int64_t K, int G, void* Y, hipStream_t stream) {
  if (G % 128 == 0) return launch_kb<BITS, ASYM, XT, 128>(X, s, packed, scales, zeros, M, N, K, G, Y, stream);
  if (G % 64 == 0) return launch_kb<BITS, ASYM, XT, 64>(X, s, packed, scales, zeros, M, N, K, G, Y, stream);
  return launch_kb<BITS, ASYM, XT, 32>(X, s, packed, scales, zeros, M, N, K, G, Y, stream);
}

template <int BITS, bool ASYM>
hipError_t launch_asym(const void* X, int xdtype, const float* s, const void* packed, const void* scales,
                       const void* zeros, int64_t M, int64_t N, int64_t K, int G, void* Y, hipStream_t stream) {
  return xdtype == 0 ? launch_xt<BITS, ASYM, F16>(X, s, packed, scales, zeros, M, N, K, G, Y, stream)
                     : launch_xt<BITS, ASYM, BF16>(X, s, packed, scales, zeros, M, N, K, G, Y, stream);
}

}  // namespace

// Rows of X from which the LDS-staged MFMA kernel replaces the direct-decode
// kernel; its fp16 variant steps K by 64.
constexpr int64_t kLdsGemmMinM = 128;

hipError_t launch_gemm(const void* X, int xdtype, const float* act_scale, const void* packed, const void* scales,
                       const void* zeros, int64_t M, int64_t N, int64_t K, int bits, int group_size, bool asymmetric,
                       void* Y, hipStream_t stream) {
  if (M >= kLdsGemmMinM && (xdtype != 0 || K % 64 == 0))
    return launch_gemm_lds(X, xdtype, act_scale, packed, scales, zeros, M, N, K, bits, group_size, asymmetric, Y,
                           stream);
  if (bits == 4)
    return asymmetric
               ? launch_asym<4, true>(X, xdtype, act_scale, packed, scales, zeros, M, N, K, group_size, Y, stream)
               : launch_asym<4, false>(X, xdtype, act_scale, packed, scales, zeros, M, N, K, group_size, Y, stream);
  return asymmetric
             ? launch_asym<3, true>(X, xdtype, act_scale, packed, scales, zeros, M, N, K, group_size, Y, stream)
             : launch_asym<3, false>(X, xdtype, act_scale, packed, scales, zeros, M, N, K, group_size, Y, stream);
}

}  // namespace woq
