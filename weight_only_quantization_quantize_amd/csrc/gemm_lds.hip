// Large-M fused dequantize + GEMM on gfx950 matrix cores (prefill shapes):
// bf16 activations, 3-bit codes, and fp16 shapes whose 256 x 256 tiles fill
// the compute units in whole rounds (fp16 with 4-bit codes otherwise goes to
// gemm_regb.hip).
//
// At large M the product is compute-bound, which is why weight-only
// quantization brings no speed-up there ("CMU 11-868 L19-L20", section "Back
// to the question: where does the speed come from?"); the packed weights only
// have to be dequantized once per workgroup tile and fed to fp16/bf16 MFMA.
//
// Tiling: a workgroup of 8 waves computes a 256 x 256 tile of Y (2 x 4 waves,
// 128 x 64 each, as 4 x 2 v_mfma_f32_32x32x16 tiles with 128 fp32
// accumulators per lane; two waves per SIMD hide each other's waits).  The K
// loop advances BK (64 for fp16, 32 for bf16) at a time through a
// double-buffered LDS stage holding
//   A: X[m0:m0+256, k:k+BK] (for fp16 with an AWQ scale, x * act_recip(s)
//      rounded once),
//   B: w_hat[n0:n0+256, k:k+BK] = (u - Z) * S rounded to the activation type
//      (for bf16 with an AWQ scale, (u - Z) * S * act_recip(s)),
// decoded once per workgroup from the packed codes: thread t owns half of
// column n0 + t/2 (BK/2 codes, which never cross a group since G % 32 == 0)
// and its (S, Z).  The code pair is widened exactly, (1024 + u) - (1024 + Z) =
// u - Z in fp16, and multiplied by S once (the only rounding of the weight).
// bf16 has only 8 significant bits, so for bf16 activations the weight is
// kept as the sum of two bf16 values, hi = bf16(w_hat) and lo = bf16(w_hat -
// hi), and each K step issues the MFMAs twice (X hi + X lo): the weight error
// drops from 2^-9 to about 2^-17 relative, at twice the MFMA work of fp16.
//
// X is loaded two blocks ahead and the packed codes kPB blocks ahead, each in
// a ring of registers; block k + 1 is written to the other LDS stage after
// block k's MFMAs, so one barrier per block suffices.  Tiles are assigned so that each of the 8 XCDs works on a
// contiguous range of the tile grid with the N tile index fastest: the
// 256-row X tile a range shares stays in that XCD's L2.
//
// MFMA operand slots (32x32x16): lane l supplies A[m = l%32][k = 8(l/32)+j]
// and B[k = 8(l/32)+j][n = l%32], j = 0..7, and holds C[m = 8(v/4) + 4(l/32) +
// v%4][n = l%32] in accumulator v = 0..15.
#include "woq_device.h"
#include "woq_internal.h"

namespace woq {
namespace {

typedef float float16_t __attribute__((ext_vector_type(16)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = 256, kBN = 256;
constexpr int kThreads = 512;

// K block per LDS stage: 64 for fp16 (two stages of A and B fill 144 KiB of
// LDS), 32 for bf16, which also stages the low halves of the split weight.
template <class XT>
struct Tiling {
  static constexpr bool kSplit = XT::kMagic2 == BF16::kMagic2;
  static constexpr int BK = kSplit ? 32 : 64;
  static constexpr int LD = BK + 8;  // row pitch in halves; odd multiple of 16 B keeps ds_read_b128 conflict-free
  static constexpr int kStage = kBM * LD;  // halves per operand stage (kBM == kBN)
  static constexpr int kSegs = BK / 8;     // 16-byte segments per row
  static constexpr int kAUnits = kBM * kSegs / kThreads;  // A segments per thread
  static constexpr int kCodes = BK / 2;    // codes per thread (two threads per column)
};

__device__ inline float16_t mfma32(u32x4_t a, u32x4_t b, float16_t c, F16) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0,
                                                0, 0);
}
__device__ inline float16_t mfma32(u32x4_t a, u32x4_t b, float16_t c, BF16) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf168_t, a), __builtin_bit_cast(bf168_t, b), c,
                                                 0, 0, 0);
}

// fp16 pair (u - Z) * S for codes held in the low bits of each 16-bit half:
// (1024 + u) - (1024 + Z) is exact, the product is the one rounding.
__device__ inline uint32_t dequant_pair_f16(uint32_t codes2, uint32_t zmagic2, uint32_t s2) {
  const h2_t p = __builtin_bit_cast(h2_t, codes2 | 0x64006400u);
  const h2_t d = p - __builtin_bit_cast(h2_t, zmagic2);
  return __builtin_bit_cast(uint32_t, d * __builtin_bit_cast(h2_t, s2));
}

// bf16 pair (hi, lo) with hi + lo = (u - Z) * S * r to about 16 significant
// bits; (u - Z) * S is exact in fp32, r is the folded activation factor.
template <bool SCALE>
__device__ inline void dequant_pair_split(uint32_t codes2, float Z, float S, float r0, float r1, uint32_t& hi,
                                          uint32_t& lo) {
  float a = ((float)(codes2 & 0xFFFFu) - Z) * S;
  float b = ((float)(codes2 >> 16) - Z) * S;
  if constexpr (SCALE) {
    a *= r0;
    b *= r1;
  }
  const uint16_t ah = BF16::from_f32(a), bh = BF16::from_f32(b);
  const uint16_t al = BF16::from_f32(a - BF16::to_f32(ah)), bl = BF16::from_f32(b - BF16::to_f32(bh));
  hi = (uint32_t)ah | ((uint32_t)bh << 16);
  lo = (uint32_t)al | ((uint32_t)bl << 16);
}

// Code pair t (K offsets 2t, 2t + 1 of this thread's codes) in the low bits of
// each 16-bit half.  4-bit: word t / 4 holds 8 codes, pair t % 4 at bits
// [4 (t % 4)] and [16 + 4 (t % 4)].  3-bit: w[0..2] are the three words of the
// 32-code unit and the thread's codes start at pair pair_base of the unit (0,
// or 8 when two threads share a unit).
template <int BITS>
__device__ inline uint32_t code_pair(const uint32_t* w, int t, int pair_base) {
  if constexpr (BITS == 4) {
    return (w[t >> 2] >> (4 * (t & 3))) & 0x000F000Fu;
  } else {
    return pair3(w[0], w[1], w[2], pair_base + t, 0u);
  }
}

#ifndef WOQ_LDS_PB
#define WOQ_LDS_PB 2
#endif
constexpr int kPB = WOQ_LDS_PB;  // blocks of packed codes in flight
// Blocks of X in flight: 2, except for bf16 with an AWQ scale, whose folded
// weight path needs the registers.
template <class XT, bool SCALE>
constexpr int x_prefetch() {
  return XT::kMagic2 == BF16::kMagic2 && SCALE ? 1 : 2;
}

template <int BITS, bool ASYM, class XT, bool SCALE>
__global__ __launch_bounds__(kThreads) void gemm_lds_kernel(
    const uint16_t* __restrict__ X, const float* __restrict__ s, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int M, int N, int K, int G,
    uint16_t* __restrict__ Y, int tiles_m, int tiles_n) {
  using TL = Tiling<XT>;
  constexpr int BK = TL::BK, LD = TL::LD, kStage = TL::kStage;
  constexpr bool kSplit = TL::kSplit;
  // [A0 | A1 | B0 | B1 (| Bl0 | Bl1)], each stage kStage halves
  __shared__ __attribute__((aligned(16))) uint16_t lds[(kSplit ? 6 : 4) * kStage];

  // XCD-aware tile order: consecutive workgroup ids go to different XCDs, so
  // give XCD x the contiguous tile range [x * per_xcd, (x + 1) * per_xcd).
  const int T = tiles_m * tiles_n;
  const int per_xcd = (T + 7) / 8;
  const int tile = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (tile >= T) return;
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves of 128 x 64
  const int gpr = K / G;
  const int kblocks = K / BK;

  // A staging: thread t owns segment t % kSegs of rows t / kSegs + i * (512 /
  // kSegs).  Rows past M read row M - 1; their outputs are never stored.
  constexpr int kRowStep = kThreads / TL::kSegs;
  const int a_seg = tid % TL::kSegs, a_r0 = tid / TL::kSegs;
  const uint16_t* a_src[TL::kAUnits];
#pragma unroll
  for (int i = 0; i < TL::kAUnits; ++i) {
    const int r = m0 + a_r0 + kRowStep * i;
    a_src[i] = X + (int64_t)(r < M ? r : M - 1) * K + 8 * a_seg;
  }
  const uint32_t a_dst = (uint32_t)(a_r0 * LD + 8 * a_seg);
  // B staging: thread t owns half h = t % 2 of the codes of column n0 + t / 2.
  const int b_half = tid & 1, b_lcol = tid >> 1;
  const int b_col = n0 + b_lcol < N ? n0 + b_lcol : N - 1;
  const uint8_t* b_src = packed + (int64_t)b_col * (K * BITS / 8);
  const int64_t g_row = (int64_t)b_col * gpr;
  const uint32_t b_dst = (uint32_t)(2 * kStage + b_lcol * LD + (BK / 2) * b_half);

  // With an AWQ scale, fp16 stages x * act_recip(s) in A; bf16 keeps X exact
  // and folds act_recip(s) into the split weight instead, since rounding x / s
  // to 8 significant bits would dominate the error when a few scaled channels
  // carry the output.
  constexpr bool kScaleA = SCALE && !kSplit, kScaleB = SCALE && kSplit;
  constexpr int kPA = x_prefetch<XT, SCALE>();
  // X is loaded kPA blocks ahead and the packed codes kPB blocks ahead, each
  // in a ring of registers.
  struct ARegs {
    u32x4_t a[TL::kAUnits];
    float4_t sv[kScaleB ? TL::kCodes / 4 : 1];  // s[k] of this thread's codes
  };
  struct BRegs {
    uint32_t w[BITS == 4 ? TL::kCodes / 8 : 3];
    uint16_t s16, z16;
  };
  auto load_a = [&](ARegs& R, int kb) {
#pragma unroll
    for (int i = 0; i < TL::kAUnits; ++i) R.a[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + kb);
    if constexpr (kScaleB) {
      const int kc = kb + (BK / 2) * b_half;
#pragma unroll
      for (int j = 0; j < TL::kCodes / 4; ++j) R.sv[j] = *reinterpret_cast<const float4_t*>(s + kc + 4 * j);
    }
  };
  auto load_b = [&](BRegs& R, int kb) {
    const int kc = kb + (BK / 2) * b_half;  // first K of this thread's codes
    if constexpr (BITS == 4) {
      if constexpr (TL::kCodes == 32) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(b_src + kc / 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) R.w[j] = v[j];
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(b_src + kc / 2);
        R.w[0] = v.x;
        R.w[1] = v.y;
      }
    } else {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(b_src + (kc / 32) * 12);
      R.w[0] = p[0];
      R.w[1] = p[1];
      R.w[2] = p[2];
    }
    const int64_t gi = g_row + kc / G;
    R.s16 = scales[gi];
    R.z16 = ASYM ? zeros[gi] : (uint16_t)0;
  };
  auto store_block = [&](const ARegs& RA, const BRegs& R, int st, int kb) {
    uint16_t* base = lds + st * kStage;
    float inv[8];
    if constexpr (kScaleA) {
      const float4_t s0 = *reinterpret_cast<const float4_t*>(s + kb + 8 * a_seg);
      const float4_t s1 = *reinterpret_cast<const float4_t*>(s + kb + 8 * a_seg + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        inv[e] = act_recip(s0[e]);
        inv[e + 4] = act_recip(s1[e]);
      }
    }
#pragma unroll
    for (int i = 0; i < TL::kAUnits; ++i) {
      u32x4_t v = RA.a[i];
      if constexpr (kScaleA) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = XT::to_f32((uint16_t)(v[e] & 0xFFFFu)) * inv[2 * e];
          const float x1 = XT::to_f32((uint16_t)(v[e] >> 16)) * inv[2 * e + 1];
          v[e] = (uint32_t)XT::from_f32(x0) | ((uint32_t)XT::from_f32(x1) << 16);
        }
      }
      *reinterpret_cast<u32x4_t*>(base + a_dst + kRowStep * LD * i) = v;
    }
    const float S = half_bits_to_f32(R.s16);
    const float Z = ASYM ? half_bits_to_f32(R.z16) : (float)(1 << (BITS - 1));
    const int pair_base = TL::kCodes == 32 ? 0 : 8 * ((kb / 16 + b_half) & 1);
    constexpr int kPairs = TL::kCodes / 2;
    uint32_t hi[kPairs], lo[kPairs];
    if constexpr (kSplit) {
#pragma unroll
      for (int t = 0; t < kPairs; ++t) {
        float r0 = 1.0f, r1 = 1.0f;
        if constexpr (kScaleB) {
          r0 = act_recip(RA.sv[t >> 1][2 * (t & 1)]);
          r1 = act_recip(RA.sv[t >> 1][2 * (t & 1) + 1]);
        }
        dequant_pair_split<kScaleB>(code_pair<BITS>(R.w, t, pair_base), Z, S, r0, r1, hi[t], lo[t]);
      }
    } else {
      const uint32_t zh = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(1024.0f + Z));
      const uint32_t zmagic2 = zh | (zh << 16);
      const uint32_t s2 = (uint32_t)R.s16 | ((uint32_t)R.s16 << 16);
#pragma unroll
      for (int t = 0; t < kPairs; ++t) hi[t] = dequant_pair_f16(code_pair<BITS>(R.w, t, pair_base), zmagic2, s2);
    }
#pragma unroll
    for (int q = 0; q < kPairs / 4; ++q) {
      *reinterpret_cast<u32x4_t*>(base + b_dst + 8 * q) = u32x4_t{hi[4 * q], hi[4 * q + 1], hi[4 * q + 2], hi[4 * q + 3]};
      if constexpr (kSplit)
        *reinterpret_cast<u32x4_t*>(base + 2 * kStage + b_dst + 8 * q) =
            u32x4_t{lo[4 * q], lo[4 * q + 1], lo[4 * q + 2], lo[4 * q + 3]};
    }
  };

  float16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int fr = lane & 31, fk = 8 * (lane >> 5);
  const uint32_t a_rd = (uint32_t)((wm * 128 + fr) * LD + fk);
  const uint32_t b_rd = (uint32_t)(2 * kStage + (wn * 64 + fr) * LD + fk);
  auto mma_block = [&](int st) {
    const uint16_t* base = lds + st * kStage;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4_t a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const u32x4_t*>(base + a_rd + 32 * LD * i + 16 * ks);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const u32x4_t*>(base + b_rd + 32 * LD * j + 16 * ks);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j], XT{});
      if constexpr (kSplit) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          b[j] = *reinterpret_cast<const u32x4_t*>(base + 2 * kStage + b_rd + 32 * LD * j + 16 * ks);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j], XT{});
      }
    }
  };

  // Two LDS stages: while block kt is multiplied, X up to block kt + kPA and
  // codes up to block kt + kPB are in flight; block kt + 1 is then written to
  // the other stage; one barrier per block.  Block indices past the end are
  // clamped to the last block (reloaded, written to the unused stage), which
  // keeps the loop free of branches.
  const int last = kblocks - 1;
  ARegs RA[kPA];
  BRegs RB[kPB];
#pragma unroll
  for (int j = 0; j < kPA; ++j) load_a(RA[j], (j < last ? j : last) * BK);
#pragma unroll
  for (int j = 0; j < kPB; ++j) load_b(RB[j], (j < last ? j : last) * BK);
  store_block(RA[0], RB[0], 0, 0);
  __syncthreads();
  for (int kt = 0; kt < kblocks; ++kt) {
    const int nxt = kt + 1 < kblocks ? kt + 1 : last;
    const int far_a = kt + kPA < kblocks ? kt + kPA : last;
    const int far_b = kt + kPB < kblocks ? kt + kPB : last;
#pragma unroll
    for (int j = 0; j + 1 < kPA; ++j) RA[j] = RA[j + 1];
    load_a(RA[kPA - 1], far_a * BK);
#pragma unroll
    for (int j = 0; j + 1 < kPB; ++j) RB[j] = RB[j + 1];
    load_b(RB[kPB - 1], far_b * BK);
    mma_block(kt & 1);
    store_block(RA[0], RB[0], (kt + 1) & 1, nxt * BK);
    __syncthreads();
  }

  // Epilogue: for accumulator (i, j, v) the 32 lanes of each half-wave hold
  // 32 consecutive columns of one row.
  const int row_base = m0 + wm * 128 + 4 * (lane >> 5);
  const int col_base = n0 + wn * 64 + fr;
  uint16_t* __restrict__ yb = Y + (int64_t)row_base * N + col_base;
  if (m0 + kBM <= M && n0 + kBN <= N) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        uint16_t* __restrict__ yr = yb + (int64_t)(32 * i + 8 * (v >> 2) + (v & 3)) * N;
#pragma unroll
        for (int j = 0; j < 2; ++j) yr[32 * j] = XT::from_f32(acc[i][j][v]);
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int dm = 32 * i + 8 * (v >> 2) + (v & 3);
        if (row_base + dm >= M) continue;
        uint16_t* __restrict__ yr = yb + (int64_t)dm * N;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (col_base + 32 * j < N) yr[32 * j] = XT::from_f32(acc[i][j][v]);
      }
  }
}

template <int BITS, bool ASYM, class XT>
hipError_t launch_xt(const void* X, const float* s, const void* packed, const void* scales, const void* zeros,
                     int64_t M, int64_t N, int64_t K, int G, void* Y, hipStream_t stream) {
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kBN - 1) / kBN);
  const int T = tiles_m * tiles_n;
  const unsigned blocks = 8u * (unsigned)((T + 7) / 8);
  if (s) {
    hipLaunchKernelGGL((gemm_lds_kernel<BITS, ASYM, XT, true>), dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(X), s, static_cast<const uint8_t*>(packed),
                       static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), (int)M, (int)N,
                       (int)K, G, static_cast<uint16_t*>(Y), tiles_m, tiles_n);
  } else {
    hipLaunchKernelGGL((gemm_lds_kernel<BITS, ASYM, XT, false>), dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(X), s, static_cast<const uint8_t*>(packed),
                       static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), (int)M, (int)N,
                       (int)K, G, static_cast<uint16_t*>(Y), tiles_m, tiles_n);
  }
  return hipGetLastError();
}

template <int BITS, bool ASYM>
hipError_t launch_asym(const void* X, int xdtype, const float* s, const void* packed, const void* scales,
                       const void* zeros, int64_t M, int64_t N, int64_t K, int G, void* Y, hipStream_t stream) {
  return xdtype == 0 ? launch_xt<BITS, ASYM, F16>(X, s, packed, scales, zeros, M, N, K, G, Y, stream)
                     : launch_xt<BITS, ASYM, BF16>(X, s, packed, scales, zeros, M, N, K, G, Y, stream);
}

}  // namespace

hipError_t launch_gemm_lds(const void* X, int xdtype, const float* act_scale, const void* packed,
                           const void* scales, const void* zeros, int64_t M, int64_t N, int64_t K, int bits,
                           int group_size, bool asymmetric, void* Y, hipStream_t stream) {
  if (bits == 4)
    return asymmetric
               ? launch_asym<4, true>(X, xdtype, act_scale, packed, scales, zeros, M, N, K, group_size, Y, stream)
               : launch_asym<4, false>(X, xdtype, act_scale, packed, scales, zeros, M, N, K, group_size, Y, stream);
  return asymmetric
             ? launch_asym<3, true>(X, xdtype, act_scale, packed, scales, zeros, M, N, K, group_size, Y, stream)
             : launch_asym<3, false>(X, xdtype, act_scale, packed, scales, zeros, M, N, K, group_size, Y, stream);
}

}  // namespace woq
