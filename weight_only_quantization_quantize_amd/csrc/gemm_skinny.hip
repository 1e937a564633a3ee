// Small-batch fused dequantize + GEMM (2 <= M <= 64, 4-bit codes, group 128)
// on gfx950 matrix cores:
//   Y[m, n] = sum_g S[n,g] * sum_{k in g} x'[m,k] (u[n,k] - Z[n,g]),  x' = X / s.
//
// At a few rows of X the layer is still bound by streaming the packed weights
// from HBM, as for the M = 1 decode GEMV ("MIT 6.5940 Lab 4 + Lab 5", Lab 4
// "Starting point and setup"; "CMU 11-868 L19-L20", section "Back to the
// question: where does the speed come from?").  This kernel keeps the whole
// of X' a wave needs in registers and streams the codes past it, so that the
// only traffic per output column is its codes, scales and zero points.
//
// Work split.  A workgroup is 16 waves; wave w owns the K blocks
// [w BPW, (w + 1) BPW) of 128 weights (one group each), so K = 2048 BPW
// (BPW = 1, 2 or 4).  It loads its A fragments (16 rows of X', rows >= M as
// zeros) once: 16 BPW registers per lane.  The workgroup then walks output
// tiles of 16 columns, tile = g, g + G, ... for its column group g of G:
// every wave computes the 16 x 16 partial of its K blocks with
// v_mfma_f32_16x16x32_{f16,bf16}, the 16 partials meet in LDS (one barrier
// per tile, double-buffered) and four waves add them in a fixed order and
// store Y.  More than 16 rows are cut into row tiles of 16, one workgroup
// each, whose workgroups run side by side on one XCD so that the codes they
// share are fetched from HBM about once.
//
// K order inside a block.  Lane (r, q) (r = lane % 16, q = lane / 16) supplies
// at MFMA step s the 8 slots of K offsets 32 q + 8 s + j (j = 0..7) for both
// A and B, so each slot is summed once and a lane's codes of the block are one
// 16-byte chunk of layout v2, word s holding step s.
//
// Loads.  Codes and X are read in row-contiguous runs (a load never splits a
// row's segment over lanes of different rows) and turned into MFMA fragments
// through a per-wave LDS buffer that only the wave itself touches.
//
// Decode.  A code pair becomes the 16-bit floats MAGIC + u (one v_and_or_b32),
// and per group acc += S (part - (MAGIC + Z) sum x), where sum x over the
// group comes from MFMAs against an all-ones B fragment, computed once per
// workgroup and kept in LDS.  The weights are never rounded; the only
// roundings are the MFMA's fp32 accumulation and the final conversion of Y.
//
// Pipelining.  The next tile's codes, scales and zero points are loaded as
// soon as the current tile's codes are staged, so one tile is always in
// flight per wave (16 waves per compute unit).
#include "woq_device.h"
#include "woq_internal.h"

namespace woq {
namespace {

constexpr int kSkWaves = 16;          // waves per workgroup
constexpr int kSkBlock = 128;         // K per block (= the group size)
constexpr int kSkMaxBlocks = 4;       // K blocks per wave (K <= 8192; 3 would spill registers)
constexpr int kSkTargetBlocks = 256;  // workgroups: one per compute unit
constexpr int kSkPitch = 272;         // staged row of 256 bytes + 16 against LDS bank conflicts

template <class XT, int BPW, bool ASYM, bool SCALE>
__global__ __launch_bounds__(kSkWaves * 64) void gemm_skinny_kernel(
    const uint16_t* __restrict__ X, const float* __restrict__ s, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int M, int N, int K, int rtp,
    uint16_t* __restrict__ Y) {
  // Workgroup b = x + 8 (rt + rtp z), x < 8: row tile rt (rows 16 rt ..
  // 16 rt + 15) of column group x + 8 z.  The rtp row tiles of a column group
  // are 8 apart in dispatch order, so they land on the same XCD and share its
  // L2: the codes come from HBM about once and the other row tiles read them
  // from L2 at the same time.
  const int bx = (int)blockIdx.x & 7, brest = (int)blockIdx.x >> 3;
  const int rt = brest % rtp, cgroup = bx + 8 * (brest / rtp), ngroups = (int)gridDim.x / rtp;
  const int row0 = 16 * rt;
  if (row0 >= M) return;  // a row tile past M: the whole workgroup leaves before any barrier
  X += (int64_t)row0 * K;
  Y += (int64_t)row0 * N;
  M = M - row0 < 16 ? M - row0 : 16;
  // Per wave: a 16-row staging buffer that turns row-contiguous global loads
  // into MFMA fragments; the partials of the cross-wave sum; sum x per block.
  __shared__ __attribute__((aligned(16))) uint8_t stage_all[kSkWaves][16 * kSkPitch];
  __shared__ float red[2][kSkWaves][256];
  __shared__ float4_t xgl[kSkWaves][BPW][4];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int kw = wave * BPW * kSkBlock;  // first K of this wave's blocks
  const int gpr = K / kSkBlock;
  const int g0 = wave * BPW;             // first group of this wave's blocks
  const int tiles = (N + 15) >> 4;
  const uint32_t magic2 = vgpr_const(XT::kMagic2);
  const uint32_t ones2 = XT::kMagic2 == F16::kMagic2 ? 0x3C003C00u : 0x3F803F80u;
  uint8_t* const stage = stage_all[wave];

  // Codes of a tile: each of the 16 columns holds 64 BPW bytes of this wave's
  // K range.  Load i reads CPI whole column segments (LPC lanes of 16 bytes
  // each), so every load covers contiguous runs of memory; the segments are
  // staged in LDS with pitch CP and lane (r, q) reads its chunk of block b at
  // column r, byte 64 b + 16 q.
  constexpr int LPC = 4 * BPW, CPI = 16 / BPW, CP = 64 * BPW + 16;
  u32x4_t c[BPW];
  auto load_codes = [&](int tile) {
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      int n = tile * 16 + i * CPI + lane / LPC;
      n = n < N ? n : N - 1;  // past N: column N - 1, never stored
      c[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(packed + (int64_t)n * (K / 2) + kw / 2 + 16 * (lane % LPC)));
    }
  };
  auto stage_codes = [&]() {
#pragma unroll
    for (int i = 0; i < BPW; ++i)
      *reinterpret_cast<u32x4_t*>(stage + (i * CPI + lane / LPC) * CP + 16 * (lane % LPC)) = c[i];
  };
  // Scales and zero points of the lane's column for the wave's BPW groups:
  // 32-bit loads when BPW is even (the host checks 4-byte alignment).
  constexpr int kSZW = BPW % 2 == 0 ? BPW / 2 : BPW;
  uint32_t sw[kSZW], zw[kSZW];
  auto load_sz = [&](int tile) {
    int n = tile * 16 + lr;
    n = n < N ? n : N - 1;
    const int64_t gi = (int64_t)n * gpr + g0;
#pragma unroll
    for (int j = 0; j < kSZW; ++j) {
      if constexpr (BPW % 2 == 0) {
        sw[j] = reinterpret_cast<const uint32_t*>(scales + gi)[j];
        if (ASYM) zw[j] = reinterpret_cast<const uint32_t*>(zeros + gi)[j];
      } else {
        sw[j] = scales[gi + j];
        if (ASYM) zw[j] = zeros[gi + j];
      }
    }
  };
  auto half_of = [&](const uint32_t (&w)[kSZW], int b) -> uint16_t {
    if constexpr (BPW % 2 == 0) return (uint16_t)(w[b >> 1] >> (16 * (b & 1)));
    return (uint16_t)w[b];
  };

  // X' rows 0..15 of this wave's K range (rows >= M are zeros).  Load i of
  // block b reads rows 4 i .. 4 i + 3, 256 contiguous bytes each; after
  // staging, lane (r, q) holds at step st the 8 values of row r at K offsets
  // 128 b + 32 q + 8 st + j of the range (the same K order as its codes).
  u32x4_t a[BPW][4];
#pragma unroll
  for (int b = 0; b < BPW; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * i + (lane >> 4);
      a[b][i] = row < M ? *reinterpret_cast<const u32x4_t*>(X + (int64_t)row * K + kw + kSkBlock * b + 8 * lr)
                        : u32x4_t{0u, 0u, 0u, 0u};
    }
  int tile = cgroup;
  load_codes(tile);
  load_sz(tile);

  if constexpr (SCALE) {
    // x' = x * (1 / s) rounded once to the activation type
#pragma unroll
    for (int b = 0; b < BPW; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* sp = s + kw + kSkBlock * b + 8 * lr;
        const float4_t s0 = *reinterpret_cast<const float4_t*>(sp);
        const float4_t s1 = *reinterpret_cast<const float4_t*>(sp + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t v = a[b][i][e];
          const float d0 = e < 2 ? s0[2 * e] : s1[2 * e - 4];
          const float d1 = e < 2 ? s0[2 * e + 1] : s1[2 * e - 3];
          const uint16_t h0 = XT::from_f32(XT::to_f32((uint16_t)(v & 0xFFFFu)) * act_recip(d0));
          const uint16_t h1 = XT::from_f32(XT::to_f32((uint16_t)(v >> 16)) * act_recip(d1));
          a[b][i][e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        }
      }
  }
  // Through the staging buffer, one block at a time (LDS operations of a wave
  // run in order, so block b + 1 may overwrite what block b's reads took).
#pragma unroll
  for (int b = 0; b < BPW; ++b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t*>(stage + (4 * i + (lane >> 4)) * kSkPitch + 16 * lr) = a[b][i];
#pragma unroll
    for (int st = 0; st < 4; ++st)
      a[b][st] = *reinterpret_cast<const u32x4_t*>(stage + lr * kSkPitch + 64 * lq + 16 * st);
  }

  // Sum of x' over each block, in the C layout (rows 4 q + i), from MFMAs
  // against an all-ones B fragment; lanes of column 0 keep it in LDS.
  const u32x4_t ones = u32x4_t{ones2, ones2, ones2, ones2};
#pragma unroll
  for (int b = 0; b < BPW; ++b) {
    float4_t xg = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) xg = XT::mfma16x16x32(a[b][st], ones, xg);
    if (lr == 0) xgl[wave][b][lq] = xg;
  }

  const float zsym = 8.0f;  // symmetric 4-bit codes are stored as q + 8
  for (int it = 0; tile < tiles; tile += ngroups, ++it) {
    const int next = tile + ngroups < tiles ? tile + ngroups : tiles - 1;
    float S[BPW], C[BPW];
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
      S[b] = half_bits_to_f32(half_of(sw, b));
      C[b] = XT::kMagic + (ASYM ? half_bits_to_f32(half_of(zw, b)) : zsym);
    }
    load_sz(next);  // a whole tile ahead, like the codes
    stage_codes();
    load_codes(next);  // clamped in range on the last tile
    float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
      const u32x4_t ch = *reinterpret_cast<const u32x4_t*>(stage + lr * CP + 64 * b + 16 * lq);
      float4_t part = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        u32x4_t bf;
#pragma unroll
        for (int t = 0; t < 4; ++t) bf[t] = pair4(ch[st], t, magic2);
        part = XT::mfma16x16x32(a[b][st], bf, part);
      }
      const float4_t xg = xgl[wave][b][lq];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += S[b] * (part[i] - C[b] * xg[i]);
    }

    // acc holds rows 4 q + i of column r of this wave's partial.
    float* r = &red[it & 1][wave][0];
#pragma unroll
    for (int i = 0; i < 4; ++i) r[(4 * lq + i) * 16 + lr] = acc[i];
    __syncthreads();
    if (threadIdx.x < 256) {
      const int o = threadIdx.x, m = o >> 4;
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kSkWaves; ++w) v += red[it & 1][w][o];
      const int n = tile * 16 + (o & 15);
      if (m < M && n < N) Y[(int64_t)m * N + n] = XT::from_f32(v);
    }
  }
}

template <class XT, int BPW, bool ASYM>
hipError_t launch_bpw(const void* X, const float* s, const void* packed, const void* scales, const void* zeros,
                      int64_t M, int64_t N, int64_t K, void* Y, hipStream_t stream) {
  // Row tiles of 16 (1, 2 or 4 slots; a slot past M exits at once) times
  // column groups, a multiple of 8 so that every XCD holds whole groups.
  const int rt = (int)((M + 15) / 16), rtp = rt == 1 ? 1 : (rt == 2 ? 2 : 4);
  const int64_t tiles = (N + 15) / 16, tiles8 = (tiles + 7) / 8 * 8;
  const int64_t groups = tiles8 < kSkTargetBlocks / rtp ? tiles8 : kSkTargetBlocks / rtp;
  const unsigned grid = (unsigned)(groups * rtp);
  constexpr bool kF16 = XT::kMagic2 == F16::kMagic2;  // bf16 with a scale goes to the direct kernel
  if (kF16 && s)
    hipLaunchKernelGGL((gemm_skinny_kernel<XT, BPW, ASYM, kF16>), dim3(grid), dim3(kSkWaves * 64), 0, stream,
                       static_cast<const uint16_t*>(X), s, static_cast<const uint8_t*>(packed),
                       static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), (int)M, (int)N,
                       (int)K, rtp, static_cast<uint16_t*>(Y));
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<XT, BPW, ASYM, false>), dim3(grid), dim3(kSkWaves * 64), 0, stream,
                       static_cast<const uint16_t*>(X), s, static_cast<const uint8_t*>(packed),
                       static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), (int)M, (int)N,
                       (int)K, rtp, static_cast<uint16_t*>(Y));
  return hipGetLastError();
}

template <class XT, bool ASYM>
hipError_t launch_xt(const void* X, const float* s, const void* packed, const void* scales, const void* zeros,
                     int64_t M, int64_t N, int64_t K, void* Y, hipStream_t stream) {
  switch (K / (kSkWaves * kSkBlock)) {
    case 1:
      return launch_bpw<XT, 1, ASYM>(X, s, packed, scales, zeros, M, N, K, Y, stream);
    case 2:
      return launch_bpw<XT, 2, ASYM>(X, s, packed, scales, zeros, M, N, K, Y, stream);
    case 4:
      return launch_bpw<XT, 4, ASYM>(X, s, packed, scales, zeros, M, N, K, Y, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

bool gemm_skinny_supported(int64_t M, int64_t N, int64_t K, int xdtype, bool act_scale, int bits, int group_size,
                           const void* scales, const void* zeros) {
  if (M < 2 || M > 64 || N < 1 || bits != 4 || group_size != kSkBlock) return false;
  if (K % (kSkWaves * kSkBlock) != 0) return false;
  const int64_t bpw = K / (kSkWaves * kSkBlock);
  if (bpw != 1 && bpw != 2 && bpw != kSkMaxBlocks) return false;
  if (M > 16 && K < 4096) return false;        // measured: the direct kernel is faster there
  if (xdtype != 0 && act_scale) return false;  // bf16 x / s needs the hi + lo pair: direct kernel
  // 32-bit scale / zero loads when the blocks per wave are even
  if (bpw > 1 && ((reinterpret_cast<uintptr_t>(scales) | reinterpret_cast<uintptr_t>(zeros)) & 3) != 0) return false;
  return true;
}

hipError_t launch_gemm_skinny(const void* X, int xdtype, const float* act_scale, const void* packed,
                              const void* scales, const void* zeros, int64_t M, int64_t N, int64_t K, bool asymmetric,
                              void* Y, hipStream_t stream) {
  if (xdtype == 0)
    return asymmetric ? launch_xt<F16, true>(X, act_scale, packed, scales, zeros, M, N, K, Y, stream)
                      : launch_xt<F16, false>(X, act_scale, packed, scales, zeros, M, N, K, Y, stream);
  return asymmetric ? launch_xt<BF16, true>(X, act_scale, packed, scales, zeros, M, N, K, Y, stream)
                    : launch_xt<BF16, false>(X, act_scale, packed, scales, zeros, M, N, K, Y, stream);
}

}  // namespace woq
