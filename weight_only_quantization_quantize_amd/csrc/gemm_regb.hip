// Large-M fused dequantize + GEMM with the weights decoded straight into
// matrix-core operand registers (fp16 activations, 4-bit codes).
//
// At large M the product is compute-bound ("CMU 11-868 L19-L20", section
// "Back to the question: where does the speed come from?"), so the weights
// only have to be dequantized once per use in a tile and fed to fp16 MFMA.
// This kernel spends LDS only on the activations:
//
//   * A workgroup of 4 waves computes a 128 x 256 tile of Y; wave w owns
//     columns [64 w, 64 w + 64) for all 128 rows (4 x 2 tiles of
//     v_mfma_f32_32x32x16_f16, 128 fp32 accumulators per lane), so no weight
//     is decoded twice.
//   * X[m0:m0+128, k:k+64] goes through a double-buffered LDS stage (one
//     barrier per 64-wide K block) and is read back as A fragments.
//   * B fragments never touch LDS.  Inside one 64-wide K block, lane half h of
//     a wave supplies K offsets [32 h, 32 h + 32) over the four 16-deep MFMA
//     steps (step s: offsets 32 h + 8 s .. + 8) instead of the usual 8 h + 16 s
//     ordering; A fragments are read with the same mapping, so each step still
//     sums every K offset exactly once.  With that order a lane's B data for
//     the whole block is one 16-byte chunk of layout v2 (32 codes of one
//     output column, inside one group since G % 32 == 0), and the code word s
//     of the chunk holds exactly the 8 K offsets of step s, as the pairs
//     (w >> 4t) & 0x000F000F, t = 0..3.
//   * Each pair is widened exactly, (1024 + u) - (1024 + Z) = u - Z in fp16,
//     and multiplied by S once: the weight is the same fp16 w_hat as in the
//     LDS-staged kernel.  The pair one nibble up is OR-ed into 0x5400 (64 + u)
//     and loses 64 + Z' = fp16(1024 + Z) - 960 instead, the same exact
//     difference, so a code word costs one shift instead of three.
//   * Codes and X are read through buffer resources over the tile's columns
//     and rows (a 32-bit offset per lane, the K block's offset in a scalar
//     register), and a lane's group index is one multiply by ceil(2^32 / G)
//     (exact for K * G < 2^32): no address or division arithmetic per block.  With an AWQ scale, A holds x * act_recip(s) rounded
//     once to fp16, also as there.
//
// The tile's scales and zero points (K / G <= 40 groups) are staged in LDS
// once, with contiguous loads: one 2-byte load per lane and block from 32
// different rows would cost as much as the codes themselves.  Loads for
// block k + 1 (X into registers and the codes) are issued at the top of block
// k, before block k's codes are first used, so they stay in flight through
// block k's MFMAs.  Tiles are assigned so
// that each of the 8 XCDs works on a contiguous range of the tile grid with
// the N tile index fastest.
//
// bf16 X (XB) runs on the same fp16 MFMAs: a pre-pass (xb_rescale_kernel)
// writes row m of X, times the power of two f_m that puts its largest |x|
// in [2^14, 2^15), as fp16 into the caller's workspace; a bf16 value has 8
// significant bits and fp16 has 11, so the conversion is exact down to 2^-31
// of the row's largest value (fp16 subnormals below that lose bits).  This
// kernel then runs on that fp16 copy exactly as for fp16 X, and its epilogue
// multiplies row m by g_m = 1 / f_m (a power of two) and writes bf16.
//
// MFMA operand slots (32x32x16): lane l supplies A[m = l%32][8(l/32)+j] and
// B[8(l/32)+j][n = l%32] (j = 0..7, here K offsets 32(l/32) + 8s + j) and
// holds C[m = 8(v/4) + 4(l/32) + v%4][n = l%32] in accumulator v = 0..15.
#include "woq_device.h"
#include "woq_internal.h"

namespace woq {
namespace {

typedef float float16_t __attribute__((ext_vector_type(16)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = 128, kBN = 256, kBK = 64;
constexpr int kGroupM = 8;  // M tiles per group of the XCD-local tile order

// Strides between the entries of a batched launch (elements of each array).
struct RegbBatch {
  int64_t s_stride, packed_stride, sz_stride, y_stride;
};
constexpr int kThreads = 256;
constexpr int kLD = kBK + 8;                          // A row pitch in halves (144 B: conflict-free ds_read_b128)
constexpr int kStage = kBM * kLD;                     // halves per A stage
constexpr int kASegs = kBK / 8;                       // 16-byte segments per A row
constexpr int kAUnits = kBM * kASegs / kThreads;      // A segments per thread
constexpr int kARowStep = kThreads / kASegs;          // rows between a thread's segments
constexpr int kSZMaxGroups = 40;                      // K / G up to which S and Z are staged in LDS
constexpr int kSZWords = kBN * (kSZMaxGroups + 1);    // S | Z << 16 per (column, group), odd pitch

__device__ inline float16_t mfma32(u32x4_t a, u32x4_t b, float16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0,
                                                0, 0);
}

// fp16 pair (u - Z) * S from the pair 1024 + u (codes OR-ed into 0x6400).
__device__ inline uint32_t dequant_pair(uint32_t magic_codes2, uint32_t zmagic2, uint32_t s2) {
  const h2_t p = __builtin_bit_cast(h2_t, magic_codes2);
  const h2_t d = p - __builtin_bit_cast(h2_t, zmagic2);
  return __builtin_bit_cast(uint32_t, d * __builtin_bit_cast(h2_t, s2));
}

// SZ: how the tile's scales and zero points reach the MFMA loop.
//   0: one 2-byte load per lane and block (K / G above the LDS limit);
//   1: staged in LDS once per tile with 2-byte loads;
//   2: staged in LDS once per tile from 16-byte loads, every load issued
//      before the first is waited for (arrays 16-byte aligned, K / G % 8 == 0).
// XB: X is the rescaled fp16 copy of bf16 X and Y is bf16; rs holds f_m
// (M floats) then g_m (M floats).
template <bool ASYM, bool SCALE, int SZ, bool XB>
__global__ __launch_bounds__(kThreads, 2) void gemm_regb_kernel(
    const uint16_t* __restrict__ X, const float* __restrict__ s, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int M, int N, int K, int G,
    uint16_t* __restrict__ Y, int tiles_m, int tiles_n, RegbBatch bt, const float* __restrict__ rs) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kStage];
  // Batch entry blockIdx.y (one entry unless batched): its own scale vector,
  // packed set and output over the same X.
  {
    const int64_t b = blockIdx.y;
    if (SCALE) s += b * bt.s_stride;
    packed += b * bt.packed_stride;
    scales += b * bt.sz_stride;
    if (ASYM) zeros += b * bt.sz_stride;
    Y += b * bt.y_stride;
  }
  constexpr bool SZL = SZ > 0;
  __shared__ __attribute__((aligned(16))) uint32_t szs[SZL ? kSZWords : 1];

  const int T = tiles_m * tiles_n;
  const int per_xcd = (T + 7) / 8;
  const int tile = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (tile >= T) return;
  // Within an XCD's range, tiles run down kGroupM M tiles before the next N
  // tile, so the tiles resident on one XCD share a few X row blocks and a few
  // code column blocks (c5: 8 x 11 tiles instead of 2 x 43).
  const int grp = tile / (kGroupM * tiles_n), first_m = grp * kGroupM;
  const int gsz = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  const int within = tile - grp * kGroupM * tiles_n;
  const int tm = first_m + within % gsz, tn = within / gsz;
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 31, fh = lane >> 5;
  const int gpr = K / G;
  const int kblocks = K / kBK;
  // (kb + 32 h) / G for the block at kb
  const uint32_t gmag = (uint32_t)((0x100000000ull + (uint64_t)G - 1) / (uint64_t)G);
  auto group_of = [&](int kb) { return (int)__umulhi((uint32_t)(kb + 32 * fh), gmag); };

  // A staging: thread t owns segment t % 8 of rows t / 8 + 32 i.  Rows past M
  // read row M - 1; their outputs are never stored.
  const int a_seg = tid % kASegs, a_r0 = tid / kASegs;
  uint32_t a_off[kAUnits];  // bytes from row m0 of X
#pragma unroll
  for (int i = 0; i < kAUnits; ++i) {
    const int r = m0 + a_r0 + kARowStep * i;
    a_off[i] = 2u * (uint32_t)(((r < M ? r : M - 1) - m0) * K + 8 * a_seg);
  }
  const int64_t x_bytes = 2 * ((int64_t)M - m0) * K;
  const __amdgpu_buffer_rsrc_t x_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X + (int64_t)m0 * K), 0,
                                        (int)(x_bytes < 0x7FFFFFFF ? x_bytes : 0x7FFFFFFF), kBufferWord3);
  const uint32_t a_dst = (uint32_t)(a_r0 * kLD + 8 * a_seg);
  // XB: g_m of the tile's rows, in LDS (registers are at the limit of two
  // workgroups per compute unit); read only after the loop's barriers.
  __shared__ float g_tile[XB ? kBM : 1];
  if constexpr (XB) {
    if (tid < kBM) {
      const int r = m0 + tid;
      g_tile[tid] = rs[M + (r < M ? r : M - 1)];
    }
  }

  // B: subtile j of this wave is column n0 + 64 wave + 32 j + l%32 (columns
  // past N read column N - 1, never stored); this lane's chunk of a block
  // starting at k is codes [k + 32 h, k + 32 h + 32).
  uint32_t b_off[2];  // bytes from column n0 of the codes
  int64_t g_row[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int c = n0 + 64 * wave + 32 * j + fr;
    c = c < N ? c : N - 1;
    b_off[j] = (uint32_t)((c - n0) * (K / 2) + 16 * fh);
    g_row[j] = (int64_t)c * gpr;
  }
  const int64_t b_bytes = ((int64_t)N - n0) * (K / 2);
  const __amdgpu_buffer_rsrc_t b_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(packed + (int64_t)n0 * (K / 2)), 0,
                                        (int)(b_bytes < 0x7FFFFFFF ? b_bytes : 0x7FFFFFFF), kBufferWord3);

  // SZL: the tile's scales and zero points, S | Z << 16 per (column, group)
  // with pitch gpr + 1 (conflict-free for 32 consecutive columns), loaded
  // once with contiguous loads; otherwise every block loads its own.  The
  // 2-byte form waits for each load before the next (one memory latency per
  // entry a thread stages); the 16-byte form has all of a thread's loads
  // (at most 5 per array) in flight at once.
  const int szp = gpr + 1;
  constexpr int kSZChunks = kBN * kSZMaxGroups / 8 / kThreads;  // 16-byte chunks per thread and array
  u32x4_t szv_s[SZ == 2 ? kSZChunks : 1], szv_z[SZ == 2 ? kSZChunks : 1];
  const int sz_chunks = kBN * gpr / 8;
  if constexpr (SZ == 2) {
    // The tile's slice of each [N, gpr] array is 256 gpr contiguous entries
    // from entry n0 gpr; chunks past the array end (columns past N, never
    // stored) read the last chunk.
    const int64_t c0 = (int64_t)n0 * gpr / 8, clast = (int64_t)N * gpr / 8 - 1;
#pragma unroll
    for (int t = 0; t < kSZChunks; ++t) {
      const int q = tid + kThreads * t;
      int64_t ci = c0 + (q < sz_chunks ? q : sz_chunks - 1);
      ci = ci < clast ? ci : clast;
      szv_s[t] = reinterpret_cast<const u32x4_t*>(scales)[ci];
      if (ASYM) szv_z[t] = reinterpret_cast<const u32x4_t*>(zeros)[ci];
    }
  }
  if constexpr (SZ == 1) {
    const int total = kBN * gpr, q = kThreads / gpr, r = kThreads % gpr;
    int c = tid / gpr, g = tid % gpr;
    const int64_t row0 = (int64_t)n0 * gpr;
    const int64_t limit = (int64_t)N * gpr;
    for (int idx = tid; idx < total; idx += kThreads) {
      int64_t gi = row0 + idx;
      gi = gi < limit ? gi : limit - 1;  // columns past N: any valid value (never stored)
      const uint32_t sv = scales[gi], zv = ASYM ? zeros[gi] : 0u;
      szs[c * szp + g] = sv | (zv << 16);
      c += q;
      g += r;
      if (g >= gpr) {
        g -= gpr;
        ++c;
      }
    }
  }

  struct ARegs {
    u32x4_t a[kAUnits];
  };
  struct BRegs {
    u32x4_t w[2];
    uint16_t s16[2], z16[2];
  };
  auto load_a = [&](ARegs& R, int kb) {
#pragma unroll
    for (int i = 0; i < kAUnits; ++i)
      R.a[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, (int)a_off[i], 2 * kb, 0));
  };
  auto load_b = [&](BRegs& R, int kb) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      R.w[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, (int)b_off[j], kb / 2, 0));
      if constexpr (!SZL) {
        const int64_t gi = g_row[j] + group_of(kb);
        R.s16[j] = scales[gi];
        R.z16[j] = ASYM ? zeros[gi] : (uint16_t)0;
      }
    }
  };
  auto store_a = [&](const ARegs& R, int st, int kb) {
    uint16_t* base = lds + st * kStage;
    float inv[8];
    if constexpr (SCALE) {
      const float4_t s0 = *reinterpret_cast<const float4_t*>(s + kb + 8 * a_seg);
      const float4_t s1 = *reinterpret_cast<const float4_t*>(s + kb + 8 * a_seg + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        inv[e] = act_recip(s0[e]);
        inv[e + 4] = act_recip(s1[e]);
      }
    }
#pragma unroll
    for (int i = 0; i < kAUnits; ++i) {
      u32x4_t v = R.a[i];
      if constexpr (SCALE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = F16::to_f32((uint16_t)(v[e] & 0xFFFFu)) * inv[2 * e];
          const float x1 = F16::to_f32((uint16_t)(v[e] >> 16)) * inv[2 * e + 1];
          v[e] = (uint32_t)F16::from_f32(x0) | ((uint32_t)F16::from_f32(x1) << 16);
        }
      }
      *reinterpret_cast<u32x4_t*>(base + a_dst + kARowStep * kLD * i) = v;
    }
  };

  float16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const uint32_t a_rd = (uint32_t)(fr * kLD + 32 * fh);
  const uint32_t magic = vgpr_const(0x64006400u);    // 1024 + u: one v_and_or_b32 per pair
  const uint32_t magic64 = vgpr_const(0x54005400u);  // 64 + u, the pair one nibble up
  const float zsym = 8.0f;
  auto mma_block = [&](int st, const BRegs& R, int kb) {
    const uint16_t* base = lds + st * kStage;
    uint32_t zm[2], zm64[2], s2[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint16_t s16, z16;
      if constexpr (SZL) {
        const uint32_t v = szs[(64 * wave + 32 * j + fr) * szp + group_of(kb)];
        s16 = (uint16_t)(v & 0xFFFFu);
        z16 = (uint16_t)(v >> 16);
      } else {
        s16 = R.s16[j];
        z16 = R.z16[j];
      }
      const float Z = ASYM ? half_bits_to_f32(z16) : zsym;
      const uint32_t zh = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(1024.0f + Z));
      zm[j] = zh | (zh << 16);
      zm64[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, zm[j]) - (h2_t){(_Float16)960.0f, (_Float16)960.0f});
      s2[j] = (uint32_t)s16 | ((uint32_t)s16 << 16);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4_t a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const u32x4_t*>(base + a_rd + 32 * kLD * i + 8 * ks);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t w = R.w[j][ks], w8 = w >> 8;
        b[j][0] = dequant_pair((w & 0x000F000Fu) | magic, zm[j], s2[j]);
        b[j][1] = dequant_pair((w & 0x00F000F0u) | magic64, zm64[j], s2[j]);
        b[j][2] = dequant_pair((w8 & 0x000F000Fu) | magic, zm[j], s2[j]);
        b[j][3] = dequant_pair((w8 & 0x00F000F0u) | magic64, zm64[j], s2[j]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    }
  };

  // Block kt: loads for block kt + 1 first (clamped to the last block at the
  // end: reloads never used), then block kt's MFMAs with its codes, then X of
  // block kt + 1 into the other LDS stage; one barrier per block.
  const int last = kblocks - 1;
  ARegs RA;
  BRegs RB, RN;
  load_a(RA, 0);
  load_b(RB, 0);
  if constexpr (SZ == 2) {
    // chunk q holds entries 8q .. 8q + 7 of the slice: one column c, groups
    // g .. g + 7 (gpr % 8 == 0)
#pragma unroll
    for (int t = 0; t < kSZChunks; ++t) {
      const int q = tid + kThreads * t;
      if (q < sz_chunks) {
        const int e0 = 8 * q, c = e0 / gpr, g = e0 - c * gpr;
        uint32_t* dst = szs + c * szp + g;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t sv = szv_s[t][e], zv = ASYM ? szv_z[t][e] : 0u;
          dst[2 * e] = (sv & 0xFFFFu) | (zv << 16);
          dst[2 * e + 1] = (sv >> 16) | (zv & 0xFFFF0000u);
        }
      }
    }
  }
  store_a(RA, 0, 0);
  __syncthreads();
  for (int kt = 0; kt < kblocks; ++kt) {
    const int nxt = kt + 1 < kblocks ? kt + 1 : last;
    load_a(RA, nxt * kBK);
    load_b(RN, nxt * kBK);
    // keep the loads ahead of the MFMAs (the scheduler would otherwise sink
    // them next to their first use)
    __builtin_amdgcn_sched_barrier(0);
    mma_block(kt & 1, RB, kt * kBK);
    store_a(RA, (kt + 1) & 1, nxt * kBK);
    RB = RN;
    __syncthreads();
  }

  // XB: the accumulators hold the product of the rescaled rows; row m's
  // output is bf16(acc) * g_m with g_m = 1 / f_m a power of two, so the
  // multiply after the rounding is exact (bf16 has fp32's exponent range)
  // and bf16(acc) * g_m = bf16(acc * g_m).  Applying it to the 16-bit
  // values keeps the 128 accumulators free of a second live copy.
  auto unscale = [&](uint16_t b, int row) -> uint16_t {
    return BF16::from_f32(BF16::to_f32(b) * g_tile[row]);
  };
  auto out16 = [](float v) -> uint16_t { return XB ? BF16::from_f32(v) : F16::from_f32(v); };

  // Epilogue, full tiles with N % 8 == 0 and the scales staged in LDS (both
  // LDS arrays are free after the loop's last barrier): each wave writes its
  // 128 x 64 fp16 block into a region of its own (pitch 72 halves) and stores
  // it back as 16-byte row segments, 16 stores per lane instead of 128.  The
  // region is the wave's alone and a wave's LDS operations complete in
  // order, so a wavefront-scope fence stands in for a barrier.
  if constexpr (SZL) {
    if (m0 + kBM <= M && n0 + kBN <= N && N % 8 == 0) {
      constexpr int kOP = 72;
      uint16_t* region = wave < 2 ? lds + wave * (kBM * kOP)
                                  : reinterpret_cast<uint16_t*>(szs) + (wave - 2) * (kBM * kOP);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            region[(32 * i + 8 * (v >> 2) + 4 * fh + (v & 3)) * kOP + 32 * j + fr] = out16(acc[i][j][v]);
      // the lanes of this wave read what other lanes wrote: keep the reads
      // after the writes (a wavefront-scope fence; LDS order does the rest)
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      const int ch = lane & 7;
      uint16_t* __restrict__ ybase = Y + (int64_t)m0 * N + n0 + 64 * wave + 8 * ch;
#pragma unroll
      for (int it = 0; it < kBM / 8; ++it) {
        const int row = 8 * it + (lane >> 3);
        u32x4_t v = *reinterpret_cast<const u32x4_t*>(region + row * kOP + 8 * ch);
        if constexpr (XB) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = (uint32_t)unscale((uint16_t)(v[e] & 0xFFFFu), row) | ((uint32_t)unscale((uint16_t)(v[e] >> 16), row) << 16);
        }
        *reinterpret_cast<u32x4_t*>(ybase + (int64_t)row * N) = v;
      }
      return;
    }
  }
  // Otherwise: for accumulator (i, j, v) the 32 lanes of each half-wave hold
  // 32 consecutive columns of one row; one 2-byte store per output.
  const int row_base = m0 + 4 * fh;
  const int col_base = n0 + 64 * wave + fr;
  uint16_t* __restrict__ yb = Y + (int64_t)row_base * N + col_base;
  if (m0 + kBM <= M && n0 + kBN <= N) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (XB) asm volatile("" ::: "memory");  // keep each group's g_tile reads in place
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int dm = 32 * i + 8 * (v >> 2) + (v & 3);
        uint16_t* __restrict__ yr = yb + (int64_t)dm * N;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint16_t o = out16(acc[i][j][v]);
          if constexpr (XB) o = unscale(o, 4 * fh + dm);
          yr[32 * j] = o;
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (XB) asm volatile("" ::: "memory");  // keep each group's g_tile reads in place
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int dm = 32 * i + 8 * (v >> 2) + (v & 3);
        if (row_base + dm >= M) continue;
        uint16_t* __restrict__ yr = yb + (int64_t)dm * N;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (col_base + 32 * j < N) {
            uint16_t o = out16(acc[i][j][v]);
            if constexpr (XB) o = unscale(o, 4 * fh + dm);
            yr[32 * j] = o;
          }
      }
    }
  }
}

template <bool ASYM, bool SCALE, int SZ, bool XB>
hipError_t launch_sz(const void* X, const float* s, const void* packed, const void* scales, const void* zeros,
                     int64_t M, int64_t N, int64_t K, int G, void* Y, int batch, RegbBatch bt, const float* rs,
                     hipStream_t stream) {
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kBN - 1) / kBN);
  const int T = tiles_m * tiles_n;
  // a multiple of 8, so that blockIdx.x % 8 is the XCD also in a batched grid
  const unsigned blocks = 8u * (unsigned)((T + 7) / 8);
  hipLaunchKernelGGL((gemm_regb_kernel<ASYM, SCALE, SZ, XB>), dim3(blocks, (unsigned)batch), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(X), s, static_cast<const uint8_t*>(packed),
                     static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), (int)M, (int)N, (int)K,
                     G, static_cast<uint16_t*>(Y), tiles_m, tiles_n, bt, rs);
  return hipGetLastError();
}

template <bool ASYM, bool SCALE, bool XB>
hipError_t launch_one(const void* X, const float* s, const void* packed, const void* scales, const void* zeros,
                      int64_t M, int64_t N, int64_t K, int G, void* Y, int batch, RegbBatch bt, const float* rs,
                      hipStream_t stream) {
  const int64_t gpr = K / G;
  if (gpr > kSZMaxGroups)
    return launch_sz<ASYM, SCALE, 0, XB>(X, s, packed, scales, zeros, M, N, K, G, Y, batch, bt, rs, stream);
  const bool aligned16 = (reinterpret_cast<uintptr_t>(scales) % 16 == 0) &&
                         (!ASYM || reinterpret_cast<uintptr_t>(zeros) % 16 == 0) && bt.sz_stride % 8 == 0;
  if (gpr % 8 == 0 && aligned16)
    return launch_sz<ASYM, SCALE, 2, XB>(X, s, packed, scales, zeros, M, N, K, G, Y, batch, bt, rs, stream);
  return launch_sz<ASYM, SCALE, 1, XB>(X, s, packed, scales, zeros, M, N, K, G, Y, batch, bt, rs, stream);
}

template <bool XB = false>
hipError_t launch_any(const void* X, const float* act_scale, const void* packed, const void* scales,
                      const void* zeros, int64_t M, int64_t N, int64_t K, int G, bool asymmetric, void* Y, int batch,
                      RegbBatch bt, const float* rs, hipStream_t stream) {
  if (asymmetric)
    return act_scale
               ? launch_one<true, true, XB>(X, act_scale, packed, scales, zeros, M, N, K, G, Y, batch, bt, rs, stream)
               : launch_one<true, false, XB>(X, act_scale, packed, scales, zeros, M, N, K, G, Y, batch, bt, rs, stream);
  return act_scale
             ? launch_one<false, true, XB>(X, act_scale, packed, scales, zeros, M, N, K, G, Y, batch, bt, rs, stream)
             : launch_one<false, false, XB>(X, act_scale, packed, scales, zeros, M, N, K, G, Y, batch, bt, rs, stream);
}

}  // namespace

hipError_t launch_gemm_regb(const void* X, const float* act_scale, const void* packed, const void* scales,
                            const void* zeros, int64_t M, int64_t N, int64_t K, int group_size, bool asymmetric,
                            void* Y, hipStream_t stream) {
  return launch_any<false>(X, act_scale, packed, scales, zeros, M, N, K, group_size, asymmetric, Y, 1,
                           RegbBatch{0, 0, 0, 0}, nullptr, stream);
}

hipError_t launch_gemm_regb_bf16(const void* X16, const void* packed, const void* scales, const void* zeros,
                                 int64_t M, int64_t N, int64_t K, int group_size, bool asymmetric, void* Y,
                                 const float* row_scales, hipStream_t stream) {
  const RegbBatch one{0, 0, 0, 0};
  return asymmetric ? launch_one<true, false, true>(X16, nullptr, packed, scales, zeros, M, N, K, group_size, Y, 1,
                                                    one, row_scales, stream)
                    : launch_one<false, false, true>(X16, nullptr, packed, scales, zeros, M, N, K, group_size, Y, 1,
                                                     one, row_scales, stream);
}

hipError_t launch_gemm_regb_batched(const void* X, const float* act_scale, int64_t s_stride, const void* packed,
                                    int64_t packed_stride, const void* scales, const void* zeros, int64_t sz_stride,
                                    int64_t M, int64_t N, int64_t K, int group_size, bool asymmetric, void* Y,
                                    int64_t y_stride, int batch, hipStream_t stream) {
  return launch_any<false>(X, act_scale, packed, scales, zeros, M, N, K, group_size, asymmetric, Y, batch,
                           RegbBatch{s_stride, packed_stride, sz_stride, y_stride}, nullptr, stream);
}

}  // namespace woq
