// Mid-M fused dequantize + GEMM (fp16 activations, 4-bit codes): a few dozen
// rows of X against a wide weight matrix, e.g. 64 tokens through a 70B-style
// MLP up-projection (K = 8192, N = 28672).
//
// At this M the product is still bound by streaming the packed weights
// ("CMU 11-868 L19-L20", section "Back to the question: where does the speed
// come from?"), so every code must be decoded once per launch, not once per
// 16-row slice of X, and the weights are dequantized inside the matmul
// ("Quantising Large Language Models ...", section "Weight-only vs
// weight-and-activation quantisation").
//
//   * A workgroup of 8 waves computes a 64 x 128 tile of Y.  Waves 0-3 take
//     the first half of the K blocks and waves 4-7 the second half; within a
//     half, wave w owns the 32 columns [32 (w % 4), + 32) for all 64 rows
//     (2 tiles of v_mfma_f32_32x32x16_f16, 32 fp32 accumulators per lane).
//     The two halves' partial sums meet in LDS at the end, so there is no
//     workspace and no second launch, and every column of codes is read and
//     decoded exactly once.
//   * Each half stages its X[m0:m0+64, k:k+64] block through its own
//     double-buffered LDS stage (144-byte pitch, conflict-free ds_read_b128);
//     one barrier per K block for the whole workgroup.
//   * B fragments never touch LDS: inside one 64-wide K block, lane half h
//     supplies K offsets [32 h, 32 h + 32) over the four MFMA steps (step s:
//     32 h + 8 s + j), A fragments are read with the same mapping, and a
//     lane's B data for the block is one 16-byte chunk of layout v2 whose
//     code word s holds the 8 offsets of step s.  Each pair is widened
//     exactly, (1024 + u) - (1024 + Z), and multiplied by S once.
//   * The tile's scales and zero points are staged in LDS once (K / G <= 64
//     groups), from 16-byte loads when both arrays are 16-byte aligned and
//     K / G % 8 == 0.
//
// bf16 X (XB) runs on the same fp16 MFMAs through the exact per-row
// power-of-two rescale of the register-B kernel: X is the pre-pass's fp16
// copy of fp16(x * f_m), and the output is multiplied by g_m = 1 / f_m
// before its one rounding to bf16 (g_m from the caller's workspace).
//
// MFMA operand slots (32x32x16): lane l supplies A[m = l%32][8(l/32)+j] and
// B[8(l/32)+j][n = l%32] and holds C[m = 8(v/4) + 4(l/32) + v%4][n = l%32]
// in accumulator v = 0..15.
#include "woq_device.h"
#include "woq_internal.h"

namespace woq {
namespace {

typedef float float16_t __attribute__((ext_vector_type(16)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = 64, kBN = 128, kBK = 64;
constexpr int kThreads = 512;                         // 8 waves: 4 column groups x 2 K halves
constexpr int kHalf = 256;                            // threads per K half
constexpr int kLD = kBK + 8;                          // A row pitch in halves (144 B)
constexpr int kStage = kBM * kLD;                     // halves per A stage
constexpr int kASegs = kBK / 8;                       // 16-byte segments per A row
constexpr int kAUnits = kBM * kASegs / kHalf;         // A segments per thread
constexpr int kARowStep = kHalf / kASegs;             // rows between a thread's segments
constexpr int kSZMaxGroups = 64;                      // K / G up to which S and Z are staged in LDS
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

// SZ: 0 = one 2-byte S / Z load per lane and block (K / G > 64); 1 = staged
// in LDS with 2-byte loads; 2 = staged from 16-byte loads.
// kRing: K steps of loads in flight.  4 for a single row of tiles (M <= 64:
// one workgroup per compute unit at most, so the ring's registers cost no
// occupancy), 3 otherwise (two workgroups per compute unit: 4 waves per SIMD,
// at most 128 VGPRs each; the launch bound's second value is waves per SIMD).
// With one workgroup per compute unit the loads go through buffer resources
// (a 32-bit offset per lane, the block offset in a scalar register: no
// address arithmetic per load) and the group index is one multiply per step
// instead of a division (c4 M = 64: 54.1 -> 51.5 us, same bits); at 128 VGPRs
// the same code spills, so the two-workgroup instance keeps pointer loads.
template <bool ASYM, bool SCALE, int SZ, int kRing, bool XB>
__global__ __launch_bounds__(kThreads, kRing == 3 ? 4 : 2) void gemm_mid_kernel(const uint16_t* __restrict__ X,
                                                               const float* __restrict__ s,
                                                               const uint8_t* __restrict__ packed,
                                                               const uint16_t* __restrict__ scales,
                                                               const uint16_t* __restrict__ zeros, int M, int N, int K,
                                                               int G, uint16_t* __restrict__ Y, int tiles_m,
                                                               int tiles_n, const float* __restrict__ rs) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * kStage];  // [K half][stage]
  constexpr bool SZL = SZ > 0;
  constexpr bool kLean = kRing == 4;
  __shared__ uint32_t szs[SZL ? kSZWords : 1];
  // XB: g_m of the tile's rows, read in the epilogue (staged here, so the
  // epilogue's 32 scalings per lane wait on LDS rather than on global loads
  // issued after the last MFMA)
  __shared__ float g_tile[XB ? kBM : 1];

  // Tiles in XCD-contiguous ranges, N tile fastest.
  const int T = tiles_m * tiles_n;
  const int per_xcd = (T + 7) / 8;
  const int tile = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (tile >= T) return;
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cg = wave & 3, kh = wave >> 2;  // column group and K half of this wave
  if constexpr (XB) {
    if (tid < kBM) {
      const int r = m0 + tid;
      g_tile[tid] = rs[M + (r < M ? r : M - 1)];
    }
  }
  const int htid = tid & (kHalf - 1);       // thread index within the K half
  const int fr = lane & 31, fh = lane >> 5;
  const int gpr = K / G;
  const int kblocks = K / kBK;
  const int kbh = (kblocks + 1) / 2;         // block steps per half; the second may compute one fewer
  const int kb_first = kh * kbh;
  const int nsteps = kblocks - kb_first < kbh ? kblocks - kb_first : kbh;  // blocks this half computes
  auto block_k = [&](int t) {                // K offset of this half's step t (clamped: reloads never used)
    const int b = kb_first + t;
    return (b < kblocks ? b : kblocks - 1) * kBK;
  };

  // A staging: thread t of a half owns segment t % 8 of rows t / 8 + 32 i.
  // Rows past M read row M - 1; their outputs are never stored.
  const int a_seg = htid % kASegs, a_r0 = htid / kASegs;
  const uint16_t* a_src[kAUnits];
  uint32_t a_off[kAUnits];  // kLean: byte offsets from X (2 M K < 2^31)
#pragma unroll
  for (int i = 0; i < kAUnits; ++i) {
    const int r = m0 + a_r0 + kARowStep * i;
    a_src[i] = X + (int64_t)(r < M ? r : M - 1) * K + 8 * a_seg;
    a_off[i] = 2u * (uint32_t)((r < M ? r : M - 1) * K + 8 * a_seg);
  }
  const __amdgpu_buffer_rsrc_t x_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X), 0, 2 * M * K, kBufferWord3);
  const uint32_t a_dst = (uint32_t)(a_r0 * kLD + 8 * a_seg);
  uint16_t* const my_stages = lds + 2 * kh * kStage;


  // B: column n0 + 32 cg + l%32 (columns past N read column N - 1, never
  // stored); this lane's chunk of the block starting at k is codes
  // [k + 32 h, k + 32 h + 32).
  int bc = n0 + 32 * cg + fr;
  bc = bc < N ? bc : N - 1;
  const uint8_t* b_src = packed + (int64_t)bc * (K / 2) + 16 * fh;
  const int64_t g_row = (int64_t)bc * gpr;
  const int64_t b_bytes = ((int64_t)N - n0) * (K / 2);  // kLean: the tile's columns onward
  const __amdgpu_buffer_rsrc_t b_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(packed + (int64_t)n0 * (K / 2)), 0,
                                        (int)(b_bytes < 0x7FFFFFFF ? b_bytes : 0x7FFFFFFF), kBufferWord3);
  const uint32_t b_off = (uint32_t)((bc - n0) * (K / 2) + 16 * fh);
  // Group of this lane's chunk of the block at kb, (kb + 32 h) / G: kLean
  // multiplies by ceil(2^32 / G), exact for K * G < 2^32 (checked on the host).
  const uint32_t gmag = (uint32_t)((0x100000000ull + (uint64_t)G - 1) / (uint64_t)G);
  auto group_of = [&](int kb) {
    if constexpr (kLean)
      return (int)__umulhi((uint32_t)(kb + 32 * fh), gmag);
    else
      return (kb + 32 * fh) / G;
  };

  // Scales and zero points of the tile: S | Z << 16 per (column, group),
  // pitch gpr + 1.
  const int szp = gpr + 1;
  constexpr int kSZChunks = kBN * kSZMaxGroups / 8 / kThreads;  // 16-byte chunks per thread and array
  u32x4_t szv_s[SZ == 2 ? kSZChunks : 1], szv_z[SZ == 2 ? kSZChunks : 1];
  const int sz_chunks = kBN * gpr / 8;
  if constexpr (SZ == 2) {
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
    const int64_t row0 = (int64_t)n0 * gpr, limit = (int64_t)N * gpr;
    for (int idx = tid; idx < kBN * gpr; idx += kThreads) {
      int64_t gi = row0 + idx;
      gi = gi < limit ? gi : limit - 1;
      const uint32_t sv = scales[gi], zv = ASYM ? zeros[gi] : 0u;
      const int c = idx / gpr;
      szs[c * szp + (idx - c * gpr)] = sv | (zv << 16);
    }
  }

  struct ARegs {
    u32x4_t a[kAUnits];
  };
  struct BRegs {
    u32x4_t w;
    uint16_t s16, z16;
  };
  auto load_a = [&](ARegs& R, int kb) {
#pragma unroll
    for (int i = 0; i < kAUnits; ++i) {
      if constexpr (kLean)
        R.a[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, (int)a_off[i], 2 * kb, 0));
      else
        R.a[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + kb);
    }
  };
  auto load_b = [&](BRegs& R, int kb) {
    if constexpr (kLean)
      R.w = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, (int)b_off, kb / 2, 0));
    else
      R.w = *reinterpret_cast<const u32x4_t*>(b_src + kb / 2);
    if constexpr (!SZL) {
      const int64_t gi = g_row + group_of(kb);
      R.s16 = scales[gi];
      R.z16 = ASYM ? zeros[gi] : (uint16_t)0;
    }
  };
  auto store_a = [&](const ARegs& R, int st, int kb) {
    uint16_t* base = my_stages + st * kStage;
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

  float16_t acc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;

  const uint32_t a_rd = (uint32_t)(fr * kLD + 32 * fh);
  const uint32_t magic = vgpr_const(0x64006400u);  // one v_and_or_b32 per pair
  // live == false (a step past this half's last block): the scale is 0, so
  // the step's MFMAs add exact zeros (X is finite) and the unrolled ring has
  // no branch.
  auto mma_block = [&](int st, const BRegs& R, int kb, bool live) {
    const uint16_t* base = my_stages + st * kStage;
    uint16_t s16, z16;
    if constexpr (SZL) {
      const uint32_t v = szs[(32 * cg + fr) * szp + group_of(kb)];
      s16 = (uint16_t)(v & 0xFFFFu);
      z16 = (uint16_t)(v >> 16);
    } else {
      s16 = R.s16;
      z16 = R.z16;
    }
    const float Z = ASYM ? half_bits_to_f32(z16) : 8.0f;
    const uint32_t zh = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(1024.0f + Z));
    const uint32_t zm = zh | (zh << 16), s2 = live ? (uint32_t)s16 | ((uint32_t)s16 << 16) : 0u;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4_t a[2], b;
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const u32x4_t*>(base + a_rd + 32 * kLD * i + 8 * ks);
      const uint32_t w = R.w[ks];
#pragma unroll
      for (int t = 0; t < 4; ++t) b[t] = dequant_pair(((w >> (4 * t)) & 0x000F000Fu) | magic, zm, s2);
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i] = mfma32(a[i], b, acc[i]);
    }
  };

  // Loads run kRing steps ahead in a register ring (slot r of the ring holds
  // step t with t % kRing == r; the loop is unrolled over the ring so every
  // slot index is a constant and no register is read across the back edge
  // less than a ring after its load): step t computes with B slot t % kRing,
  // moves X of step t + 1 into the other LDS stage, refills its own slot
  // with step t + kRing, and ends with the workgroup's one barrier per step.
  // Steps past a half's last block compute zeros; their loads are clamped
  // reloads.
  ARegs RA[kRing];
  BRegs RB[kRing];
#pragma unroll
  for (int r = 0; r < kRing; ++r) {
    load_a(RA[r], block_k(r));
    load_b(RB[r], block_k(r));
  }
  if constexpr (SZ == 2) {
    // chunk q holds entries 8q .. 8q + 7: one column c, groups g .. g + 7
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
  store_a(RA[0], 0, block_k(0));
  __syncthreads();
  for (int t0 = 0; t0 < kbh; t0 += kRing) {
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      const int t = t0 + r;
      mma_block(t & 1, RB[r], block_k(t), t < nsteps);
      store_a(RA[(r + 1) % kRing], (t + 1) & 1, block_k(t + 1));
      load_a(RA[r], block_k(t + kRing));
      load_b(RB[r], block_k(t + kRing));
      __syncthreads();
    }
  }

  // The second half hands its partial sums to the first through LDS (the
  // A stages are free after the last barrier).
  float* red = reinterpret_cast<float*>(lds);
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[((cg * 2 + i) * 16 + v) * 64 + lane] = acc[i][v];
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] += red[((cg * 2 + i) * 16 + v) * 64 + lane];

  // Accumulator (i, v): the 32 lanes of each half-wave hold 32 consecutive
  // columns of one row.
  const int row_base = m0 + 4 * fh;
  const int col = n0 + 32 * cg + fr;
  if (col >= N) return;
  uint16_t* __restrict__ yb = Y + (int64_t)row_base * N + col;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int dm = 32 * i + 8 * (v >> 2) + (v & 3);
      if constexpr (XB) {
        // undo the row scaling (g_m = 1 / f_m: exact), then one rounding to bf16
        if (row_base + dm < M) yb[(int64_t)dm * N] = BF16::from_f32(acc[i][v] * g_tile[4 * fh + dm]);
      } else {
        if (row_base + dm < M) yb[(int64_t)dm * N] = F16::from_f32(acc[i][v]);
      }
    }
}

template <bool ASYM, bool SCALE, int SZ, bool XB>
hipError_t launch_sz(const void* X, const float* s, const void* packed, const void* scales, const void* zeros,
                     int64_t M, int64_t N, int64_t K, int G, void* Y, const float* rs, hipStream_t stream) {
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kBN - 1) / kBN);
  const int T = tiles_m * tiles_n;
  const unsigned blocks = 8u * (unsigned)((T + 7) / 8);  // blockIdx.x % 8 is the XCD
  if (tiles_m == 1)
    hipLaunchKernelGGL((gemm_mid_kernel<ASYM, SCALE, SZ, 4, XB>), dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(X), s, static_cast<const uint8_t*>(packed),
                       static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), (int)M, (int)N,
                       (int)K, G, static_cast<uint16_t*>(Y), tiles_m, tiles_n, rs);
  else
    hipLaunchKernelGGL((gemm_mid_kernel<ASYM, SCALE, SZ, 3, XB>), dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(X), s, static_cast<const uint8_t*>(packed),
                       static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), (int)M, (int)N,
                       (int)K, G, static_cast<uint16_t*>(Y), tiles_m, tiles_n, rs);
  return hipGetLastError();
}

template <bool ASYM, bool SCALE, bool XB>
hipError_t launch_one(const void* X, const float* s, const void* packed, const void* scales, const void* zeros,
                      int64_t M, int64_t N, int64_t K, int G, void* Y, const float* rs, hipStream_t stream) {
  const int64_t gpr = K / G;
  if (gpr > kSZMaxGroups)
    return launch_sz<ASYM, SCALE, 0, XB>(X, s, packed, scales, zeros, M, N, K, G, Y, rs, stream);
  const bool aligned16 = (reinterpret_cast<uintptr_t>(scales) % 16 == 0) &&
                         (!ASYM || reinterpret_cast<uintptr_t>(zeros) % 16 == 0);
  if (gpr % 8 == 0 && aligned16)
    return launch_sz<ASYM, SCALE, 2, XB>(X, s, packed, scales, zeros, M, N, K, G, Y, rs, stream);
  return launch_sz<ASYM, SCALE, 1, XB>(X, s, packed, scales, zeros, M, N, K, G, Y, rs, stream);
}

template <bool XB>
hipError_t launch_xb(const void* X, const float* act_scale, const void* packed, const void* scales, const void* zeros,
                     int64_t M, int64_t N, int64_t K, int group_size, bool asymmetric, void* Y, const float* rs,
                     hipStream_t stream) {
  if (asymmetric)
    return act_scale
               ? launch_one<true, true, XB>(X, act_scale, packed, scales, zeros, M, N, K, group_size, Y, rs, stream)
               : launch_one<true, false, XB>(X, act_scale, packed, scales, zeros, M, N, K, group_size, Y, rs, stream);
  return act_scale
             ? launch_one<false, true, XB>(X, act_scale, packed, scales, zeros, M, N, K, group_size, Y, rs, stream)
             : launch_one<false, false, XB>(X, act_scale, packed, scales, zeros, M, N, K, group_size, Y, rs, stream);
}

}  // namespace

hipError_t launch_gemm_mid(const void* X, const float* act_scale, const void* packed, const void* scales,
                           const void* zeros, int64_t M, int64_t N, int64_t K, int group_size, bool asymmetric,
                           void* Y, hipStream_t stream) {
  return launch_xb<false>(X, act_scale, packed, scales, zeros, M, N, K, group_size, asymmetric, Y, nullptr, stream);
}

hipError_t launch_gemm_mid_rescaled_bf16(const void* X16, const void* packed, const void* scales, const void* zeros,
                                         int64_t M, int64_t N, int64_t K, int group_size, bool asymmetric, void* Y,
                                         const float* row_scales, hipStream_t stream) {
  return asymmetric ? launch_one<true, false, true>(X16, nullptr, packed, scales, zeros, M, N, K, group_size, Y,
                                                    row_scales, stream)
                    : launch_one<false, false, true>(X16, nullptr, packed, scales, zeros, M, N, K, group_size, Y,
                                                     row_scales, stream);
}

}  // namespace woq
