// Mid-M fused dequantize + GEMM for bf16 activations and 4-bit codes (33..127
// rows of X against a wide weight matrix), the bf16 counterpart of
// gemm_mid.hip with the same tiles and work split: 64 x 128 tiles, 8 waves,
// the K blocks split between two halves of the workgroup that meet in LDS,
// codes and X several K steps ahead in a register ring.
//
// The weights are never rounded.  bf16 has 8 significant bits, too few for
// w_hat = (u - Z) S itself, so the B operand is the exact bf16 value 128 + u
// (one v_and_or_b32 per code pair) and each group's partial sum is scaled in
// fp32 when the group ends:
//   acc += S * (sum_k x (128 + u) - (128 + Z) * sum_k x),
// the zero-point form of the dequantization ("CMU 11-868 L19-L20 Model
// Quantization", the absmax / zero-point code) folded into the sum, with the
// weights dequantized inside the matmul ("Quantising Large Language Models
// ...", section "Weight-only vs weight-and-activation quantisation").
//
// A group must not straddle a 64-wide K step, so the group size is a power of
// two of at least 64.  sum_k x per row and group is taken while X passes
// through LDS: the 8 threads that stage a row's 64 values of a step sum them
// with v_dot2 against ones and a DPP reduction; the last one keeps the running
// sum of the group and writes it to LDS at the group's last step (two buffers,
// alternating per group).  The MFMA waves read the 32 sums their accumulators
// need when the group ends.
//
// MFMA operand slots (32x32x16): lane l supplies A[m = l%32][8(l/32)+j] and
// B[8(l/32)+j][n = l%32] and holds C[m = 8(v/4) + 4(l/32) + v%4][n = l%32]
// in accumulator v = 0..15.  Inside one 64-wide K block, lane half h supplies
// the K offsets [32 h, 32 h + 32) over the four MFMA steps (step s:
// 32 h + 8 s + j); a lane's B data for the block is one 16-byte layout-v2 chunk.
#include "woq_device.h"
#include "woq_internal.h"

namespace woq {
namespace {

typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 64, kBN = 128, kBK = 64;
constexpr int kThreads = 512;                       // 8 waves: 4 column groups x 2 K halves
constexpr int kHalf = 256;                          // threads per K half
constexpr int kLD = kBK + 8;                        // A row pitch in halves (144 B)
constexpr int kStage = kBM * kLD;                   // halves per A stage
constexpr int kASegs = kBK / 8;                     // 16-byte segments per A row
constexpr int kAUnits = kBM * kASegs / kHalf;       // A segments per thread (2)
constexpr int kARowStep = kHalf / kASegs;           // rows between a thread's segments (32)
constexpr int kSZMaxGroups = 64;                    // K / G up to which S and Z are staged in LDS
constexpr int kSZWords = kBN * (kSZMaxGroups + 1);  // S | Z << 16 per (column, group), odd pitch

__device__ inline float16_t mfma32_bf16(u32x4_t a, u32x4_t b, float16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf168_t, a), __builtin_bit_cast(bf168_t, b), c, 0,
                                                 0, 0);
}

// v + the value of the lane the DPP control selects (0 where there is none).
template <int CTRL>
__device__ inline float add_dpp(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf,
                                                                   true));
}

// Sum over the 8 lanes 8r .. 8r + 7; lanes 8r + 4 .. 8r + 7 hold it.
__device__ inline float sum8(float v) {
  v = add_dpp<0xb1>(v);   // quad_perm [1,0,3,2]
  v = add_dpp<0x4e>(v);   // quad_perm [2,3,0,1]
  v = add_dpp<0x114>(v);  // row_shr:4
  return v;
}

// SZ: 0 = one 2-byte S / Z load per lane and block (K / G > 64); 1 = staged
// in LDS with 2-byte loads; 2 = staged from 16-byte loads.  kRing: K steps of
// loads in flight.
template <bool ASYM, int SZ, int kRing>
__global__ __launch_bounds__(kThreads, 1) void gemm_mid_bf16_kernel(const uint16_t* __restrict__ X,
                                                                   const uint8_t* __restrict__ packed,
                                                                   const uint16_t* __restrict__ scales,
                                                                   const uint16_t* __restrict__ zeros, int M, int N,
                                                                   int K, int G, uint16_t* __restrict__ Y,
                                                                   int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * kStage];  // [K half][stage]
  __shared__ __attribute__((aligned(16))) float xsum[2][2][kBM];     // [K half][group parity][row]
  constexpr bool SZL = SZ > 0;
  __shared__ uint32_t szs[SZL ? kSZWords : 1];

  const int T = tiles_m * tiles_n;
  const int per_xcd = (T + 7) / 8;
  const int tile = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (tile >= T) return;
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cg = wave & 3, kh = wave >> 2;
  const int htid = tid & (kHalf - 1);
  const int fr = lane & 31, fh = lane >> 5;
  const int gpr = K / G;
  const int gmask = G - 1, gshift = __builtin_ctz(G);  // G is a power of two
  const int kblocks = K / kBK;
  const int kbh = (kblocks + 1) / 2;
  const int kb_first = kh * kbh;
  const int nsteps = kblocks - kb_first < kbh ? kblocks - kb_first : kbh;
  auto block_k = [&](int t) {
    const int b = kb_first + t;
    return (b < kblocks ? b : kblocks - 1) * kBK;
  };
  // Step t of this half starts / ends a group (the half's own first and last
  // blocks count as both, so a group split between the halves is summed as
  // two parts with the same S and Z).
  auto group_first = [&](int t) { return t == 0 || ((kb_first + t) * kBK & gmask) == 0; };
  auto group_last = [&](int t) {
    return t < nsteps && (t == nsteps - 1 || (((kb_first + t + 1) * kBK) & gmask) == 0);
  };
  auto group_of = [&](int t) { return ((kb_first + t) * kBK) >> gshift; };

  // A staging: thread t of a half owns segment t % 8 of rows t / 8 + 32 i;
  // the 8 threads of a row are 8 consecutive lanes of one wave.
  const int a_seg = htid % kASegs, a_r0 = htid / kASegs;
  const uint16_t* a_src[kAUnits];
#pragma unroll
  for (int i = 0; i < kAUnits; ++i) {
    const int r = m0 + a_r0 + kARowStep * i;
    a_src[i] = X + (int64_t)(r < M ? r : M - 1) * K + 8 * a_seg;
  }
  const uint32_t a_dst = (uint32_t)(a_r0 * kLD + 8 * a_seg);
  uint16_t* const my_stages = lds + 2 * kh * kStage;

  int bc = n0 + 32 * cg + fr;
  bc = bc < N ? bc : N - 1;
  const uint8_t* b_src = packed + (int64_t)bc * (K / 2) + 16 * fh;
  const int64_t g_row = (int64_t)bc * gpr;

  const int szp = gpr + 1;
  constexpr int kSZChunks = kBN * kSZMaxGroups / 8 / kThreads;
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
    for (int i = 0; i < kAUnits; ++i) R.a[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + kb);
  };
  auto load_b = [&](BRegs& R, int kb) {
    R.w = *reinterpret_cast<const u32x4_t*>(b_src + kb / 2);
    if constexpr (!SZL) {
      const int64_t gi = g_row + (kb >> gshift);  // both lane halves: one group per 64-wide step
      R.s16 = scales[gi];
      R.z16 = ASYM ? zeros[gi] : (uint16_t)0;
    }
  };
  // X of this half's step t into stage st, and its rows' sums into the
  // group's running sums (lane 8r + 7 of each row's 8 threads keeps them).
  float xrun[kAUnits] = {0.0f, 0.0f};
  const uint32_t ones2 = 0x3F803F80u;  // bf16 pair (1, 1)
  auto store_a = [&](const ARegs& R, int st, int t) {
    uint16_t* base = my_stages + st * kStage;
#pragma unroll
    for (int i = 0; i < kAUnits; ++i) *reinterpret_cast<u32x4_t*>(base + a_dst + kARowStep * kLD * i) = R.a[i];
    if (t < nsteps) {  // uniform per half
      const bool first = group_first(t), last = group_last(t);
#pragma unroll
      for (int i = 0; i < kAUnits; ++i) {
        float v = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) v = BF16::dot2(R.a[i][e], ones2, v);
        v = sum8(v);
        xrun[i] = (first ? 0.0f : xrun[i]) + v;
        if (last && (lane & 7) == 7) xsum[kh][group_of(t) & 1][a_r0 + kARowStep * i] = xrun[i];
      }
    }
  };

  float16_t acc[2], part[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = part[i][v] = 0.0f;

  const uint32_t a_rd = (uint32_t)(fr * kLD + 32 * fh);
  const uint32_t magic = vgpr_const(0x43004300u);  // bf16 128: 128 + u in one v_and_or_b32 per pair
  // Step t: MFMAs into the group's partial sums; at the group's last step the
  // partials are scaled into acc and cleared.  Steps past the half's end run
  // on clamped reloads and leave partial sums that are never scaled, so the
  // unrolled ring has no branch around its MFMAs.
  auto mma_block = [&](int st, const BRegs& R, int t) {
    const uint16_t* base = my_stages + st * kStage;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4_t a[2], b;
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const u32x4_t*>(base + a_rd + 32 * kLD * i + 8 * ks);
      const uint32_t w = R.w[ks];
#pragma unroll
      for (int q = 0; q < 4; ++q) b[q] = ((w >> (4 * q)) & 0x000F000Fu) | magic;
#pragma unroll
      for (int i = 0; i < 2; ++i) part[i] = mfma32_bf16(a[i], b, part[i]);
    }
    if (group_last(t)) {
      uint16_t s16, z16;
      if constexpr (SZL) {
        const uint32_t v = szs[(32 * cg + fr) * szp + group_of(t)];
        s16 = (uint16_t)(v & 0xFFFFu);
        z16 = (uint16_t)(v >> 16);
      } else {
        s16 = R.s16;
        z16 = R.z16;
      }
      const float S = half_bits_to_f32(s16);
      const float mz = -(128.0f + (ASYM ? half_bits_to_f32(z16) : 8.0f));
      const float* xs = xsum[kh][group_of(t) & 1];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // accumulators v = 4q .. 4q + 3: rows 32 i + 8 q + 4 h + 0..3
          const float4_t x4 = *reinterpret_cast<const float4_t*>(xs + 32 * i + 8 * q + 4 * fh);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * q + e;
            acc[i][v] = __builtin_fmaf(S, __builtin_fmaf(mz, x4[e], part[i][v]), acc[i][v]);
            part[i][v] = 0.0f;
          }
        }
    }
  };

  ARegs RA[kRing];
  BRegs RB[kRing];
#pragma unroll
  for (int r = 0; r < kRing; ++r) {
    load_a(RA[r], block_k(r));
    load_b(RB[r], block_k(r));
  }
  if constexpr (SZ == 2) {
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
  store_a(RA[0], 0, 0);
  __syncthreads();
  for (int t0 = 0; t0 < kbh; t0 += kRing) {
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      const int t = t0 + r;
      mma_block(t & 1, RB[r], t);
      store_a(RA[(r + 1) % kRing], (t + 1) & 1, t + 1);
      load_a(RA[r], block_k(t + kRing));
      load_b(RB[r], block_k(t + kRing));
      __syncthreads();
    }
  }

  // The second half hands its sums to the first through LDS.
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

  const int row_base = m0 + 4 * fh;
  const int col = n0 + 32 * cg + fr;
  if (col >= N) return;
  uint16_t* __restrict__ yb = Y + (int64_t)row_base * N + col;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int dm = 32 * i + 8 * (v >> 2) + (v & 3);
      if (row_base + dm < M) yb[(int64_t)dm * N] = BF16::from_f32(acc[i][v]);
    }
}

template <bool ASYM, int SZ>
hipError_t launch_sz(const void* X, const void* packed, const void* scales, const void* zeros, int64_t M, int64_t N,
                     int64_t K, int G, void* Y, hipStream_t stream) {
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kBN - 1) / kBN);
  const int T = tiles_m * tiles_n;
  const unsigned blocks = 8u * (unsigned)((T + 7) / 8);  // blockIdx.x % 8 is the XCD
  if (tiles_m == 1)
    hipLaunchKernelGGL((gemm_mid_bf16_kernel<ASYM, SZ, 4>), dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(X), static_cast<const uint8_t*>(packed),
                       static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), (int)M, (int)N,
                       (int)K, G, static_cast<uint16_t*>(Y), tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((gemm_mid_bf16_kernel<ASYM, SZ, 3>), dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(X), static_cast<const uint8_t*>(packed),
                       static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), (int)M, (int)N,
                       (int)K, G, static_cast<uint16_t*>(Y), tiles_m, tiles_n);
  return hipGetLastError();
}

template <bool ASYM>
hipError_t launch_one(const void* X, const void* packed, const void* scales, const void* zeros, int64_t M, int64_t N,
                      int64_t K, int G, void* Y, hipStream_t stream) {
  const int64_t gpr = K / G;
  if (gpr > kSZMaxGroups) return launch_sz<ASYM, 0>(X, packed, scales, zeros, M, N, K, G, Y, stream);
  const bool aligned16 = (reinterpret_cast<uintptr_t>(scales) % 16 == 0) &&
                         (!ASYM || reinterpret_cast<uintptr_t>(zeros) % 16 == 0);
  if (gpr % 8 == 0 && aligned16) return launch_sz<ASYM, 2>(X, packed, scales, zeros, M, N, K, G, Y, stream);
  return launch_sz<ASYM, 1>(X, packed, scales, zeros, M, N, K, G, Y, stream);
}

}  // namespace

bool gemm_mid_bf16_supported(int64_t K, int group_size) {
  return K % 64 == 0 && group_size >= 64 && (group_size & (group_size - 1)) == 0;
}

hipError_t launch_gemm_mid_bf16(const void* X, const void* packed, const void* scales, const void* zeros, int64_t M,
                                int64_t N, int64_t K, int group_size, bool asymmetric, void* Y, hipStream_t stream) {
  return asymmetric ? launch_one<true>(X, packed, scales, zeros, M, N, K, group_size, Y, stream)
                    : launch_one<false>(X, packed, scales, zeros, M, N, K, group_size, Y, stream);
}

}  // namespace woq
