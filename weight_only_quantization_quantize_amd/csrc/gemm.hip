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
// Direct-decode kernel (this file): a workgroup owns a tile of 16*MT rows of
// X and 4 * 16*NT columns of W, and splits K between NS slices of 4 waves
// (their partial sums meet in LDS at the end).  Per K-block of KB (32, 64 or
// 128, never crossing a group):
//  * X[m0:m0+16MT, kb:kb+KB] is staged through LDS once for a slice's 4 waves
//    (divided by the AWQ scale and rounded when one is given);
//  * every lane loads the codes of its own B fragment straight from HBM (one
//    16-byte load per column tile for KB = 128), turns each code into the
//    16-bit float MAGIC + u (exact, one v_and_or_b32 per pair) and issues
//    KB/32 MFMAs per (mt, nt), plus one per mt against an all-ones fragment
//    that sums x over the group in the same layout;
//  * at the end of a group the fp32 partial sums are corrected and scaled,
//    acc += S (part - (MAGIC + Z) * sum x), so the only roundings are the
//    MFMA's fp32 accumulation and the final conversion of Y.
// Codes and X travel a few blocks ahead in register rings; the scales and
// zero points of the workgroup's columns are staged in LDS once.
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

// B fragment (8 consecutive K of one column) for MFMA q of the K-block;
// magic2 = MAGIC in both halves, held in a VGPR (one v_and_or_b32 per pair).
template <int BITS, int KB, class XT>
__device__ inline u32x4_t b_fragment(const BCodes<BITS, KB>& b, int q, int t0, uint32_t magic2) {
  u32x4_t f;
  if (BITS == 4) {
#pragma unroll
    for (int t = 0; t < 4; ++t) f[t] = pair4(b.w[q], t, magic2);
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) f[t] = pair3(b.w[0], b.w[1], b.w[2], t0 + 4 * q + t, magic2);
  }
  return f;
}

// Codes of one K-block for one column tile, with the block's scale and zero
// point (a K-block never crosses a group).
template <int BITS, int KB>
struct BBlock {
  BCodes<BITS, KB> c;
  uint16_t s16, z16;
};

// Scale / zero entries a workgroup can hold in LDS (per array).
constexpr int kSZLds = 8192;

// NS: K slices per workgroup.  The workgroup is NS groups of 4 waves; slice
// q runs the K-blocks [q bps, (q + 1) bps) of the same BN columns, and the NS
// partial results are summed through LDS at the end.  Small M has little
// work per column, so splitting K is what gives each CU enough waves (and
// loads in flight) to keep HBM busy.
template <int BITS, bool ASYM, class XT, int MT, int NT, int KB, bool SCALE, int P, bool SZL, int NS>
__global__ __launch_bounds__(kThreads * NS) void gemm_direct_kernel(
    const uint16_t* __restrict__ X, const float* __restrict__ s, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int M, int N, int K, int G,
    uint16_t* __restrict__ Y) {
  constexpr int BM = 16 * MT;
  constexpr int BN = 4 * 16 * NT;
  constexpr int XP = KB + 8;   // LDS row pitch in halves (16 B pad against bank conflicts)
  constexpr int SEG = KB / 8;  // 16-byte segments per staged row
  constexpr int UNITS = BM * SEG;
  constexpr int XU = (UNITS + kThreads - 1) / kThreads;  // X segments per thread of a slice
  // bf16 with an AWQ scale: x / s is staged as a bf16 pair hi + lo (about 16
  // significant bits) and each MFMA is issued for both halves.
  constexpr bool kSplitX = SCALE && XT::kMagic2 == BF16::kMagic2;
  // Two X stages (one barrier per K-block); the codes and X are loaded P
  // blocks ahead into register rings.
  __shared__ __attribute__((aligned(16))) uint16_t xs[NS][2][BM * XP];
  __shared__ __attribute__((aligned(16))) uint16_t xl[NS][2][kSplitX ? BM * XP : 8];
  // after the K loop the slices' partial results go to the X stages when they
  // fit there, else to an array of their own
  constexpr int kRed = NS > 1 ? NS * kThreads * 4 * MT * NT : 0;
  constexpr bool kRedInX = kRed * 4 <= (int)sizeof(xs);
  __shared__ float red_own[kRedInX || kRed == 0 ? 1 : kRed];
  float* const red = kRedInX ? reinterpret_cast<float*>(&xs[0][0][0]) : red_own;
  // SZL: the scales (and zero points) of this workgroup's BN columns, all
  // groups, staged once (they are one contiguous run of each [N, K/G] array);
  // otherwise each K-block's pair rides in the code ring.
  __shared__ uint16_t s_lds[SZL ? kSZLds : 1], z_lds[SZL && ASYM ? kSZLds : 1];

  // wave-uniform indices live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3), lane = threadIdx.x & 63;
  const int slice = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8), stid = threadIdx.x & (kThreads - 1);
  const int lr = lane & 15, lg = lane >> 4;
  const int m0 = blockIdx.y * BM;
  const int nw = blockIdx.x * BN + wave * 16 * NT;
  const int gpr = K / G;
  const int nblk = K / KB;
  // this slice's K-blocks (slice boundaries fall on group boundaries)
  const int gstep = G / KB > 1 ? G / KB : 1;
  const int bps = ((nblk + NS - 1) / NS + gstep - 1) / gstep * gstep;
  const int first = slice * bps;
  const int count = nblk - first < bps ? (nblk - first > 0 ? nblk - first : 0) : bps;
  const int lastb = count > 0 ? first + count - 1 : nblk - 1;  // clamp target for loads
  const float zsym = (float)(1 << (BITS - 1));
  const uint32_t ones2 = XT::kMagic2 == F16::kMagic2 ? 0x3C003C00u : 0x3F803F80u;

  // This lane's columns (past N: column N - 1, results never stored), as
  // pointers to its codes of K-block 0.
  int col[NT];
  const uint8_t* cptr[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = nw + 16 * nt + lr;
    col[nt] = n < N ? n : N - 1;
    cptr[nt] = packed + (int64_t)col[nt] * (K / 8 * BITS) +
               (BITS == 4 ? lg * (KB / 8) : (lg * (KB / 4) / 32) * 12);
  }
  auto load_block = [&](BBlock<BITS, KB> (&b)[NT], int blk) {
    const int kb = blk * KB;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint8_t* p = cptr[nt] + (BITS == 4 ? kb / 2 : (kb / 32) * 12);
      if constexpr (BITS == 4) {
        if constexpr (KB == 128) {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
          for (int j = 0; j < 4; ++j) b[nt].c.w[j] = v[j];
        } else if constexpr (KB == 64) {
          const uint2 v = *reinterpret_cast<const uint2*>(p);
          b[nt].c.w[0] = v.x;
          b[nt].c.w[1] = v.y;
        } else {
          b[nt].c.w[0] = *reinterpret_cast<const uint32_t*>(p);
        }
      } else {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
        b[nt].c.w[0] = q[0];
        b[nt].c.w[1] = q[1];
        b[nt].c.w[2] = q[2];
      }
      if constexpr (!SZL) {
        const int64_t gi = (int64_t)col[nt] * gpr + kb / G;
        b[nt].s16 = scales[gi];
        b[nt].z16 = ASYM ? zeros[gi] : (uint16_t)0;
      }
    }
  };
  if constexpr (SZL) {
    const int n_base = blockIdx.x * BN;
    const int cnt = BN * gpr;
    for (int i = threadIdx.x; i < cnt; i += kThreads * NS) {
      const int c = i / gpr;
      const int64_t gi = (int64_t)(n_base + c < N ? n_base + c : N - 1) * gpr + (i - c * gpr);
      s_lds[i] = scales[gi];
      if (ASYM) z_lds[i] = zeros[gi];
    }
  }

  // X staging: thread t owns segments t + 256 u (row it / SEG, segment it %
  // SEG); rows past M read row M - 1 (their outputs are never stored).
  struct XRegs {
    u32x4_t v[XU];
  };
  const uint16_t* xptr[XU];
#pragma unroll
  for (int u = 0; u < XU; ++u) {
    const int it = stid + kThreads * u;
    const int m = (it < UNITS ? it : UNITS - 1) / SEG, seg = it % SEG;
    const int row = m0 + m < M ? m0 + m : M - 1;
    xptr[u] = X + (int64_t)row * K + 8 * seg;
  }
  auto load_x = [&](XRegs& xr, int blk) {
#pragma unroll
    for (int u = 0; u < XU; ++u) xr.v[u] = *reinterpret_cast<const u32x4_t*>(xptr[u] + blk * KB);
  };
  auto store_x = [&](const XRegs& xr, int st, int blk) {
    const int kb = blk * KB;
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int it = stid + kThreads * u;
      if (UNITS % kThreads != 0 && it >= UNITS) break;
      const int m = it / SEG, seg = it - m * SEG;
      u32x4_t v = xr.v[u], vl = u32x4_t{0u, 0u, 0u, 0u};
      if (SCALE) {
        const float4_t s0 = *reinterpret_cast<const float4_t*>(s + kb + 8 * seg);
        const float4_t s1 = *reinterpret_cast<const float4_t*>(s + kb + 8 * seg + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float d0 = e < 2 ? s0[2 * e] : s1[2 * e - 4];
          const float d1 = e < 2 ? s0[2 * e + 1] : s1[2 * e - 3];
          const float a0 = XT::to_f32((uint16_t)(v[e] & 0xFFFFu)) * act_recip(d0);
          const float a1 = XT::to_f32((uint16_t)(v[e] >> 16)) * act_recip(d1);
          const uint16_t h0 = XT::from_f32(a0), h1 = XT::from_f32(a1);
          v[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
          if (kSplitX)
            vl[e] = (uint32_t)XT::from_f32(a0 - XT::to_f32(h0)) | ((uint32_t)XT::from_f32(a1 - XT::to_f32(h1)) << 16);
        }
      }
      *reinterpret_cast<u32x4_t*>(&xs[slice][st][m * XP + 8 * seg]) = v;
      if (kSplitX) *reinterpret_cast<u32x4_t*>(&xl[slice][st][m * XP + 8 * seg]) = vl;
    }
  };

  // part: sum over the group of x (MAGIC + u); xg: sum of x over the group,
  // from an MFMA against an all-ones B fragment (same C layout as part).
  float4_t acc[MT][NT], part[MT][NT], xg[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc[mt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
      part[mt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
    xg[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
  const u32x4_t ones_frag = u32x4_t{ones2, ones2, ones2, ones2};

  const int t0 = BITS == 3 ? (((lg * (KB / 4)) & 31) >> 1) : 0;
  const uint32_t magic2 = vgpr_const(XT::kMagic2);
  int szrow[NT];  // this lane's row in the staged scales / zeros
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) szrow[nt] = (wave * 16 * NT + 16 * nt + lr) * gpr;
  auto compute = [&](const BBlock<BITS, KB> (&b)[NT], int st, int blk) {
#pragma unroll
    for (int q = 0; q < KB / 32; ++q) {
      u32x4_t a[MT], al[kSplitX ? MT : 1];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        a[mt] = *reinterpret_cast<const u32x4_t*>(&xs[slice][st][(16 * mt + lr) * XP + lg * (KB / 4) + 8 * q]);
        xg[mt] = XT::mfma16x16x32(a[mt], ones_frag, xg[mt]);
        if constexpr (kSplitX) {
          al[mt] = *reinterpret_cast<const u32x4_t*>(&xl[slice][st][(16 * mt + lr) * XP + lg * (KB / 4) + 8 * q]);
          xg[mt] = XT::mfma16x16x32(al[mt], ones_frag, xg[mt]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const u32x4_t bf = b_fragment<BITS, KB, XT>(b[nt].c, q, t0, magic2);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          part[mt][nt] = XT::mfma16x16x32(a[mt], bf, part[mt][nt]);
          if constexpr (kSplitX) part[mt][nt] = XT::mfma16x16x32(al[mt], bf, part[mt][nt]);
        }
      }
    }
    if (((blk + 1) * KB) % G == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float S, Z = zsym;
        if constexpr (SZL) {
          const int li = szrow[nt] + (blk * KB) / G;
          S = half_bits_to_f32(s_lds[li]);
          if (ASYM) Z = half_bits_to_f32(z_lds[li]);
        } else {
          S = half_bits_to_f32(b[nt].s16);
          if (ASYM) Z = half_bits_to_f32(b[nt].z16);
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
      for (int mt = 0; mt < MT; ++mt) xg[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
  };

  // Two rings of P blocks: ring A holds the codes of the slice's blocks
  // s P .. s P + P - 1 (and the X of the block after each), ring B those of
  // the next P blocks.  A loop iteration runs super-blocks s (ring A) and
  // s + 1 (ring B); ring B is refilled after the first step of A, ring A after
  // the first step of B, so every load has about P steps to arrive, and the
  // only registers read across the loop back edge (ring A at the top) were
  // loaded a whole super-block earlier.  Block indices past the slice's end
  // are clamped (reloads whose results are never used), which keeps every
  // load in bounds.  Every wave runs the same bps steps (one barrier each).
  auto clampb = [&](int lb) { return first + lb < lastb ? first + lb : lastb; };
  BBlock<BITS, KB> ra[P][NT], rb[P][NT];
  XRegs xa[P], xb[P];
  auto fill = [&](BBlock<BITS, KB> (&r)[P][NT], XRegs (&x)[P], int lb0) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      load_block(r[j], clampb(lb0 + j));
      load_x(x[j], clampb(lb0 + j + 1));
    }
  };
  auto run = [&](const BBlock<BITS, KB> (&r)[NT], const XRegs& x, int lb) {
    if (lb < bps) {  // uniform across the workgroup
      if (lb < count) {  // uniform across the slice
        const int st = lb & 1;
        compute(r, st, first + lb);
        store_x(x, st ^ 1, clampb(lb + 1));
      }
      __syncthreads();
    }
  };
  {
    XRegs x0;
    load_x(x0, clampb(0));
    fill(ra, xa, 0);
    store_x(x0, 0, clampb(0));
  }
  __syncthreads();
  for (int base = 0; base < bps; base += 2 * P) {
    run(ra[0], xa[0], base);
    fill(rb, xb, base + P);
#pragma unroll
    for (int j = 1; j < P; ++j) run(ra[j], xa[j], base + j);
    run(rb[0], xb[0], base + P);
    fill(ra, xa, base + 2 * P);
#pragma unroll
    for (int j = 1; j < P; ++j) run(rb[j], xb[j], base + P + j);
  }

  if constexpr (NS > 1) {
    // sum the slices' partial results (slice 0 keeps the total)
    float* my = red + (slice * kThreads + stid) * 4 * MT * NT;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) my[(mt * NT + nt) * 4 + i] = acc[mt][nt][i];
    __syncthreads();
    if (slice != 0) return;
#pragma unroll
    for (int q = 1; q < NS; ++q) {
      const float* other = red + (q * kThreads + stid) * 4 * MT * NT;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][nt][i] += other[(mt * NT + nt) * 4 + i];
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

// K-blocks per register ring (two rings: codes and X are loaded up to two
// rings ahead); 2 measured best of 2 / 4 / 6.
constexpr int kDirectRing = 2;
// K slices per workgroup (4 waves each): two (one when X is staged twice, as
// the bf16 pair hi + lo of x / s), so that two workgroups share a CU; four
// slices leave one workgroup per CU and measure slower.
template <int MT, int NT, bool SCALE, bool SPLITX>
constexpr int kDirectSlices() {
  return NT > 1 || SPLITX ? 1 : 2;
}

template <int BITS, bool ASYM, class XT, int MT, int NT, int KB, bool SZL, bool SCALE>
hipError_t launch_sz(const void* X, const float* s, const void* packed, const void* scales, const void* zeros,
                     int64_t M, int64_t N, int64_t K, int G, void* Y, hipStream_t stream) {
  constexpr bool kSplitX = SCALE && XT::kMagic2 == BF16::kMagic2;
  constexpr int NS = kDirectSlices<MT, NT, SCALE, kSplitX>();
  const dim3 grid((unsigned)((N + 64 * NT - 1) / (64 * NT)), (unsigned)((M + 16 * MT - 1) / (16 * MT)));
  hipLaunchKernelGGL((gemm_direct_kernel<BITS, ASYM, XT, MT, NT, KB, SCALE, kDirectRing, SZL, NS>), grid,
                     dim3(kThreads * NS), 0, stream, static_cast<const uint16_t*>(X), s,
                     static_cast<const uint8_t*>(packed), static_cast<const uint16_t*>(scales),
                     static_cast<const uint16_t*>(zeros), (int)M, (int)N, (int)K, G, static_cast<uint16_t*>(Y));
  return hipGetLastError();
}

template <int BITS, bool ASYM, class XT, int MT, int NT, int KB>
hipError_t launch_tile(const void* X, const float* s, const void* packed, const void* scales, const void* zeros,
                       int64_t M, int64_t N, int64_t K, int G, void* Y, hipStream_t stream) {
  const bool szl = 64 * NT * (K / G) <= kSZLds;
  if (s)
    return szl ? launch_sz<BITS, ASYM, XT, MT, NT, KB, true, true>(X, s, packed, scales, zeros, M, N, K, G, Y, stream)
               : launch_sz<BITS, ASYM, XT, MT, NT, KB, false, true>(X, s, packed, scales, zeros, M, N, K, G, Y, stream);
  return szl ? launch_sz<BITS, ASYM, XT, MT, NT, KB, true, false>(X, s, packed, scales, zeros, M, N, K, G, Y, stream)
             : launch_sz<BITS, ASYM, XT, MT, NT, KB, false, false>(X, s, packed, scales, zeros, M, N, K, G, Y, stream);
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

// Rows of X from which the large-M kernels (gemm_regb.hip for fp16 with
// 4-bit codes, gemm_lds.hip otherwise) replace the direct-decode kernel; both
// step K by 64 for fp16.
constexpr int64_t kLdsGemmMinM = 128;

// The LDS-staged kernel's 256 x 256 tiles do more per tile than the
// register-B kernel's 128 x 256 tiles, but only pay off when they fill the
// 256 compute units in whole rounds (at least 95% of the last round busy).
static bool lds_tiles_fill_chip(int64_t M, int64_t N) {
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t rounds = (tiles + 255) / 256;
  return tiles * 100 >= rounds * 256 * 95;
}

bool gemm_uses_regb(int64_t M, int64_t N, int64_t K, int bits, int xdtype) {
  // K < 2^16: the kernel's group index by multiplication needs K * G < 2^32
  return M >= kLdsGemmMinM && xdtype == 0 && bits == 4 && K % 64 == 0 && K < 65536 && !lds_tiles_fill_chip(M, N);
}

// The mid-M kernel (gemm_mid.hip, fp16 X, 4-bit codes, 64 x 128 tiles) takes
// 33..127 rows: always above 64 rows (the small-batch kernel stops at 64 and
// the direct kernel is 2.3x slower at 96..127 rows on K = 8192,
// N = 28672), and at 33..64 rows when N gives it at least 128 tiles of
// columns or the small-batch kernel cannot take the shape (measured at
// M = 64, K = 8192: 56.5 against 72.3 us at N = 28672; at N = 11008,
// K = 4096 the small-batch kernel is faster, 20.7 against 25.7 us).
constexpr int64_t kMidMinM = 33;
constexpr int64_t kMidMinN = 16384;

bool gemm_uses_mid(int64_t M, int64_t N, int64_t K, int bits, int xdtype, bool skinny_ok) {
  // K < 2^16: the kernel's group index by multiplication needs K * G < 2^32
  return M >= kMidMinM && M < kLdsGemmMinM && xdtype == 0 && bits == 4 && K % 64 == 0 && K < 65536 &&
         (M > 64 || N >= kMidMinN || !skinny_ok);
}

namespace {

// bf16 X on the fp16 MFMA kernels.  One workgroup per row m: f_m (rs[m])
// is the power of two that puts the row's largest |x| (|x * act_recip(s)|
// with an AWQ scale) in [2^14, 2^15), and X16[m] = fp16(x [* act_recip(s)]
// * f_m); a bf16 value has 8 significant bits and fp16 11, so without an AWQ
// scale the conversion is exact down to 2^-31 of the row's largest value,
// and with one it is the fp16 path's single rounding of x * act_recip(s).
// g_m = 1 / f_m (rs[M + m]) undoes the scaling in the consumer's epilogue.
// Rows of zeros, or with an infinity, keep f_m = g_m = 1 (the infinity
// reaches the output as it would through a bf16 product); NaNs do not enter
// the maximum and propagate through the product.  Up to kXbUnits 16-byte
// units per thread (K <= 16384) stay in registers between the two passes;
// longer rows are read twice.
constexpr int kXbThreads = 256, kXbUnits = 8;

template <bool SCALE>
__global__ __launch_bounds__(kXbThreads) void xb_rescale_kernel(const uint16_t* __restrict__ X,
                                                               const float* __restrict__ s, int M, int K,
                                                               uint16_t* __restrict__ X16, float* __restrict__ rs) {
  __shared__ float wmax[kXbThreads / 64];
  const int row = (int)blockIdx.x, tid = (int)threadIdx.x;
  const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(X + (int64_t)row * K);
  u32x4_t* yr = reinterpret_cast<u32x4_t*>(X16 + (int64_t)row * K);
  const int units = K / 8;
  const bool resident = units <= kXbThreads * kXbUnits;
  auto value = [&](uint32_t word, int half, int u, int e) {
    float x = BF16::to_f32((uint16_t)(word >> (16 * half)));
    if constexpr (SCALE) x *= act_recip(s[8 * u + e]);
    return x;
  };
  u32x4_t v[kXbUnits];
  float mx = 0.0f;
  for (int u0 = 0; u0 < units; u0 += kXbThreads * kXbUnits) {
#pragma unroll
    for (int i = 0; i < kXbUnits; ++i) {
      const int u = u0 + tid + kXbThreads * i;
      if (u < units) v[i] = xr[u];
    }
#pragma unroll
    for (int i = 0; i < kXbUnits; ++i) {
      const int u = u0 + tid + kXbThreads * i;
      if (u < units) {
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(value(v[i][e / 2], e & 1, u, e)));
      }
    }
  }
  mx = team_max(mx, 64);
  if ((tid & 63) == 0) wmax[tid >> 6] = mx;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kXbThreads / 64; ++w) mx = fmaxf(mx, wmax[w]);
  float f = 1.0f;
  if (mx > 0.0f && mx <= 3.40282347e38f) {
    int ef = 14 - ilogbf(mx);
    ef = ef < 127 ? ef : 127;
    f = ldexpf(1.0f, ef);
    if (tid == 0) {
      rs[row] = f;
      rs[M + row] = ldexpf(1.0f, -ef);
    }
  } else if (tid == 0) {
    rs[row] = 1.0f;
    rs[M + row] = 1.0f;
  }
  for (int u0 = 0; u0 < units; u0 += kXbThreads * kXbUnits) {
#pragma unroll
    for (int i = 0; i < kXbUnits; ++i) {
      const int u = u0 + tid + kXbThreads * i;
      if (u < units) {
        const u32x4_t w = resident ? v[i] : xr[u];
        u32x4_t o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = (uint32_t)F16::from_f32(value(w[e], 0, u, 2 * e) * f) |
                 ((uint32_t)F16::from_f32(value(w[e], 1, u, 2 * e + 1) * f) << 16);
        yr[u] = o;
      }
    }
  }
}

// Shapes whose bf16 X can run on the fp16 mid-M or register-B kernel.
// (K < 2^16: both consumers index groups by multiplication, exact for K * G < 2^32.)
bool xb_rescale_ok(int64_t M, int64_t K, int bits) {
  return M >= kMidMinM && bits == 4 && K % 64 == 0 && K < 65536;
}

}  // namespace

// Workspace of the bf16 route: f_m and g_m (8 M bytes, rounded up to 256),
// then the rescaled fp16 copy of X (2 M K bytes).
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int bits, int group_size) {
  (void)N;
  (void)group_size;
  if (!xb_rescale_ok(M, K, bits)) return 0;
  return (size_t)((8 * M + 255) / 256 * 256) + (size_t)(2 * M * K);
}

hipError_t launch_gemm_ws(const void* X, int xdtype, const float* act_scale, const void* packed, const void* scales,
                          const void* zeros, int64_t M, int64_t N, int64_t K, int bits, int group_size,
                          bool asymmetric, void* Y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const size_t need = gemm_workspace_bytes(M, N, K, bits, group_size);
  if (xdtype == 1 && need > 0 && workspace && workspace_bytes >= need) {
    // the fp16 kernels' own routing: register-B from 128 rows, mid-M below
    // where it would take fp16 X (the bf16 small-batch kernel keeps the rest)
    const bool regb = M >= kLdsGemmMinM;
    const bool mid = !regb && gemm_uses_mid(M, N, K, bits, 0,
                                            gemm_skinny_supported(M, N, K, xdtype, act_scale != nullptr, bits,
                                                                  group_size, scales, zeros));
    if (regb || mid) {
      float* rs = static_cast<float*>(workspace);
      uint16_t* X16 = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + (8 * M + 255) / 256 * 256);
      if (act_scale)
        hipLaunchKernelGGL(xb_rescale_kernel<true>, dim3((unsigned)M), dim3(kXbThreads), 0, stream,
                           static_cast<const uint16_t*>(X), act_scale, (int)M, (int)K, X16, rs);
      else
        hipLaunchKernelGGL(xb_rescale_kernel<false>, dim3((unsigned)M), dim3(kXbThreads), 0, stream,
                           static_cast<const uint16_t*>(X), act_scale, (int)M, (int)K, X16, rs);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      // the activation scale is in X16 already
      return regb ? launch_gemm_regb_bf16(X16, packed, scales, zeros, M, N, K, group_size, asymmetric, Y, rs, stream)
                  : launch_gemm_mid_rescaled_bf16(X16, packed, scales, zeros, M, N, K, group_size, asymmetric, Y, rs,
                                                  stream);
    }
  }
  return launch_gemm(X, xdtype, act_scale, packed, scales, zeros, M, N, K, bits, group_size, asymmetric, Y, stream);
}

hipError_t launch_gemm(const void* X, int xdtype, const float* act_scale, const void* packed, const void* scales,
                       const void* zeros, int64_t M, int64_t N, int64_t K, int bits, int group_size, bool asymmetric,
                       void* Y, hipStream_t stream) {
  if (gemm_uses_regb(M, N, K, bits, xdtype))
    return launch_gemm_regb(X, act_scale, packed, scales, zeros, M, N, K, group_size, asymmetric, Y, stream);
  const bool skinny_ok =
      gemm_skinny_supported(M, N, K, xdtype, act_scale != nullptr, bits, group_size, scales, zeros);
  if (gemm_uses_mid(M, N, K, bits, xdtype, skinny_ok))
    return launch_gemm_mid(X, act_scale, packed, scales, zeros, M, N, K, group_size, asymmetric, Y, stream);
  // bf16 X: the same rows and widths, for group sizes the bf16 mid-M kernel
  // takes and without an AWQ scale.
  if (M >= kMidMinM && M < kLdsGemmMinM && xdtype == 1 && bits == 4 && act_scale == nullptr &&
      gemm_mid_bf16_supported(K, group_size) && (M > 64 || N >= kMidMinN || !skinny_ok))
    return launch_gemm_mid_bf16(X, packed, scales, zeros, M, N, K, group_size, asymmetric, Y, stream);
  if (M >= kLdsGemmMinM && (xdtype != 0 || K % 64 == 0))
    return launch_gemm_lds(X, xdtype, act_scale, packed, scales, zeros, M, N, K, bits, group_size, asymmetric, Y,
                           stream);
  if (skinny_ok)
    return launch_gemm_skinny(X, xdtype, act_scale, packed, scales, zeros, M, N, K, asymmetric, Y, stream);
  if (bits == 4)
    return asymmetric
               ? launch_asym<4, true>(X, xdtype, act_scale, packed, scales, zeros, M, N, K, group_size, Y, stream)
               : launch_asym<4, false>(X, xdtype, act_scale, packed, scales, zeros, M, N, K, group_size, Y, stream);
  return asymmetric
             ? launch_asym<3, true>(X, xdtype, act_scale, packed, scales, zeros, M, N, K, group_size, Y, stream)
             : launch_asym<3, false>(X, xdtype, act_scale, packed, scales, zeros, M, N, K, group_size, Y, stream);
}

}  // namespace woq
