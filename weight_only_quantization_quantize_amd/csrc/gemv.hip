// Fused dequantize + GEMV for M = 1 decode: y[n] = sum_k x'[k] (u[n,k] - Z) S.
//
// Decode is memory-bound: a [1, K] x [K, N] GEMV does about one flop per byte
// of weights ("MIT 6.5940 Lab 4 + Lab 5", Lab 4 "Starting point and setup";
// "CMU 11-868 L19-L20", section "Back to the question: where does the speed
// come from?"), so the kernel streams the packed codes from HBM exactly once
// and dequantizes them in registers ("Quantising Large Language Models ...",
// section "Weight-only vs weight-and-activation quantisation").
//
// Work split.  A row of K weights is cut into segments of up to 64 chunks of
// 32 weights (one 16-byte / 12-byte load per lane per segment).  A workgroup
// holds RPB rows x SPR segments, one wave per (row, segment); lane p of the
// wave for segment g always owns chunk 64 g + p, so its 32 activations are
// read once (from x' = x / s staged in LDS) and stay in 16 registers (32 for
// bf16 with an AWQ scale, where x' is kept as a bf16 pair hi + lo).
//
// Order of the stream.  Workgroup b handles the row groups b, b + B, b + 2B,
// ... (B = number of workgroups), so at every step the whole GPU reads one
// contiguous window of B * RPB rows; each wave keeps 2 steps of code loads
// in flight ahead of the step it computes (4 on the general path with 8 row
// steps per workgroup).
//
// Decode.  fp16 activations: a masked 4-bit code pair (w & 0x000F000F, or
// w & 0x00F000F0 for the pair one nibble up) is read by v_dot2 as two fp16
// subnormals of value u * 2^-24 (resp. 16u * 2^-24), which v_dot2 multiplies
// exactly; one AND per pair and
//   sum x (u - Z) = 2^24 (a + b / 16) - Z * sum x.
// 3-bit codes (layout v2: each pair's three bits together) are masked where
// they sit, as subnormals of weight 1, 8 or 64.  bf16 activations
// OR the pair into the 16-bit float MAGIC + u (0x4300 = 128) and remove
// (MAGIC + Z) * sum x instead.
//
// Reduction.  Each lane keeps one fp32 partial per step in LDS; after the
// stream each wave sums the partials of a few outputs with one DPP reduction,
// so no cross-lane work interrupts the stream.
#include "woq_device.h"
#include "woq_internal.h"

namespace woq {
namespace {

constexpr int kMaxSegments = 8;      // K <= 8 * 64 * 32 = 16384 on this path
#ifndef WOQ_GEMV_WAVES
#define WOQ_GEMV_WAVES 8
#endif
constexpr int kTargetWaves = WOQ_GEMV_WAVES;  // waves per workgroup (rows x segments)
constexpr size_t kGeneralLds = 96 * 1024;     // LDS bytes up to which the general path rounds rows up
#ifndef WOQ_GEMV_BLOCKS
#define WOQ_GEMV_BLOCKS 256
#endif
#ifndef WOQ_GEMV_MAXSTEPS
#define WOQ_GEMV_MAXSTEPS 4
#endif
#ifndef WOQ_GEMV_PREFETCH
#define WOQ_GEMV_PREFETCH 2
#endif
constexpr int kTargetBlocks = WOQ_GEMV_BLOCKS;   // workgroups sweeping the matrix together
constexpr int kMaxSteps = WOQ_GEMV_MAXSTEPS;     // row steps per workgroup (at most; 2x / 4x on the general path)
constexpr int kPrefetch = WOQ_GEMV_PREFETCH;     // steps of code loads in flight ahead of compute

struct __attribute__((packed, aligned(4))) U32x3 {
  uint32_t a, b, c;
};

template <int BITS>
struct Codes;
template <>
struct Codes<4> {
  u32x4_t w;
};
template <>
struct Codes<3> {
  uint32_t w0, w1, w2;
};

template <int BITS>
__device__ inline void load_codes(const uint8_t* __restrict__ p, Codes<BITS>& c) {
  if constexpr (BITS == 4) {
    c.w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  } else {
    const U32x3 v = *reinterpret_cast<const U32x3*>(p);
    c.w0 = v.a;
    c.w1 = v.b;
    c.w2 = v.c;
  }
}

// Activation sums of one chunk: part[0] over the pairs t = 0, 2 of every
// 8-weight word, part[1] over t = 1, 3.
struct XSums {
  float part[2];
};

// sum over the chunk of x (u - Z), before the scale S.
template <int BITS, class XT>
__device__ inline float chunk_dot(const Codes<BITS>& c, const uint32_t (&xr)[16], const XSums& xs, float Z,
                                  uint32_t magic) {
  constexpr bool kF16 = XT::kMagic2 == F16::kMagic2;
  if constexpr (BITS == 4 && kF16) {
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = c.w[j], w8 = w >> 8;
      a = XT::dot2(w & 0x000F000Fu, xr[4 * j + 0], a);   // u * 2^-24, pair t = 0
      b = XT::dot2(w & 0x00F000F0u, xr[4 * j + 1], b);   // 16u * 2^-24, pair t = 1
      a = XT::dot2(w8 & 0x000F000Fu, xr[4 * j + 2], a);  // pair t = 2
      b = XT::dot2(w8 & 0x00F000F0u, xr[4 * j + 3], b);  // pair t = 3
    }
    return 16777216.0f * (a + 0.0625f * b) - Z * (xs.part[0] + xs.part[1]);
  } else if constexpr (BITS == 4) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) a = XT::dot2(((c.w[j] >> (4 * t)) & 0x000F000Fu) | magic, xr[4 * j + t], a);
    return a - (XT::kMagic + Z) * (xs.part[0] + xs.part[1]);
  } else if constexpr (kF16) {
    // Layout v2 keeps each pair's three bits together, so a masked pair is
    // read where it sits as two fp16 subnormals of a known power-of-two
    // weight (one AND and one dot2 per pair): fields j = 0, 1, 2 of word w
    // (pair 5w + j, bits 3j) weigh 1, 8, 64; after w >> 9, fields j = 3, 4
    // weigh 1, 8, and bit 6 of each half holds bit w of pair 15's codes,
    // which three masks and two shift-ORs assemble at bits 6..8 (weight 64).
    float a[3] = {0.0f, 0.0f, 0.0f};
    uint32_t hi[3];
#pragma unroll
    for (int wi = 0; wi < 3; ++wi) {
      const uint32_t w = wi == 0 ? c.w0 : (wi == 1 ? c.w1 : c.w2);
#pragma unroll
      for (int j = 0; j < 3; ++j) a[j] = XT::dot2(w & (0x00070007u << (3 * j)), xr[5 * wi + j], a[j]);
      hi[wi] = w >> 9;
      a[0] = XT::dot2(hi[wi] & 0x00070007u, xr[5 * wi + 3], a[0]);
      a[1] = XT::dot2(hi[wi] & 0x00380038u, xr[5 * wi + 4], a[1]);
    }
    const uint32_t p15 = (((((hi[2] & 0x00400040u) << 1) | (hi[1] & 0x00400040u)) << 1)) | (hi[0] & 0x00400040u);
    a[2] = XT::dot2(p15, xr[15], a[2]);
    return 16777216.0f * (a[0] + 0.125f * a[1] + 0.015625f * a[2]) - Z * (xs.part[0] + xs.part[1]);
  } else {
    float a = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t) a = XT::dot2(pair3(c.w0, c.w1, c.w2, t, 0u) | magic, xr[t], a);
    return a - (XT::kMagic + Z) * (xs.part[0] + xs.part[1]);
  }
}

// v + (v taken from the lane the DPP control selects; 0 where there is none).
template <int CTRL, int ROW_MASK>
__device__ inline float add_dpp(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                                                   0xf, true));
}

// Full 64-lane sum; the total lands in lane 63.
__device__ inline float wave_sum_lane63(float v) {
  v = add_dpp<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
  v = add_dpp<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]
  v = add_dpp<0x114, 0xf>(v);  // row_shr:4
  v = add_dpp<0x118, 0xf>(v);  // row_shr:8
  v = add_dpp<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = add_dpp<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

template <int BITS>
struct StepLoads {
  Codes<BITS> c;
  uint16_t s16, z16;
};

// Dynamic LDS layout: x' (padded to PASSES * threads 16-byte units) |
// partials [STEPS][waves][64] floats.
//
// SPR_T > 0 fixes the shape at compile time: K = 2048 * SPR_T (every segment
// full), group size 128, RPB = max(1, kTargetWaves / SPR_T) rows per workgroup.  SPR_T == 0
// is the general path (any K <= 16384 that is a multiple of 32, any group
// size that is a multiple of 32), with the shape passed at run time.
// Timeline stamp (100 MHz real-time counter), ordered after every earlier
// memory operation of the wave; used only by the TL instance.
__device__ inline uint64_t tl_stamp() {
  uint64_t t;
  asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t)::"memory");
  return t;
}

// TL: measurement instance that also writes a per-wave timeline to tl (8
// words per wave: start, x staged, first step computed, stream done, end,
// XCD id); the kernel's work is otherwise the same.
template <int BITS, bool ASYM, class XT, bool SCALE, int STEPS, int SPR_T, int PASSES, bool TL>
__global__ __launch_bounds__(1024) void gemv_kernel(const uint16_t* __restrict__ x, const float* __restrict__ s,
                                                    const uint8_t* __restrict__ packed,
                                                    const uint16_t* __restrict__ scales,
                                                    const uint16_t* __restrict__ zeros, int N, int K_rt, int G_rt,
                                                    int spr_rt, int rpb_rt, uint16_t* __restrict__ y,
                                                    uint64_t* __restrict__ tl) {
  uint64_t t_start = 0, t_x = 0, t_first = 0, t_stream = 0;
  if constexpr (TL) t_start = tl_stamp();
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  constexpr bool kFixed = SPR_T > 0;
  // the fixed shapes stage all K / 8 16-byte units of x in PASSES passes
  static_assert(!kFixed || PASSES * (SPR_T >= kTargetWaves ? 1 : kTargetWaves / SPR_T) * SPR_T * 64 >= 256 * SPR_T,
                "x staging passes do not cover K");
  // bf16 with an AWQ scale: x / s is staged as a bf16 pair hi + lo (about 16
  // significant bits, a second x region in LDS) and each chunk is dotted with
  // both halves.
  constexpr bool kSplitX = SCALE && XT::kMagic2 == BF16::kMagic2;
  const int K = kFixed ? 2048 * SPR_T : K_rt;
  const int G = kFixed ? 128 : G_rt;
  const int spr = kFixed ? SPR_T : spr_rt;
  const int rpb = kFixed ? (SPR_T >= kTargetWaves ? 1 : kTargetWaves / SPR_T) : rpb_rt;
  const int nthreads = kFixed ? rpb * spr * 64 : (int)blockDim.x;
  const int cpr = K >> 5;  // chunks per row
  uint32_t* xsh = lds;
  uint32_t* xlo = lds + PASSES * nthreads * 4;  // kSplitX only
  float* part = reinterpret_cast<float*>(lds + (kSplitX ? 2 : 1) * PASSES * nthreads * 4);
  const int waves = nthreads >> 6;
  const int lane = threadIdx.x & 63;
  // wave-uniform values live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int seg = wave % spr, rr = wave / spr;  // K segment and row slot of this wave
  const int c_raw = 64 * seg + lane;            // this lane's chunk
  const bool live = kFixed || c_raw < cpr;
  const int c = live ? c_raw : cpr - 1;         // clamped: every load stays inside the row
  const int cg = (32 * c) / G;                  // its group within the row
  const int gpr = K / G;
  const int64_t row_bytes = (int64_t)K * BITS / 8;
  const uint8_t* lane_codes = packed + (int64_t)c * (BITS == 4 ? 16 : 12);
  const int row_first = (int)blockIdx.x * rpb + rr;
  const int row_step = (int)gridDim.x * rpb;

  // Steps of code loads in flight: twice as many on the general path with 8
  // or more row steps per workgroup (few waves per compute unit there; e.g.
  // K = 11008, N = 4096: 10.60 -> 10.19 us), kPrefetch elsewhere (4 slowed
  // the fixed-shape K = N = 8192 launch, 8.30 -> 8.50 us).
  // 3-bit fixed shapes keep 1 (K = N = 8192 asymmetric: 7.72 -> 7.35 us;
  // LLaMA-2-7B gate / up with AWQ 6.78 -> 6.44 us; the 4-bit c2 launch lost
  // 1.5% with it, symmetric).
  constexpr int kPf = (!kFixed && STEPS >= 8) ? 2 * kPrefetch : (kFixed && BITS == 3 ? 1 : kPrefetch);
  StepLoads<BITS> L[STEPS];
  auto issue = [&](int st) {
    int n = row_first + st * row_step;
    n = n < N ? n : N - 1;
    load_codes<BITS>(lane_codes + (int64_t)n * row_bytes, L[st].c);
    const int64_t gi = (int64_t)n * gpr + cg;
    L[st].s16 = scales[gi];
    if (ASYM) L[st].z16 = zeros[gi];
  };

  // x loads first, then the first code loads: waiting for x (the memory
  // counter drains in issue order) does not wait for the codes.
  const int units = K >> 3;  // 16-byte units of x
  u32x4_t xv[PASSES];
  float4_t sv[PASSES][2];
#pragma unroll
  for (int it = 0; it < PASSES; ++it) {
    int i = threadIdx.x + it * nthreads;
    i = i < units ? i : units - 1;
    xv[it] = reinterpret_cast<const u32x4_t*>(x)[i];
    if (SCALE) {
      sv[it][0] = reinterpret_cast<const float4_t*>(s)[2 * i];
      sv[it][1] = reinterpret_cast<const float4_t*>(s)[2 * i + 1];
    }
  }
#pragma unroll
  for (int st = 0; st < kPf && st < STEPS; ++st) issue(st);

  // Stage x' = x * (1 / s), rounded once to the activation type, in LDS
  // (act_recip: an IEEE division per activation, up to 32 per thread at
  // K = 11008, sat in front of the workgroup's first barrier; LLaMA-2-7B down
  // projection with AWQ: 10.2 -> 9.0 us).
#pragma unroll
  for (int it = 0; it < PASSES; ++it) {
    const int i = threadIdx.x + it * nthreads;
    u32x4_t v = xv[it], vl = u32x4_t{0u, 0u, 0u, 0u};
    if (SCALE) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a0 = XT::to_f32((uint16_t)(v[e] & 0xFFFFu)) * act_recip(sv[it][e / 2][(2 * e) % 4]);
        const float a1 = XT::to_f32((uint16_t)(v[e] >> 16)) * act_recip(sv[it][e / 2][(2 * e) % 4 + 1]);
        const uint16_t h0 = XT::from_f32(a0), h1 = XT::from_f32(a1);
        v[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        if (kSplitX)
          vl[e] = (uint32_t)XT::from_f32(a0 - XT::to_f32(h0)) | ((uint32_t)XT::from_f32(a1 - XT::to_f32(h1)) << 16);
      }
    }
    // unconditional (the region is padded to PASSES * threads units): a
    // conditional store would let the compiler sink the load behind the codes
    reinterpret_cast<u32x4_t*>(xsh)[i] = v;
    if (kSplitX) reinterpret_cast<u32x4_t*>(xlo)[i] = vl;
  }
  __syncthreads();
  if constexpr (TL) t_x = tl_stamp();

  // This lane's 32 activations and their sums (lanes past the row end: 0).
  const uint32_t ones2 = XT::kMagic2 == F16::kMagic2 ? 0x3C003C00u : 0x3F803F80u;
  uint32_t xr[16], xl[kSplitX ? 16 : 1];
  XSums xs, xsl;
  xs.part[0] = xs.part[1] = xsl.part[0] = xsl.part[1] = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4_t v = reinterpret_cast<const u32x4_t*>(xsh)[4 * c + q];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xr[4 * q + e] = live ? v[e] : 0u;
      xs.part[e & 1] = XT::dot2(xr[4 * q + e], ones2, xs.part[e & 1]);
    }
    if constexpr (kSplitX) {
      const u32x4_t vl = reinterpret_cast<const u32x4_t*>(xlo)[4 * c + q];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xl[4 * q + e] = live ? vl[e] : 0u;
        xsl.part[e & 1] = XT::dot2(xl[4 * q + e], ones2, xsl.part[e & 1]);
      }
    }
  }

  const uint32_t magic = vgpr_const(XT::kMagic2);
  const float zsym = (float)(1 << (BITS - 1));
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    if (st + kPf < STEPS) issue(st + kPf);
    const float S = half_bits_to_f32(L[st].s16);
    const float Z = ASYM ? half_bits_to_f32(L[st].z16) : zsym;
    float d = chunk_dot<BITS, XT>(L[st].c, xr, xs, Z, magic);
    if constexpr (kSplitX) d += chunk_dot<BITS, XT>(L[st].c, xl, xsl, Z, magic);
    part[(st * waves + wave) * 64 + lane] = S * d;
    if constexpr (TL) {
      if (st == 0) t_first = tl_stamp();
    }
  }
  __syncthreads();
  if constexpr (TL) t_stream = tl_stamp();

  // Output o = (step, row slot): the spr * 64 partials of one row.
  for (int o = wave; o < STEPS * rpb; o += waves) {
    const int st = o / rpb, r = o - st * rpb;
    float v = 0.0f;
    for (int g = 0; g < spr; ++g) v += part[(st * waves + r * spr + g) * 64 + lane];
    v = wave_sum_lane63(v);
    const int n = row_first - rr + r + st * row_step;
    if (lane == 63 && n < N) y[n] = XT::from_f32(v);
  }
  if constexpr (TL) {
    const uint64_t t_end = tl_stamp();
    if (lane == 0) {
      uint64_t* o = tl + ((int64_t)blockIdx.x * waves + wave) * 8;
      o[0] = t_start;
      o[1] = t_x;
      o[2] = t_first;
      o[3] = t_stream;
      o[4] = t_end;
      o[5] = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // HW_REG_XCC_ID
      o[6] = 0;
      o[7] = 0;
    }
  }
}

template <int BITS, bool ASYM, class XT, bool SCALE, int STEPS, int SPR_T, int PASSES, bool TL = false>
hipError_t launch_kernel(const void* x, const float* s, const void* packed, const void* scales, const void* zeros,
                         int64_t N, int64_t K, int G, int spr, int rpb, int64_t blocks, void* y,
                         hipStream_t stream, uint64_t* tl = nullptr) {
  const int threads = rpb * spr * 64;
  constexpr bool kSplitX = SCALE && XT::kMagic2 == BF16::kMagic2;
  const size_t lds = (size_t)(kSplitX ? 2 : 1) * PASSES * threads * 16 + (size_t)STEPS * (threads / 64) * 64 * 4;
  hipLaunchKernelGGL((gemv_kernel<BITS, ASYM, XT, SCALE, STEPS, SPR_T, PASSES, TL>), dim3((unsigned)blocks), dim3(threads), lds,
                     stream, static_cast<const uint16_t*>(x), s, static_cast<const uint8_t*>(packed),
                     static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros), (int)N, (int)K, G, spr,
                     rpb, static_cast<uint16_t*>(y), tl);
  return hipGetLastError();
}

// Shapes compiled with K and the group size fixed.
inline bool fixed_shape(int64_t K, int G) {
  return G == 128 && (K == 2048 || K == 4096 || K == 8192 || K == 16384);
}

template <int BITS, bool ASYM, class XT, bool SCALE, int STEPS>
hipError_t launch_steps(const void* x, const float* s, const void* packed, const void* scales, const void* zeros,
                        int64_t N, int64_t K, int G, int spr, int rpb, int64_t blocks, void* y, hipStream_t stream) {
#define WOQ_FIXED(SPR, PASSES)                                                                                    \
  if (G == 128 && K == 2048 * SPR)                                                                                \
    return launch_kernel<BITS, ASYM, XT, SCALE, STEPS, SPR, PASSES>(x, s, packed, scales, zeros, N, K, G, spr, rpb, blocks, \
                                                             y, stream);
  if constexpr (STEPS <= kMaxSteps) {
    WOQ_FIXED(1, 1)
    WOQ_FIXED(2, 1)
    WOQ_FIXED(4, 2)
    WOQ_FIXED(8, 4)
  }
#undef WOQ_FIXED
  // General shapes: x staging covers K/8 units in at most 4 passes (K/8 <= 256
  // spr and the workgroup has at least 64 spr threads).
  return launch_kernel<BITS, ASYM, XT, SCALE, STEPS, 0, 4>(x, s, packed, scales, zeros, N, K, G, spr, rpb, blocks, y,
                                                    stream);
}

template <int BITS, bool ASYM, class XT, bool SCALE>
hipError_t launch_scale(const void* x, const float* s, const void* packed, const void* scales, const void* zeros,
                     int64_t N, int64_t K, int G, void* y, hipStream_t stream) {
  const int64_t cpr = K / 32;
  const int spr = (int)((cpr + 63) / 64);
  if (spr > kMaxSegments) return hipErrorInvalidValue;
  const bool fixed = fixed_shape(K, G);
  // The general path's lanes do more per step (run-time shape), so it takes up
  // to twice as many steps per workgroup (measured: K = 11008 12.3 -> 10.9 us),
  // and four times as many with an AWQ scale, whose x staging (x and the fp32
  // s, one reciprocal per activation) every workgroup repeats: LLaMA-2-7B down
  // projection (K = 11008) 9.0 -> 8.35 us at 256 workgroups of 16 steps.
  // Without the scale, and on the fixed shapes (gate / up 6.88 -> 7.18 us),
  // more steps were slower.
  const int max_steps = fixed ? kMaxSteps : (SCALE ? 4 : 2) * kMaxSteps;
  // Rows per workgroup: kTargetWaves / segments, rounded up on the general
  // path where the segments do not divide it, unless the LDS would then pass
  // kGeneralLds (LLaMA-2-7B down projection with AWQ, K = 11008, 6 segments:
  // 1 -> 2 rows, 6 -> 12 waves, 8.28 -> 8.04 us, same bits).  A 16-wave
  // target everywhere was slower where 8 already divides: K = 8192 at G = 64
  // 8.95 -> 9.59 us, q_proj with AWQ 4.00 -> 4.25 us.
  constexpr bool kSplitX = SCALE && XT::kMagic2 == BF16::kMagic2;
  int rpb = 1, steps = 1;
  int64_t groups = N;
  for (int up = fixed ? 0 : 1;; up = 0) {
    rpb = spr >= kTargetWaves ? 1 : (kTargetWaves + (up ? spr - 1 : 0)) / spr;
    groups = (N + rpb - 1) / rpb;
    steps = 1;
    while (steps < max_steps && groups / (2 * steps) >= kTargetBlocks) steps *= 2;
    const size_t lds = (size_t)(kSplitX ? 2 : 1) * 4 * rpb * spr * 64 * 16 + (size_t)steps * rpb * spr * 64 * 4;
    if (!up || lds <= kGeneralLds) break;
  }
  const int64_t blocks = (groups + steps - 1) / steps;
  switch (steps) {
    case 1:
      return launch_steps<BITS, ASYM, XT, SCALE, 1>(x, s, packed, scales, zeros, N, K, G, spr, rpb, blocks, y, stream);
    case 2:
      return launch_steps<BITS, ASYM, XT, SCALE, 2>(x, s, packed, scales, zeros, N, K, G, spr, rpb, blocks, y, stream);
    case 4:
      return launch_steps<BITS, ASYM, XT, SCALE, 4>(x, s, packed, scales, zeros, N, K, G, spr, rpb, blocks, y, stream);
    case 8:
      return launch_steps<BITS, ASYM, XT, SCALE, 8>(x, s, packed, scales, zeros, N, K, G, spr, rpb, blocks, y, stream);
    case 16:
      return launch_steps<BITS, ASYM, XT, SCALE, 16>(x, s, packed, scales, zeros, N, K, G, spr, rpb, blocks, y, stream);
    default:
      return hipErrorInvalidValue;
  }
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

// Largest K the register-resident GEMV handles (8 segments of 64 chunks).
int gemv_max_k() { return kMaxSegments * 64 * 32; }

namespace {
// Launch shape of the K = 8192, G = 128 fixed-shape GEMV for N rows (the
// same rule launch_scale applies).
constexpr int kTlSpr = 4, kTlRpb = kTargetWaves / kTlSpr;
int64_t timeline_shape(int64_t N, int& steps) {
  const int64_t groups = (N + kTlRpb - 1) / kTlRpb;
  steps = 1;
  while (steps < kMaxSteps && groups / (2 * steps) >= kTargetBlocks) steps *= 2;
  return (groups + steps - 1) / steps;
}
}  // namespace

size_t gemv_timeline_words(int64_t N) {
  int steps = 0;
  return (size_t)timeline_shape(N, steps) * kTlRpb * kTlSpr * 8;
}

hipError_t launch_gemv_timeline(const void* x, const void* packed, const void* scales, const void* zeros, int64_t N,
                                void* y, uint64_t* tl, hipStream_t stream) {
  int steps = 0;
  const int64_t blocks = timeline_shape(N, steps);
  switch (steps) {
    case 1:
      return launch_kernel<4, true, F16, false, 1, kTlSpr, 2, true>(x, nullptr, packed, scales, zeros, N, 8192, 128,
                                                                   kTlSpr, kTlRpb, blocks, y, stream, tl);
    case 2:
      return launch_kernel<4, true, F16, false, 2, kTlSpr, 2, true>(x, nullptr, packed, scales, zeros, N, 8192, 128,
                                                                   kTlSpr, kTlRpb, blocks, y, stream, tl);
    case 4:
      return launch_kernel<4, true, F16, false, 4, kTlSpr, 2, true>(x, nullptr, packed, scales, zeros, N, 8192, 128,
                                                                   kTlSpr, kTlRpb, blocks, y, stream, tl);
    default:
      return hipErrorInvalidValue;
  }
}

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
