// Measurement aids: the ceilings the quantized kernels are measured against.
//
// A decode GEMV streams its weights once and does about one flop per byte,
// so its time floor is the time to read those bytes ("MIT 6.5940 Lab 4 +
// Lab 5", Lab 4 "Starting point and setup").  A large-batch GEMM is bound by
// the matrix units instead ("CMU 11-868 L19-L20", section "Back to the
// question: where does the speed come from?").  These kernels measure what
// the chip sustains for each on its own, with no decode: a read-only stream
// over the same number of bytes, an empty launch (the fixed cost of one
// dispatch), and back-to-back fp16 MFMAs on random operands.
#include "woq_device.h"
#include "woq_internal.h"

namespace woq {
namespace {

typedef _Float16 half8_vt __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

// Each thread reads UNROLL 16-byte units per round, units of one round
// UNROLL * blockDim apart inside the block's window, windows of consecutive
// blocks back to back; rounds advance by the whole grid.  The XOR of every
// word read is stored only when `store` is set at run time, so no load can
// be dropped.
template <int UNROLL>
__global__ __launch_bounds__(1024) void stream_read_kernel(const u32x4_t* __restrict__ p, int64_t units,
                                                           uint32_t* __restrict__ sink, int store) {
  const int64_t per_round = (int64_t)gridDim.x * blockDim.x * UNROLL;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x * UNROLL + threadIdx.x; base < units; base += per_round) {
    u32x4_t v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      int64_t i = base + (int64_t)u * blockDim.x;
      i = i < units ? i : units - 1;
      v[u] = __builtin_nontemporal_load(p + i);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (store) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ void empty_kernel() {}

// ITERS steps of 4 independent v_mfma_f32_32x32x16_f16 chains per wave on
// operands loaded from `src` (random fp16 data); the accumulators are stored
// only when `store` is set.
__global__ __launch_bounds__(256) void mfma_rate_kernel(const u32x4_t* __restrict__ src, int iters,
                                                        float* __restrict__ sink, int store) {
  const int lane = threadIdx.x & 63;
  const int wave = (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
  u32x4_t a[4], b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = src[((wave * 8 + j) & 1023) * 64 + lane];
    b[j] = src[((wave * 8 + 4 + j) & 1023) * 64 + lane];
  }
  float16_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = float16_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_vt, a[j]),
                                                      __builtin_bit_cast(half8_vt, b[(j + it) & 3]), acc[j], 0, 0, 0);
  }
  if (store) {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[j][e];
    sink[(int64_t)wave * 64 + lane] = s;
  }
}

// MFMA / VALU co-issue: ITERS steps of NM v_mfma_f32_32x32x16_f16 (NM / 4
// per chain, 4 independent chains) and NV independent 32-bit integer VALU
// operations (8 chains of v_xad_u32) per wave.  Wave 0 of each workgroup
// records the shader clock counter (s_memtime) and the 100 MHz real-time
// counter (s_memrealtime) at its start and end in clocks[4 * block ..], so
// the host can derive the clock the SIMDs ran at.
template <int NM, int NV>
__global__ __launch_bounds__(256) void mfma_valu_kernel(const u32x4_t* __restrict__ src, int iters,
                                                        float* __restrict__ sink, uint64_t* __restrict__ clocks,
                                                        int store) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  const int lane = threadIdx.x & 63;
  const int wave = (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
  u32x4_t a[4], b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = src[((wave * 8 + j) & 1023) * 64 + lane];
    b[j] = src[((wave * 8 + 4 + j) & 1023) * 64 + lane];
  }
  float16_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = float16_t{};
  uint32_t v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = a[j & 3][j >> 2] + (uint32_t)lane;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NM; ++j)
      acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_vt, a[j & 3]),
                                                          __builtin_bit_cast(half8_vt, b[j & 3]), acc[j & 3], 0, 0, 0);
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k & 7] = (v[k & 7] ^ 0x9E3779B9u) + (uint32_t)k;
  }
  if (store) {
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += acc[j][e];
    uint32_t t = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) t ^= v[j];
    sink[(int64_t)wave * 64 + lane] = sum + (float)t;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    uint64_t* o = clocks + 4 * (int64_t)blockIdx.x;
    o[0] = c0;
    o[1] = c1;
    o[2] = r0;
    o[3] = r1;
  }
}

}  // namespace

hipError_t launch_mfma_valu(const void* src, int blocks, int iters, int mfma_per_iter, int valu_per_iter, float* sink,
                            uint64_t* clocks, int store, hipStream_t stream) {
  const u32x4_t* p = static_cast<const u32x4_t*>(src);
  const dim3 g((unsigned)blocks), t(256);
#define WOQ_MV(NM, NV)                                                                                  \
  if (mfma_per_iter == NM && valu_per_iter == NV) {                                                     \
    hipLaunchKernelGGL((mfma_valu_kernel<NM, NV>), g, t, 0, stream, p, iters, sink, clocks, store);      \
    return hipGetLastError();                                                                           \
  }
  WOQ_MV(4, 0)
  WOQ_MV(4, 16)
  WOQ_MV(4, 32)
  WOQ_MV(4, 64)
  WOQ_MV(0, 32)
  WOQ_MV(0, 64)
#undef WOQ_MV
  return hipErrorInvalidValue;
}

hipError_t launch_stream_read(const void* p, int64_t bytes, int blocks, int threads, int unroll, void* sink,
                              int store, hipStream_t stream) {
  const int64_t units = bytes / 16;
  const dim3 g((unsigned)blocks), t((unsigned)threads);
  const u32x4_t* src = static_cast<const u32x4_t*>(p);
  uint32_t* s = static_cast<uint32_t*>(sink);
  switch (unroll) {
    case 1:
      hipLaunchKernelGGL(stream_read_kernel<1>, g, t, 0, stream, src, units, s, store);
      break;
    case 2:
      hipLaunchKernelGGL(stream_read_kernel<2>, g, t, 0, stream, src, units, s, store);
      break;
    case 4:
      hipLaunchKernelGGL(stream_read_kernel<4>, g, t, 0, stream, src, units, s, store);
      break;
    case 8:
      hipLaunchKernelGGL(stream_read_kernel<8>, g, t, 0, stream, src, units, s, store);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_empty(int blocks, int threads, hipStream_t stream) {
  hipLaunchKernelGGL(empty_kernel, dim3((unsigned)blocks), dim3((unsigned)threads), 0, stream);
  return hipGetLastError();
}

hipError_t launch_mfma_rate(const void* src, int blocks, int iters, float* sink, int store, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const u32x4_t*>(src), iters, sink, store);
  return hipGetLastError();
}

}  // namespace woq
