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

}  // namespace

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
