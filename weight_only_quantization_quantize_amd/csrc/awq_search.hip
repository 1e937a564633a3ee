// AWQ exponent search on the GPU.
//
// For alpha_i = i / n_grid (i = 0 .. n_grid - 1) the per-channel scale is
// s = max(mean_t |x_t|, 1e-4)^alpha; the weights are scaled up by s and
// quantized, the calibration activations are divided by s, and the layer's
// output error || X W^T - (X / s) Q(W s)^T ||_F^2 is measured; the first
// alpha with the smallest error wins ("MIT 6.5940 Lab 4 + Lab 5", Question 2:
// compute the scale, scale up, quantize, scale down; the layer-wise
// reconstruction objective of "Quantising Large Language Models ...", section
// "Post-training methods for 4-bit weights").
//
// The loop over alpha runs on the host and only enqueues work: per alpha one
// scale kernel, the library's quantize_pack and GEMM, and a two-pass
// deterministic reduction of the squared error in fp64.  Where the GEMM is
// the register-B kernel, the products of up to 8 alphas run as one batched
// launch (the same kernel per tile, so the same outputs), which fills the
// compute units that one product's tiles would leave idle.  The reference
// output X W^T (fp32, from a dense fp16 MFMA kernel) and the channel means
// (fp64) are computed once.  Everything lives in the caller's workspace.
#include <mutex>

#include "woq_device.h"
#include "woq_internal.h"

namespace woq {
namespace {

// Scratch of the allocation-free search: a file-scope device array (each GPU
// that loads the library holds its own copy until the process ends).  In
// host code `scratch` only names the symbol; its device address on the
// current device comes from hipGetSymbolAddress, taken once per device.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
__device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr double kScaleFloor = 1e-4;
constexpr int kPartials = 1024;  // blocks of the first reduction pass

// m[k] = mean over t of |x[t, k]|, summed in fp64 and divided once.  Every
// fp16 magnitude is an integer multiple of 2^-24 below 2^16, so sums of fewer
// than 8192 of them are exact in fp64 in any order.  A workgroup takes 64
// channels; its 16 waves take every 16th token and meet in LDS.
constexpr int kMeanChannels = 64, kMeanSlices = 16;
__global__ __launch_bounds__(kMeanChannels * kMeanSlices) void channel_mean_kernel(const uint16_t* __restrict__ X,
                                                                                   int T, int K,
                                                                                   double* __restrict__ m) {
  __shared__ double part[kMeanSlices][kMeanChannels];
  const int c = threadIdx.x % kMeanChannels, sl = threadIdx.x / kMeanChannels;
  const int k = blockIdx.x * kMeanChannels + c;
  const int kk = k < K ? k : K - 1;
  double acc = 0.0;
  for (int t = sl; t < T; t += kMeanSlices) acc += fabs((double)half_bits_to_f32(X[(int64_t)t * K + kk]));
  part[sl][c] = acc;
  __syncthreads();
  if (sl == 0 && k < K) {
    double v = 0.0;
#pragma unroll
    for (int j = 0; j < kMeanSlices; ++j) v += part[j][c];
    m[k] = v / T;
  }
}

// s[k] = fl32(max(m[k], floor)^alpha).
__global__ void awq_scale_kernel(const double* __restrict__ m, double alpha, int K, float* __restrict__ s) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  s[k] = (float)pow(fmax(m[k], kScaleFloor), alpha);
}

// Y[t, n] = sum_k X[t, k] W[n, k] in fp32: a 64 x 64 tile per workgroup, one
// 32 x 32 v_mfma_f32_32x32x16_f16 tile per wave, operands loaded straight
// from global memory (lane l: row l % 32, K half l / 32 of each 16-wide step).
// Rows and columns past T / N read the last row (results not stored).
__global__ __launch_bounds__(256) void dense_ref_kernel(const uint16_t* __restrict__ X,
                                                        const uint16_t* __restrict__ W, int T, int N, int K,
                                                        float* __restrict__ Y) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.y * 64 + 32 * (wave >> 1), n0 = blockIdx.x * 64 + 32 * (wave & 1);
  const int r = lane & 31, h = lane >> 5;
  const int ta = t0 + r < T ? t0 + r : T - 1;
  const int nb = n0 + r < N ? n0 + r : N - 1;
  const uint16_t* xa = X + (int64_t)ta * K + 8 * h;
  const uint16_t* wb = W + (int64_t)nb * K + 8 * h;
  float16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  // 8 steps of operands loaded before their MFMAs (K % 128 == 0 here, the
  // remainder one step at a time); the MFMAs run in K order either way.
  constexpr int kU = 8;
  int k = 0;
  for (; k + 16 * kU <= K; k += 16 * kU) {
    u32x4_t a[kU], b[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      a[u] = *reinterpret_cast<const u32x4_t*>(xa + k + 16 * u);
      b[u] = *reinterpret_cast<const u32x4_t*>(wb + k + 16 * u);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a[u]), __builtin_bit_cast(half8_t, b[u]),
                                                   acc, 0, 0, 0);
  }
  for (; k < K; k += 16) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(xa + k);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(wb + k);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), acc,
                                                 0, 0, 0);
  }
  // accumulator v holds C[m = 8 (v / 4) + 4 h + v % 4][n = r]
  const int n = n0 + r;
  if (n >= N) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int t = t0 + 8 * (v >> 2) + 4 * h + (v & 3);
    if (t < T) Y[(int64_t)t * N + n] = acc[v];
  }
}

// First pass: block b sums (yref - yq)^2 over its grid-stride share in fp64
// and writes partial[b]; a fixed-order tree makes the result deterministic.
__global__ __launch_bounds__(256) void sqdiff_partial_kernel(const float* __restrict__ yref,
                                                             const uint16_t* __restrict__ yq, int64_t count,
                                                             double* __restrict__ partial) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
    const double d = (double)yref[i] - (double)half_bits_to_f32(yq[i]);
    acc += d * d;
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

// Second pass: one block adds the kPartials partial sums in a fixed order.
__global__ __launch_bounds__(256) void sqdiff_finish_kernel(const double* __restrict__ partial,
                                                            double* __restrict__ loss) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int i = threadIdx.x; i < kPartials; i += 256) acc += partial[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = red[0];
}

// The first alpha with the smallest loss; its scale for every channel.
__global__ void awq_select_kernel(const double* __restrict__ losses, int n_grid, const double* __restrict__ m, int K,
                                  float* __restrict__ best_scale, int32_t* __restrict__ best_index) {
  int best = 0;
  for (int i = 1; i < n_grid; ++i)
    if (losses[i] < losses[best]) best = i;
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k == 0) *best_index = best;
  if (k < K) best_scale[k] = (float)pow(fmax(m[k], kScaleFloor), (double)best / n_grid);
}

constexpr size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Alphas per batched GEMM launch: enough register-B tiles (128 x 256) for two
// workgroups on each of the 256 compute units, at most 8; 1 where the GEMM is
// another kernel.
int awq_batch(int64_t T, int64_t N, int64_t K, int bits) {
  if (!gemm_uses_regb(T, N, K, bits, 0)) return 1;
  const int64_t tiles = ((T + 127) / 128) * ((N + 255) / 256);
  const int64_t b = (512 + tiles - 1) / tiles;
  return (int)(b > 8 ? 8 : b);
}

struct AwqLayout {
  int batch;
  size_t m, s, packed, scales, zeros, yref, yq, partial, total;
  size_t packed_bytes, sz_elems, yq_elems;  // per batch entry
};

AwqLayout awq_layout(int64_t T, int64_t N, int64_t K, int bits, int G, bool asym, int max_batch = 8) {
  AwqLayout L{};
  const int b = awq_batch(T, N, K, bits);
  L.batch = b < max_batch ? b : max_batch;
  L.packed_bytes = (size_t)N * K * bits / 8;  // a multiple of 16 (K % 32 == 0)
  L.sz_elems = (size_t)N * (K / G);
  L.yq_elems = (size_t)T * N;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  L.m = take(sizeof(double) * K);
  L.s = take(sizeof(float) * K * L.batch);
  L.packed = take(L.packed_bytes * L.batch);
  L.scales = take(sizeof(uint16_t) * L.sz_elems * L.batch);
  L.zeros = take(asym ? sizeof(uint16_t) * L.sz_elems * L.batch : 0);
  L.yref = take(sizeof(float) * T * N);
  L.yq = take(sizeof(uint16_t) * L.yq_elems * L.batch);
  L.partial = take(sizeof(double) * kPartials);
  L.total = off;
  return L;
}

}  // namespace

hipError_t launch_dense_ref(const void* A, const void* B, int64_t M, int64_t N, int64_t K, float* Y,
                            hipStream_t stream) {
  hipLaunchKernelGGL(dense_ref_kernel, dim3((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64)), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), (int)M, (int)N, (int)K,
                     Y);
  return hipGetLastError();
}

size_t awq_search_workspace_bytes(int64_t T, int64_t N, int64_t K, int bits, int group_size, bool asymmetric) {
  return awq_layout(T, N, K, bits, group_size, asymmetric).total;
}

size_t awq_search_noalloc_max_bytes() { return kNoAllocScratchBytes; }

// The most exponents per batched GEMM launch whose layout fits the static
// scratch (the batch does not change any output: every batched tile runs the
// same kernel code as a single product); 0 if not even one fits.
int awq_noalloc_batch(int64_t T, int64_t N, int64_t K, int bits, int group_size, bool asymmetric) {
  for (int b = 8; b >= 1; --b)
    if (awq_layout(T, N, K, bits, group_size, asymmetric, b).total <= kNoAllocScratchBytes) return b;
  return 0;
}

hipError_t awq_noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_awq_search(const void* X, const void* W, int64_t T, int64_t N, int64_t K, int bits,
                             int group_size, bool asymmetric, int n_grid, double* losses, float* best_scale,
                             int32_t* best_index, void* workspace, hipStream_t stream, int max_batch) {
  const AwqLayout L = awq_layout(T, N, K, bits, group_size, asymmetric, max_batch);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  double* m = reinterpret_cast<double*>(ws + L.m);
  float* s = reinterpret_cast<float*>(ws + L.s);
  uint8_t* packed = ws + L.packed;
  uint16_t* scales = reinterpret_cast<uint16_t*>(ws + L.scales);
  uint16_t* zeros = asymmetric ? reinterpret_cast<uint16_t*>(ws + L.zeros) : nullptr;
  float* yref = reinterpret_cast<float*>(ws + L.yref);
  uint16_t* yq = reinterpret_cast<uint16_t*>(ws + L.yq);
  double* partial = reinterpret_cast<double*>(ws + L.partial);
  const uint16_t* X16 = static_cast<const uint16_t*>(X);
  const uint16_t* W16 = static_cast<const uint16_t*>(W);

  const unsigned kblocks = (unsigned)((K + 255) / 256);
  hipLaunchKernelGGL(channel_mean_kernel, dim3((unsigned)((K + kMeanChannels - 1) / kMeanChannels)),
                     dim3(kMeanChannels * kMeanSlices), 0, stream, X16, (int)T, (int)K, m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_dense_ref(X16, W16, T, N, K, yref, stream)) != hipSuccess) return e;
  for (int i0 = 0; i0 < n_grid; i0 += L.batch) {
    const int nb = n_grid - i0 < L.batch ? n_grid - i0 : L.batch;
    for (int j = 0; j < nb; ++j) {
      float* sj = s + (int64_t)j * K;
      hipLaunchKernelGGL(awq_scale_kernel, dim3(kblocks), dim3(256), 0, stream, m, (double)(i0 + j) / n_grid, (int)K,
                         sj);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = launch_quantize_pack(W, sj, N, K, bits, group_size, asymmetric, packed + j * L.packed_bytes,
                                    scales + j * L.sz_elems, zeros ? zeros + j * L.sz_elems : nullptr, stream)) !=
          hipSuccess)
        return e;
    }
    e = L.batch > 1 ? launch_gemm_regb_batched(X, s, K, packed, (int64_t)L.packed_bytes, scales, zeros,
                                               (int64_t)L.sz_elems, T, N, K, group_size, asymmetric, yq,
                                               (int64_t)L.yq_elems, nb, stream)
                    : launch_gemm(X, 0, s, packed, scales, zeros, T, N, K, bits, group_size, asymmetric, yq, stream);
    if (e != hipSuccess) return e;
    for (int j = 0; j < nb; ++j) {
      hipLaunchKernelGGL(sqdiff_partial_kernel, dim3(kPartials), dim3(256), 0, stream, yref,
                         static_cast<const uint16_t*>(yq + j * L.yq_elems), T * N, partial);
      hipLaunchKernelGGL(sqdiff_finish_kernel, dim3(1), dim3(256), 0, stream, partial, losses + i0 + j);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL(awq_select_kernel, dim3(kblocks), dim3(256), 0, stream, losses, n_grid, m, (int)K, best_scale,
                     best_index);
  return hipGetLastError();
}

}  // namespace woq
