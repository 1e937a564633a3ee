// GPTQ on the GPU, writing layout v1.
//
// What is computed ("CMU 11-868 L19-L20 Model Quantization", section "The
// algorithm in four steps"; the layer-wise objective of "Quantising Large
// Language Models for Efficient Inference", section "Post-training methods
// for 4-bit weights"):
//
//   H = 2 X^T X over the calibration tokens; an input channel whose diagonal
//   is 0 never fires: its diagonal becomes 1 and its weights 0; then
//   H += damp * mean(diag H) * I.  U is the upper triangular factor with
//   U^T U = H^-1.  Column by column, k = 0 .. K-1: quantize column k with the
//   group's parameters (taken from the group's current weights when its
//   first column is reached), err = (w - w_hat) / U[k, k], and every later
//   column j loses err * U[k, j].
//
// How it runs: everything in fp64 except the rounding decisions, which are
// taken on the fp32 value of the current weight by the same rules as
// quantize_pack.
//   1. M = J H J (J reverses the channel order), the lower triangle from a
//      tiled fp64 product over the tokens; damping and dead channels on its
//      diagonal.
//   2. Blocked Cholesky M = L L^T (64-wide panels: a one-workgroup diagonal
//      factorization, a triangular solve of the panel below it and a
//      symmetric update of the trailing lower triangle).
//   3. Y = L^-1 by block rows (each block a product over the blocks already
//      inverted, then a solve with the diagonal block).
//   4. U = J Y J (upper, since J H^-1 J = Y^T Y), written over M.
//   5. Columns in blocks of 128: one wave per 64 rows quantizes the block
//      column by column in LDS, applying the updates inside the block at once
//      and saving the scaled errors E; then one tiled product applies
//      W[:, later] -= E U[block, later] to every later column.
// Step 5's deferred update reorders the sums of the column-by-column form
// without changing what it computes.
#include "rtn_rules.h"
#include "woq_internal.h"

namespace woq {
namespace {

constexpr int kPanel = 64;   // Cholesky / inverse block
constexpr int kColBlock = 128;  // GPTQ column block
constexpr int kTileK = 16;   // inner-dimension step of the fp64 tile product
constexpr int kPitch = 65;   // LDS pitch (doubles) of 64-wide fp64 tiles

// 64 x 64 fp64 tile product acc += A B over P inner steps on 256 threads.
// Thread (tr = tid / 16, tc = tid % 16) owns rows tr + 16 a and columns
// tc + 16 b (a, b = 0..3).  fa(i, p) and fb(p, j) return the operands (0 past
// their ends); A_PFAST / B_PFAST say which index is contiguous in memory so
// that the loads of one wave are coalesced.
template <bool A_PFAST, bool B_PFAST, class FA, class FB>
__device__ inline void tile_product(FA fa, FB fb, int P, double (&acc)[4][4], double (*As)[kPitch],
                                    double (*Bs)[kPitch]) {
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
  for (int p0 = 0; p0 < P; p0 += kTileK) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e;
      const int ai = A_PFAST ? idx >> 4 : idx & 63, ap = A_PFAST ? idx & 15 : idx >> 6;
      const int bj = B_PFAST ? idx >> 4 : idx & 63, bp = B_PFAST ? idx & 15 : idx >> 6;
      As[ap][ai] = p0 + ap < P ? fa(ai, p0 + ap) : 0.0;
      Bs[bp][bj] = p0 + bp < P ? fb(p0 + bp, bj) : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int p = 0; p < kTileK; ++p) {
      double a[4], b[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        a[r] = As[p][tr + 16 * r];
        b[r] = Bs[p][tc + 16 * r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = __builtin_fma(a[r], b[c], acc[r][c]);
    }
    __syncthreads();
  }
}

__device__ inline void zero_acc(double (&acc)[4][4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.0;
}

// M[i][j] = 2 sum_t x[t, K-1-i] x[t, K-1-j] for the lower blocks (bi >= bj).
__global__ __launch_bounds__(256) void hessian_kernel(const uint16_t* __restrict__ X, int64_t T, int64_t K,
                                                      double* __restrict__ M) {
  const int bi = blockIdx.y, bj = blockIdx.x;
  if (bj > bi) return;
  __shared__ double As[kTileK][kPitch], Bs[kTileK][kPitch];
  const int64_t ci = K - 1 - (int64_t)bi * kPanel, cj = K - 1 - (int64_t)bj * kPanel;
  double acc[4][4];
  zero_acc(acc);
  tile_product<false, false>(
      [&](int i, int t) { return (double)half_bits_to_f32(X[(int64_t)t * K + ci - i]); },
      [&](int t, int j) { return (double)half_bits_to_f32(X[(int64_t)t * K + cj - j]); }, (int)T, acc, As, Bs);
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      M[((int64_t)bi * kPanel + tr + 16 * r) * K + (int64_t)bj * kPanel + tc + 16 * c] = 2.0 * acc[r][c];
}

// Dead channels and damping on the diagonal of M (one workgroup):
// dead[k] = (H[k, k] == 0); H[k, k] := 1 there; lambda = damp * mean(diag H);
// diag += lambda.  The sum runs in a fixed order.
__global__ __launch_bounds__(256) void damp_kernel(double* __restrict__ M, int64_t K, double damp,
                                                   uint8_t* __restrict__ dead) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < K; i += 256) {
    const double d = M[i * K + i];
    acc += d == 0.0 ? 1.0 : d;
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  const double lambda = damp * (red[0] / (double)K);
  for (int64_t i = threadIdx.x; i < K; i += 256) {
    const double d = M[i * K + i];
    dead[K - 1 - i] = d == 0.0;
    M[i * K + i] = (d == 0.0 ? 1.0 : d) + lambda;
  }
}

// Cholesky of the diagonal block of panel p, in LDS, in place in M (lower
// triangle; the strictly upper part of the block is set to 0).
__global__ __launch_bounds__(256) void potrf_diag_kernel(double* __restrict__ M, int64_t K, int p) {
  __shared__ double a[kPanel][kPitch];
  const int64_t P0 = (int64_t)p * kPanel;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < kPanel * kPanel; idx += 256) {
    const int r = idx >> 6, c = idx & 63;
    a[r][c] = c <= r ? M[(P0 + r) * K + P0 + c] : 0.0;
  }
  __syncthreads();
  for (int j = 0; j < kPanel; ++j) {
    if (tid == 0) a[j][j] = __builtin_sqrt(a[j][j]);
    __syncthreads();
    if (tid > j && tid < kPanel) a[tid][j] /= a[j][j];
    __syncthreads();
    const int m = kPanel - 1 - j;
    for (int idx = tid; idx < m * m; idx += 256) {
      const int r = j + 1 + idx / m, c = j + 1 + idx % m;
      if (c <= r) a[r][c] = __builtin_fma(-a[r][j], a[c][j], a[r][c]);
    }
    __syncthreads();
  }
  for (int idx = tid; idx < kPanel * kPanel; idx += 256) {
    const int r = idx >> 6, c = idx & 63;
    M[(P0 + r) * K + P0 + c] = a[r][c];
  }
}

// Panel below the diagonal block: L[I, P] = A[I, P] L[P, P]^-T, block row
// I = p + 1 + blockIdx.x, one lane per row.
__global__ __launch_bounds__(64) void trsm_panel_kernel(double* __restrict__ M, int64_t K, int p) {
  __shared__ double l[kPanel][kPitch], v[kPanel][kPitch];
  const int64_t P0 = (int64_t)p * kPanel, I0 = (int64_t)(p + 1 + blockIdx.x) * kPanel;
  const int lane = threadIdx.x;
  for (int r = 0; r < kPanel; ++r) {
    l[r][lane] = M[(P0 + r) * K + P0 + lane];
    v[lane][r] = M[(I0 + r) * K + P0 + lane];
  }
  __syncthreads();
  for (int c = 0; c < kPanel; ++c) {
    double s = v[c][lane];
    for (int q = 0; q < c; ++q) s = __builtin_fma(-v[q][lane], l[c][q], s);
    v[c][lane] = s / l[c][c];
  }
  __syncthreads();
  for (int r = 0; r < kPanel; ++r) M[(I0 + r) * K + P0 + lane] = v[lane][r];
}

// Trailing update of the lower blocks (I, J), p < J <= I:
// A[I, J] -= L[I, P] L[J, P]^T.
__global__ __launch_bounds__(256) void syrk_trailing_kernel(double* __restrict__ M, int64_t K, int p) {
  const int bi = p + 1 + blockIdx.y, bj = p + 1 + blockIdx.x;
  if (bj > bi) return;
  __shared__ double As[kTileK][kPitch], Bs[kTileK][kPitch];
  const int64_t P0 = (int64_t)p * kPanel, I0 = (int64_t)bi * kPanel, J0 = (int64_t)bj * kPanel;
  double acc[4][4];
  zero_acc(acc);
  tile_product<true, true>([&](int i, int q) { return M[(I0 + i) * K + P0 + q]; },
                           [&](int q, int j) { return M[(J0 + j) * K + P0 + q]; }, kPanel, acc, As, Bs);
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      double* dst = &M[(I0 + tr + 16 * r) * K + J0 + tc + 16 * c];
      *dst -= acc[r][c];
    }
}

// Block row i of Y = L^-1: for block column j = blockIdx.x <= i,
// R = (j == i ? I : -sum_{m=j}^{i-1} L[i, m] Y[m, j]) and Y[i, j] = L[i, i]^-1 R.
__global__ __launch_bounds__(256) void trtri_row_kernel(const double* __restrict__ M, double* __restrict__ Y,
                                                        int64_t K, int i) {
  __shared__ double As[kTileK][kPitch], Bs[kTileK][kPitch];
  __shared__ double l[kPanel][kPitch], rs[kPanel][kPitch];
  const int j = blockIdx.x;
  const int64_t I0 = (int64_t)i * kPanel, J0 = (int64_t)j * kPanel;
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
  double acc[4][4];
  zero_acc(acc);
  if (j < i)
    tile_product<true, false>([&](int r, int q) { return M[(I0 + r) * K + J0 + q]; },
                              [&](int q, int c) { return Y[(J0 + q) * K + J0 + c]; }, (i - j) * kPanel, acc, As, Bs);
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int rr = tr + 16 * r, cc = tc + 16 * c;
      rs[rr][cc] = j == i ? (rr == cc ? 1.0 : 0.0) : -acc[r][c];
    }
  for (int idx = tid; idx < kPanel * kPanel; idx += 256) {
    const int r = idx >> 6, c = idx & 63;
    l[r][c] = M[(I0 + r) * K + I0 + c];
  }
  __syncthreads();
  if (tid < kPanel) {
    const int c = tid;
    for (int r = 0; r < kPanel; ++r) {
      double s = rs[r][c];
      for (int q = 0; q < r; ++q) s = __builtin_fma(-l[r][q], rs[q][c], s);
      rs[r][c] = s / l[r][r];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < kPanel * kPanel; idx += 256) {
    const int r = idx >> 6, c = idx & 63;
    Y[(I0 + r) * K + J0 + c] = rs[r][c];
  }
}

// U[a][b] = Y[K-1-a][K-1-b] for a <= b, 0 below the diagonal.
__global__ __launch_bounds__(256) void reverse_factor_kernel(const double* __restrict__ Y, int64_t K,
                                                             double* __restrict__ U) {
  const int64_t total = K * K;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t a = e / K, b = e - a * K;
    U[e] = a <= b ? Y[(K - 1 - a) * K + (K - 1 - b)] : 0.0;
  }
}

// Working copy of the weights in fp64, dead channels zeroed.
__global__ __launch_bounds__(256) void init_weights_kernel(const uint16_t* __restrict__ W, const uint8_t* __restrict__ dead,
                                                           int64_t N, int64_t K, double* __restrict__ W64) {
  const int64_t total = N * K;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t k = e % K;
    W64[e] = dead[k] ? 0.0 : (double)half_bits_to_f32(W[e]);
  }
}

// Statistic of one group of a row from its current fp32 values (symmetric:
// hi = max|w|; asymmetric: lo = min, hi = max), as quantize_pack takes it.
template <bool ASYM>
__device__ inline void fold_stat(float w, float& lo, float& hi) {
  if (ASYM) {
    lo = fminf(lo, w);
    hi = fmaxf(hi, w);
  } else {
    hi = fmaxf(hi, fabsf(w));
  }
}

// Parameters of groups that span whole 128-column blocks (group_size a
// multiple of 128), from the current weights at the group's first column:
// one wave per row.
template <int BITS, bool ASYM>
__global__ __launch_bounds__(256) void wide_group_params_kernel(const double* __restrict__ W64, int64_t N, int64_t K,
                                                                int G, int64_t c0, uint16_t* __restrict__ scales,
                                                                uint16_t* __restrict__ zeros) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const double* row = W64 + n * K + c0;
  float lo = (float)row[0], hi = ASYM ? lo : 0.0f;
  for (int c = lane; c < G; c += 64) fold_stat<ASYM>((float)row[c], lo, hi);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, off));
    hi = fmaxf(hi, __shfl_xor(hi, off));
  }
  if (lane == 0) {
    const GroupParams<BITS, ASYM> p = group_params<BITS, ASYM>(lo, hi);
    const int64_t gi = n * (K / G) + c0 / G;
    scales[gi] = p.S16;
    if (ASYM) zeros[gi] = f32_to_half_bits((float)p.Z);
  }
}

// One 128-column block of 64 rows, one wave, one lane per row.  The rows'
// block values live in LDS as w[c][lane]; U[block, block] is read with
// wave-uniform addresses.  Writes the codes (layout v1), the parameters of
// the groups that start in the block (group_size 32 or 64 or 128) and the
// scaled errors Et[c][n].
template <int BITS, bool ASYM>
__global__ __launch_bounds__(64) void gptq_block_kernel(const double* __restrict__ W64, const double* __restrict__ U,
                                                        int64_t N, int64_t K, int G, int64_t c0, int64_t Npad,
                                                        uint8_t* __restrict__ packed, uint16_t* __restrict__ scales,
                                                        uint16_t* __restrict__ zeros, double* __restrict__ Et) {
  __shared__ double w[kColBlock][kPitch];
  __shared__ uint8_t us[kColBlock][64];
  const int lane = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * 64, n = n0 + lane;
  for (int r = 0; r < 64; ++r) {
    const int64_t nr = n0 + r < N ? n0 + r : N - 1;
    w[lane][r] = W64[nr * K + c0 + lane];
    w[lane + 64][r] = W64[nr * K + c0 + lane + 64];
  }
  __syncthreads();
  const int64_t ng = K / G;
  const int64_t nc = n < N ? n : N - 1;
  GroupParams<BITS, ASYM> p{};
  if (G >= kColBlock) {
    const int64_t gi = nc * ng + c0 / G;
    p.S16 = scales[gi];
    p.S = half_bits_to_f32(p.S16);
    p.Z = ASYM ? (int)half_bits_to_f32(zeros[gi]) : 1 << (BITS - 1);
    p.zero = p.S == 0.0f;
  }
  const double* Ub = U + c0 * K + c0;
  for (int c = 0; c < kColBlock; ++c) {
    if (G < kColBlock && c % G == 0) {
      float lo = (float)w[c][lane], hi = ASYM ? lo : 0.0f;
      for (int q = 0; q < G; ++q) fold_stat<ASYM>((float)w[c + q][lane], lo, hi);
      p = group_params<BITS, ASYM>(lo, hi);
      if (n < N) {
        const int64_t gi = n * ng + (c0 + c) / G;
        scales[gi] = p.S16;
        if (ASYM) zeros[gi] = f32_to_half_bits((float)p.Z);
      }
    }
    const double wc = w[c][lane];
    const uint32_t u = code_of<BITS, ASYM>((float)wc, p);
    us[c][lane] = (uint8_t)u;
    const double what = ((double)(int)u - (double)p.Z) * (double)p.S;
    const double err = (wc - what) / Ub[(int64_t)c * K + c];
    Et[(int64_t)c * Npad + n] = err;
    for (int j = c + 1; j < kColBlock; ++j) w[j][lane] = __builtin_fma(-err, Ub[(int64_t)c * K + j], w[j][lane]);
  }
  if (n >= N) return;
#pragma unroll
  for (int kc = 0; kc < kColBlock / 32; ++kc) {
    uint32_t u[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) u[i] = us[32 * kc + i][lane];
    store_chunk<BITS>(packed, n, (int)K, (int)(c0 / 32 + kc), u);
  }
}

// Deferred update of every later column: W[n][c] -= sum_q Et[q][n] U[c0 + q][c]
// for c >= c0 + 128; a 64 x 64 tile per workgroup.
__global__ __launch_bounds__(256) void gptq_update_kernel(double* __restrict__ W64, const double* __restrict__ U,
                                                          const double* __restrict__ Et, int64_t N, int64_t K,
                                                          int64_t c0, int64_t Npad) {
  __shared__ double As[kTileK][kPitch], Bs[kTileK][kPitch];
  const int64_t n0 = (int64_t)blockIdx.x * 64, j0 = c0 + kColBlock + (int64_t)blockIdx.y * 64;
  double acc[4][4];
  zero_acc(acc);
  tile_product<false, false>([&](int i, int q) { return Et[(int64_t)q * Npad + n0 + i]; },
                             [&](int q, int j) { return U[(c0 + q) * K + j0 + j]; }, kColBlock, acc, As, Bs);
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t n = n0 + tr + 16 * r;
    if (n >= N) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      double* dst = &W64[n * K + j0 + tc + 16 * c];
      *dst -= acc[r][c];
    }
  }
}

constexpr size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct GptqLayout {
  size_t m, y, w64, et, dead, total;
};

GptqLayout gptq_layout(int64_t N, int64_t K) {
  GptqLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  const size_t npad = (size_t)((N + 63) / 64) * 64;
  L.m = take(sizeof(double) * K * K);
  L.y = take(sizeof(double) * K * K);
  L.w64 = take(sizeof(double) * N * K);
  L.et = take(sizeof(double) * kColBlock * npad);
  L.dead = take((size_t)K);
  L.total = off;
  return L;
}

template <int BITS, bool ASYM>
hipError_t run_columns(const double* U, double* W64, double* Et, int64_t N, int64_t K, int G, uint8_t* packed,
                       uint16_t* scales, uint16_t* zeros, hipStream_t stream) {
  const int64_t npad = (N + 63) / 64 * 64;
  for (int64_t c0 = 0; c0 < K; c0 += kColBlock) {
    if (G >= kColBlock && c0 % G == 0)
      hipLaunchKernelGGL((wide_group_params_kernel<BITS, ASYM>), dim3((unsigned)((N + 3) / 4)), dim3(256), 0, stream,
                         W64, N, K, G, c0, scales, zeros);
    hipLaunchKernelGGL((gptq_block_kernel<BITS, ASYM>), dim3((unsigned)(npad / 64)), dim3(64), 0, stream, W64, U, N, K,
                       G, c0, npad, packed, scales, zeros, Et);
    if (c0 + kColBlock < K)
      hipLaunchKernelGGL(gptq_update_kernel, dim3((unsigned)(npad / 64), (unsigned)((K - c0 - kColBlock) / 64)),
                         dim3(256), 0, stream, W64, U, Et, N, K, c0, npad);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t gptq_workspace_bytes(int64_t T, int64_t N, int64_t K) {
  (void)T;
  return gptq_layout(N, K).total;
}

hipError_t launch_gptq(const void* X, const void* W, int64_t T, int64_t N, int64_t K, int bits, int group_size,
                       bool asymmetric, double damp, void* packed, void* scales, void* zeros, void* workspace,
                       hipStream_t stream) {
  const GptqLayout L = gptq_layout(N, K);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  double* M = reinterpret_cast<double*>(ws + L.m);
  double* Y = reinterpret_cast<double*>(ws + L.y);
  double* W64 = reinterpret_cast<double*>(ws + L.w64);
  double* Et = reinterpret_cast<double*>(ws + L.et);
  uint8_t* dead = ws + L.dead;
  const int nb = (int)(K / kPanel);

  hipLaunchKernelGGL(hessian_kernel, dim3(nb, nb), dim3(256), 0, stream, static_cast<const uint16_t*>(X), T, K, M);
  hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(256), 0, stream, M, K, damp, dead);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int p = 0; p < nb; ++p) {
    hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(256), 0, stream, M, K, p);
    const int m = nb - 1 - p;
    if (m > 0) {
      hipLaunchKernelGGL(trsm_panel_kernel, dim3(m), dim3(64), 0, stream, M, K, p);
      hipLaunchKernelGGL(syrk_trailing_kernel, dim3(m, m), dim3(256), 0, stream, M, K, p);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  for (int i = 0; i < nb; ++i) {
    hipLaunchKernelGGL(trtri_row_kernel, dim3(i + 1), dim3(256), 0, stream, M, Y, K, i);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const unsigned fill_blocks = 2048;
  hipLaunchKernelGGL(reverse_factor_kernel, dim3(fill_blocks), dim3(256), 0, stream, Y, K, M);
  hipLaunchKernelGGL(init_weights_kernel, dim3(fill_blocks), dim3(256), 0, stream, static_cast<const uint16_t*>(W),
                     dead, N, K, W64);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  uint8_t* pk = static_cast<uint8_t*>(packed);
  uint16_t* sc = static_cast<uint16_t*>(scales);
  uint16_t* zr = static_cast<uint16_t*>(zeros);
  if (bits == 4)
    return asymmetric ? run_columns<4, true>(M, W64, Et, N, K, group_size, pk, sc, zr, stream)
                      : run_columns<4, false>(M, W64, Et, N, K, group_size, pk, sc, zr, stream);
  return asymmetric ? run_columns<3, true>(M, W64, Et, N, K, group_size, pk, sc, zr, stream)
                    : run_columns<3, false>(M, W64, Et, N, K, group_size, pk, sc, zr, stream);
}

}  // namespace woq
