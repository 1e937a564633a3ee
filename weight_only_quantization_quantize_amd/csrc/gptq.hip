// GPTQ on the GPU, writing layout v2.
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
//   2. Blocked Cholesky M = L L^T (64-wide panels: a one-wave factorization
//      and inversion of the diagonal block, the panel below it multiplied by
//      that inverse's transpose, and a symmetric update of the trailing lower
//      triangle).
//   3. Y = L^-1 by recursive doubling over the diagonal blocks.
//   4. U = J Y J (upper, since J H^-1 J = Y^T Y), written over M.
//   5. Columns in blocks of 128: a workgroup per 64 rows quantizes the block
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

// Orders this wave's LDS accesses for the compiler without waiting for them:
// LDS operations of one wave execute in issue order, so a value one lane
// writes is seen by every lane's later read.  A workgroup barrier would add an
// s_waitcnt lgkmcnt(0) and drain every read in flight.
__device__ inline void wave_sync() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); }

// Diagonal block of panel p (one wave): Cholesky factor L[P, P] in place in
// M (strictly upper part set to 0) and its inverse into Y[P, P].
//  - Factor, right-looking, lane r holding row r in registers: for column j,
//    L[j][j] = sqrt(a[j][j]); L[r][j] = a[r][j] / L[j][j]; then
//    a[r][c] -= L[r][j] L[c][j] for c > j (lanes r < c update entries that
//    are never read), the pivot and the column published through LDS.
//  - Inverse, lane c solving L z = e_c, right-looking over rows with the
//    columns of L read as LDS broadcasts: z_r = s_r * (1 / L[r][r]), then
//    s_r' -= L[r'][r] z_r for r' > r (z_r = 0 for r < c exactly).
__global__ __launch_bounds__(64) void potrf_inv_kernel(double* __restrict__ M, double* __restrict__ Y, int64_t K,
                                                       int p) {
  __shared__ double col[kPanel], rd[kPanel];
  __shared__ double lt[kPanel][kPitch];  // lt[q][r] = L[r][q]
  const int64_t P0 = (int64_t)p * kPanel;
  const int lane = threadIdx.x;
  double a[kPanel];
#pragma unroll
  for (int c = 0; c < kPanel; ++c) a[c] = c <= lane ? M[(P0 + lane) * K + P0 + c] : 0.0;
#pragma unroll
  for (int j = 0; j < kPanel; ++j) {
    if (lane == j) col[j] = __builtin_sqrt(a[j]);
    wave_sync();
    const double d = col[j];
    const double l = lane == j ? d : a[j] / d;
    a[j] = lane >= j ? l : 0.0;
    wave_sync();
    col[lane] = l;
    wave_sync();
#pragma unroll
    for (int c = j + 1; c < kPanel; ++c) a[c] = __builtin_fma(-l, col[c], a[c]);
    wave_sync();
  }
#pragma unroll
  for (int c = 0; c < kPanel; ++c) {
    const double v = c <= lane ? a[c] : 0.0;
    lt[c][lane] = v;
    M[(P0 + lane) * K + P0 + c] = v;
  }
  wave_sync();
  rd[lane] = 1.0 / lt[lane][lane];
  wave_sync();
  double z[kPanel];
#pragma unroll
  for (int r = 0; r < kPanel; ++r) z[r] = r == lane ? 1.0 : 0.0;
#pragma unroll
  for (int r = 0; r < kPanel; ++r) {
    z[r] = z[r] * rd[r];
#pragma unroll
    for (int q = r + 1; q < kPanel; ++q) z[q] = __builtin_fma(-lt[r][q], z[r], z[q]);
  }
#pragma unroll
  for (int r = 0; r < kPanel; ++r) Y[(P0 + r) * K + P0 + lane] = z[r];
}

// Panel below the diagonal block: L[I, P] = A[I, P] L[P, P]^-T as a tile
// product with the inverse from potrf_inv_kernel, block row
// I = p + 1 + blockIdx.x, in place (each workgroup reads its rows completely
// before writing them).
__global__ __launch_bounds__(256) void trsm_panel_kernel(double* __restrict__ M, const double* __restrict__ Y,
                                                         int64_t K, int p) {
  __shared__ double As[kTileK][kPitch], Bs[kTileK][kPitch];
  const int64_t P0 = (int64_t)p * kPanel, I0 = (int64_t)(p + 1 + blockIdx.x) * kPanel;
  double acc[4][4];
  zero_acc(acc);
  tile_product<true, true>([&](int i, int q) { return M[(I0 + i) * K + P0 + q]; },
                           [&](int q, int j) { return Y[(P0 + j) * K + P0 + q]; }, kPanel, acc, As, Bs);
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) M[(I0 + tr + 16 * r) * K + P0 + tc + 16 * c] = acc[r][c];
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

// Y = L^-1 by recursive doubling.  The 64 x 64 diagonal blocks are inverted
// with the factorization (potrf_inv_kernel); then, for s = 64, 128, ... while s < K, each diagonal
// segment [2 s z, min(2 s (z + 1), K)) = [[A, 0], [B, C]] with A of size s and
// C of size sc = min(s, K - 2 s z - s) > 0 (A and C already inverted) gets its
// lower-left block -C^-1 B A^-1, as two batched products through a
// temporary (pair z's s x sc product at offset z s^2; at most s (K - s) <=
// K^2 / 4 doubles).

// Level s, first product: Tmp[p] = B_p A_p^-1 for pair p = blockIdx.z (pair
// origin o = 2 s p; rows past sc and pairs with sc <= 0 return at once):
// B_p = L[o+s .., o ..] (sc x s), A_p^-1 = Y[o .., o ..] (s x s, lower
// triangular, so the inner index starts at the tile's first column).
__global__ __launch_bounds__(256) void pair_left_kernel(const double* __restrict__ M, const double* __restrict__ Y,
                                                        int64_t K, int64_t s, double* __restrict__ Tmp) {
  __shared__ double As[kTileK][kPitch], Bs[kTileK][kPitch];
  const int64_t o = 2 * s * blockIdx.z, r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int64_t sc = K - o - s < s ? K - o - s : s;
  if (r0 >= sc) return;
  double acc[4][4];
  zero_acc(acc);
  tile_product<true, false>([&](int i, int q) { return M[(o + s + r0 + i) * K + o + c0 + q]; },
                            [&](int q, int j) { return Y[(o + c0 + q) * K + o + c0 + j]; }, (int)(s - c0), acc, As,
                            Bs);
  double* T = Tmp + (int64_t)blockIdx.z * s * s;
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) T[(r0 + tr + 16 * r) * s + c0 + tc + 16 * c] = acc[r][c];
}

// Level s, second product: Y[o+s .., o ..] = -C_p^-1 Tmp[p], C_p^-1 =
// Y[o+s .., o+s ..] (lower triangular: the inner index stops after the tile's
// last row).
__global__ __launch_bounds__(256) void pair_right_kernel(double* __restrict__ Y, int64_t K, int64_t s,
                                                         const double* __restrict__ Tmp) {
  __shared__ double As[kTileK][kPitch], Bs[kTileK][kPitch];
  const int64_t o = 2 * s * blockIdx.z, r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int64_t sc = K - o - s < s ? K - o - s : s;
  if (r0 >= sc) return;
  const double* T = Tmp + (int64_t)blockIdx.z * s * s;
  double acc[4][4];
  zero_acc(acc);
  tile_product<true, false>([&](int i, int q) { return Y[(o + s + r0 + i) * K + o + s + q]; },
                            [&](int q, int j) { return T[q * s + c0 + j]; }, (int)(r0 + 64), acc, As, Bs);
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) Y[(o + s + r0 + tr + 16 * r) * K + o + c0 + tc + 16 * c] = -acc[r][c];
}

// Zero fill (the upper blocks of Y are read as zeros by the products).
__global__ __launch_bounds__(256) void zero_kernel(double* __restrict__ p, int64_t count) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < count; e += (int64_t)gridDim.x * 256) p[e] = 0.0;
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

// One 128-column block of 64 rows on eight waves.  Wave v keeps columns
// [16 v, 16 v + 16) of row `lane` in registers; U[block, block] sits in LDS
// (its zeros below the diagonal included).  Column c belongs to wave c / 16,
// which quantizes it for its 64 rows and publishes the scaled errors through
// LDS (double-buffered, one barrier per column); then every wave subtracts
// err * U[c][j] from its 16 columns.  Columns j < c see U[c][j] = 0 and
// column c itself becomes w_hat, neither of which is read again.  Group
// statistics (group size 32 or 64) combine eight per-wave partials in a
// fixed order.  Writes the codes (layout v2), the parameters of the groups
// that start in the block and the scaled errors Et[c][n].
constexpr int kBlockWaves = 8;
constexpr int kOwn = kColBlock / kBlockWaves;

template <int BITS, bool ASYM>
__global__ __launch_bounds__(64 * kBlockWaves) void gptq_block_kernel(
    const double* __restrict__ W64, const double* __restrict__ U, int64_t N, int64_t K, int G, int64_t c0,
    int64_t Npad, uint8_t* __restrict__ packed, uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros,
    double* __restrict__ Et) {
  __shared__ double ub[kColBlock][kColBlock];
  __shared__ double errs[2][64];
  __shared__ float stat[2][kBlockWaves][64];
  __shared__ uint8_t us[kColBlock][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * 64, n = n0 + lane;
  const int64_t nc = n < N ? n : N - 1;
  for (int idx = tid; idx < kColBlock * kColBlock; idx += 64 * kBlockWaves) {
    const int c = idx >> 7, j = idx & (kColBlock - 1);
    ub[c][j] = U[(c0 + c) * K + c0 + j];
  }
  double w[kOwn];
  const double* src = W64 + nc * K + c0 + kOwn * wave;
#pragma unroll
  for (int q = 0; q < kOwn; ++q) w[q] = src[q];
  __syncthreads();

  const int64_t ng = K / G;
  GroupParams<BITS, ASYM> p{};
  if (G >= kColBlock) {
    const int64_t gi = nc * ng + c0 / G;
    p.S16 = scales[gi];
    p.S = half_bits_to_f32(p.S16);
    p.Z = ASYM ? (int)half_bits_to_f32(zeros[gi]) : 1 << (BITS - 1);
    p.zero = p.S == 0.0f;
    set_reciprocal(p);
  }
  for (int c = 0; c < kColBlock; ++c) {
    const int owner = c / kOwn, slot = c % kOwn;
    if (G < kColBlock && c % G == 0) {
      float lo = __builtin_huge_valf(), hi = ASYM ? -__builtin_huge_valf() : 0.0f;
#pragma unroll
      for (int q = 0; q < kOwn; ++q) {
        const int j = kOwn * wave + q;
        if (j >= c && j < c + G) fold_stat<ASYM>((float)w[q], lo, hi);
      }
      stat[0][wave][lane] = lo;
      stat[1][wave][lane] = hi;
      __syncthreads();
      lo = stat[0][0][lane];
      hi = stat[1][0][lane];
#pragma unroll
      for (int v = 1; v < kBlockWaves; ++v) {
        lo = fminf(lo, stat[0][v][lane]);
        hi = fmaxf(hi, stat[1][v][lane]);
      }
      p = group_params<BITS, ASYM>(lo, hi);
      if (wave == owner && n < N) {
        const int64_t gi = n * ng + (c0 + c) / G;
        scales[gi] = p.S16;
        if (ASYM) zeros[gi] = f32_to_half_bits((float)p.Z);
      }
    }
    if (wave == owner) {
      double wc = w[0];
#pragma unroll
      for (int q = 1; q < kOwn; ++q) wc = slot == q ? w[q] : wc;
      const uint32_t u = code_of<BITS, ASYM>((float)wc, p);
      const double what = ((double)(int)u - (double)p.Z) * (double)p.S;
      const double err = (wc - what) / ub[c][c];
      errs[c & 1][lane] = err;
      us[c][lane] = (uint8_t)u;
      Et[(int64_t)c * Npad + n] = err;
    }
    __syncthreads();
    const double err = errs[c & 1][lane];
    const double* urow = &ub[c][kOwn * wave];
#pragma unroll
    for (int q = 0; q < kOwn; ++q) w[q] = __builtin_fma(-err, urow[q], w[q]);
  }
  if (n >= N) return;
  if (wave < kColBlock / 32) {
    uint32_t uc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) uc[i] = us[32 * wave + i][lane];
    store_chunk<BITS>(packed, n, (int)K, (int)(c0 / 32 + wave), uc);
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
  size_t m, y, tmp, w64, et, dead, total;
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
  L.tmp = take(sizeof(double) * K * K / 4);
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
    hipLaunchKernelGGL((gptq_block_kernel<BITS, ASYM>), dim3((unsigned)(npad / 64)), dim3(64 * kBlockWaves), 0, stream, W64, U, N, K,
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
  double* Tmp = reinterpret_cast<double*>(ws + L.tmp);
  double* W64 = reinterpret_cast<double*>(ws + L.w64);
  double* Et = reinterpret_cast<double*>(ws + L.et);
  uint8_t* dead = ws + L.dead;
  const int nb = (int)(K / kPanel);

  hipLaunchKernelGGL(hessian_kernel, dim3(nb, nb), dim3(256), 0, stream, static_cast<const uint16_t*>(X), T, K, M);
  hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(256), 0, stream, M, K, damp, dead);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned fill_blocks = 2048;
  hipLaunchKernelGGL(zero_kernel, dim3(fill_blocks), dim3(256), 0, stream, Y, K * K);
  for (int p = 0; p < nb; ++p) {
    hipLaunchKernelGGL(potrf_inv_kernel, dim3(1), dim3(64), 0, stream, M, Y, K, p);
    const int m = nb - 1 - p;
    if (m > 0) {
      hipLaunchKernelGGL(trsm_panel_kernel, dim3(m), dim3(256), 0, stream, M, Y, K, p);
      hipLaunchKernelGGL(syrk_trailing_kernel, dim3(m, m), dim3(256), 0, stream, M, K, p);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  for (int64_t s = kPanel; s < K; s *= 2) {
    const unsigned t = (unsigned)(s / 64), pairs = (unsigned)((K + 2 * s - 1) / (2 * s));
    hipLaunchKernelGGL(pair_left_kernel, dim3(t, t, pairs), dim3(256), 0, stream, M, Y, K, s, Tmp);
    hipLaunchKernelGGL(pair_right_kernel, dim3(t, t, pairs), dim3(256), 0, stream, Y, K, s, Tmp);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
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
