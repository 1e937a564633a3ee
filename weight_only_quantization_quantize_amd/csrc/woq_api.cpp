// C ABI of libwoq: argument validation, kernel dispatch and error reporting.
// Declarations and the contract of every entry point are in include/woq.h.
#include "../../include/woq.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <exception>
#include <string>
#include <vector>

#include "woq_internal.h"

namespace woq {
int gemv_max_k();
}

namespace {

thread_local std::string g_last_error;

woq_status fail(woq_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

woq_status fail(woq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

woq_status ok() {
  g_last_error.clear();
  return WOQ_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Checks shared by every entry point that takes a packed matrix.
woq_status check_qparams(int64_t N, int64_t K, int32_t bits, int32_t group_size) {
  if (bits != 3 && bits != 4) return fail(WOQ_ERR_INVALID_ARGUMENT, "bits must be 3 or 4 (got %d)", bits);
  if (N < 1) return fail(WOQ_ERR_INVALID_ARGUMENT, "N must be >= 1 (got %lld)", (long long)N);
  if (K < 32 || K % 32 != 0)
    return fail(WOQ_ERR_INVALID_ARGUMENT, "K must be a positive multiple of 32 (got %lld)", (long long)K);
  if (group_size < 32 || group_size % 32 != 0)
    return fail(WOQ_ERR_INVALID_ARGUMENT, "group_size must be a positive multiple of 32 (got %d)", group_size);
  if (K % group_size != 0)
    return fail(WOQ_ERR_INVALID_ARGUMENT, "K (%lld) must be a multiple of group_size (%d)", (long long)K,
                group_size);
  if (N > INT32_MAX || K > INT32_MAX / 2)
    return fail(WOQ_ERR_UNSUPPORTED, "N or K too large for this library (N=%lld, K=%lld)", (long long)N,
                (long long)K);
  return WOQ_OK;
}

woq_status check_packed_inputs(const void* packed, const void* scales, const void* zeros, int32_t asymmetric) {
  if (!packed || !scales) return fail(WOQ_ERR_INVALID_ARGUMENT, "packed and scales must not be NULL");
  if (!aligned(packed, 16)) return fail(WOQ_ERR_INVALID_ARGUMENT, "packed must be 16-byte aligned");
  if (!aligned(scales, 2)) return fail(WOQ_ERR_INVALID_ARGUMENT, "scales must be 2-byte aligned");
  if (asymmetric && !zeros) return fail(WOQ_ERR_INVALID_ARGUMENT, "zeros must not be NULL when asymmetric");
  if (!asymmetric && zeros) return fail(WOQ_ERR_INVALID_ARGUMENT, "zeros must be NULL when symmetric");
  if (zeros && !aligned(zeros, 2)) return fail(WOQ_ERR_INVALID_ARGUMENT, "zeros must be 2-byte aligned");
  return WOQ_OK;
}

woq_status check_act_scale(const float* act_scale) {
  if (act_scale && !aligned(act_scale, 16))
    return fail(WOQ_ERR_INVALID_ARGUMENT, "act_scale must be 16-byte aligned");
  return WOQ_OK;
}

woq_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(WOQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define WOQ_TRY(expr)                   \
  do {                                  \
    const woq_status st_ = (expr);      \
    if (st_ != WOQ_OK) return st_;      \
  } while (0)

#define WOQ_GUARD_BEGIN try {
#define WOQ_GUARD_END                                                        \
  }                                                                          \
  catch (const std::exception& e) {                                          \
    return fail(WOQ_ERR_INTERNAL, "internal error: %s", e.what());           \
  }                                                                          \
  catch (...) {                                                              \
    return fail(WOQ_ERR_INTERNAL, "internal error: unknown exception");      \
  }

// Arguments of the AWQ search other than its scratch.
woq_status check_awq_args(const void* X, const void* W, int64_t T, int64_t N, int64_t K, int32_t bits,
                          int32_t group_size, int32_t n_grid, const double* losses, const float* best_scale,
                          const int32_t* best_index) {
  WOQ_TRY(check_qparams(N, K, bits, group_size));
  if (T < 1) return fail(WOQ_ERR_INVALID_ARGUMENT, "T must be >= 1 (got %lld)", (long long)T);
  if (T > INT32_MAX / 2 || T * N > (int64_t)1 << 40)
    return fail(WOQ_ERR_UNSUPPORTED, "T x N too large for this library (T=%lld, N=%lld)", (long long)T, (long long)N);
  if (n_grid < 1 || n_grid > 64) return fail(WOQ_ERR_INVALID_ARGUMENT, "n_grid must be in [1, 64] (got %d)", n_grid);
  if (!X || !W) return fail(WOQ_ERR_INVALID_ARGUMENT, "X and W must not be NULL");
  if (!aligned(X, 16) || !aligned(W, 16)) return fail(WOQ_ERR_INVALID_ARGUMENT, "X and W must be 16-byte aligned");
  if (!losses || !aligned(losses, 8)) return fail(WOQ_ERR_INVALID_ARGUMENT, "losses must be non-NULL, 8-byte aligned");
  if (!best_scale || !aligned(best_scale, 16))
    return fail(WOQ_ERR_INVALID_ARGUMENT, "best_scale must be non-NULL, 16-byte aligned");
  if (!best_index || !aligned(best_index, 4))
    return fail(WOQ_ERR_INVALID_ARGUMENT, "best_index must be non-NULL, 4-byte aligned");
  return WOQ_OK;
}

// GPTQ runs 128-column blocks whose groups either split a block evenly or
// cover whole blocks; the factorization uses 64-wide panels.
woq_status check_gptq(int64_t T, int64_t N, int64_t K, int32_t bits, int32_t group_size) {
  WOQ_TRY(check_qparams(N, K, bits, group_size));
  if (T < 1) return fail(WOQ_ERR_INVALID_ARGUMENT, "T must be >= 1 (got %lld)", (long long)T);
  if (K % 128 != 0) return fail(WOQ_ERR_UNSUPPORTED, "gptq needs K %% 128 == 0 (got K=%lld)", (long long)K);
  if (128 % group_size != 0 && group_size % 128 != 0)
    return fail(WOQ_ERR_UNSUPPORTED, "gptq needs group_size dividing 128 or a multiple of 128 (got %d)", group_size);
  if (K > 32768 || T > INT32_MAX || N > ((int64_t)1 << 31))
    return fail(WOQ_ERR_UNSUPPORTED, "gptq sizes too large for this library (T=%lld, N=%lld, K=%lld)", (long long)T,
                (long long)N, (long long)K);
  return WOQ_OK;
}

}  // namespace

extern "C" {

int32_t woq_layout_version(void) { return WOQ_LAYOUT_V2; }

size_t woq_packed_bytes(int64_t N, int64_t K, int32_t bits) {
  if ((bits != 3 && bits != 4) || N < 1 || K < 32 || K % 32 != 0) return 0;
  return (size_t)N * (size_t)K * (size_t)bits / 8;
}

size_t woq_scales_bytes(int64_t N, int64_t K, int32_t group_size) {
  if (N < 1 || K < 1 || group_size < 1 || K % group_size != 0) return 0;
  return (size_t)N * (size_t)(K / group_size) * 2;
}

size_t woq_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t bits, int32_t group_size) {
  if (M < 1 || M > INT32_MAX / 2 || N < 1 || N > INT32_MAX || K < 32 || K % 32 != 0 || K > INT32_MAX / 2 ||
      (bits != 3 && bits != 4) || group_size < 32 || group_size % 32 != 0 || K % group_size != 0)
    return 0;
  return woq::gemm_workspace_bytes(M, N, K, bits, group_size);
}

woq_status woq_quantize_pack(const void* W, const float* act_scale, int64_t N, int64_t K, int32_t bits,
                             int32_t group_size, int32_t asymmetric, void* packed, void* scales, void* zeros,
                             void* stream) {
  WOQ_GUARD_BEGIN
  WOQ_TRY(check_qparams(N, K, bits, group_size));
  if (!W) return fail(WOQ_ERR_INVALID_ARGUMENT, "W must not be NULL");
  if (!aligned(W, 16)) return fail(WOQ_ERR_INVALID_ARGUMENT, "W must be 16-byte aligned");
  WOQ_TRY(check_packed_inputs(packed, scales, zeros, asymmetric));
  WOQ_TRY(check_act_scale(act_scale));
  return from_hip(woq::launch_quantize_pack(W, act_scale, N, K, bits, group_size, asymmetric != 0, packed, scales,
                                            zeros, static_cast<hipStream_t>(stream)),
                  "quantize_pack launch");
  WOQ_GUARD_END
}

woq_status woq_quantize_pack_many(const woq_qmatrix* mats, int32_t count, int32_t bits, int32_t group_size,
                                  int32_t asymmetric, void* stream) {
  WOQ_GUARD_BEGIN
  if (!mats) return fail(WOQ_ERR_INVALID_ARGUMENT, "mats must not be NULL");
  if (count < 1) return fail(WOQ_ERR_INVALID_ARGUMENT, "count must be >= 1 (got %d)", count);
  std::vector<woq::QpMatrix> qm((size_t)count);
  for (int32_t i = 0; i < count; ++i) {
    const woq_qmatrix& m = mats[i];
    woq_status st = check_qparams(m.N, m.K, bits, group_size);
    if (st == WOQ_OK && !m.W) st = fail(WOQ_ERR_INVALID_ARGUMENT, "W must not be NULL");
    if (st == WOQ_OK && !aligned(m.W, 16)) st = fail(WOQ_ERR_INVALID_ARGUMENT, "W must be 16-byte aligned");
    if (st == WOQ_OK) st = check_packed_inputs(m.packed, m.scales, m.zeros, asymmetric);
    if (st == WOQ_OK) st = check_act_scale(m.act_scale);
    if (st != WOQ_OK) return fail(st, "matrix %d: %s", i, g_last_error.c_str());
    qm[(size_t)i] = woq::QpMatrix{m.W, m.act_scale, m.packed, m.scales, m.zeros, m.N, m.K};
  }
  return from_hip(woq::launch_quantize_pack_many(qm.data(), count, bits, group_size, asymmetric != 0,
                                                 static_cast<hipStream_t>(stream)),
                  "quantize_pack_many launch");
  WOQ_GUARD_END
}

woq_status woq_w4a16_gemv(const void* x, int32_t xdtype, const float* act_scale, const void* packed,
                          const void* scales, const void* zeros, int64_t N, int64_t K, int32_t bits,
                          int32_t group_size, int32_t asymmetric, void* y, void* workspace, size_t workspace_bytes,
                          void* stream) {
  WOQ_GUARD_BEGIN
  (void)workspace;
  (void)workspace_bytes;
  WOQ_TRY(check_qparams(N, K, bits, group_size));
  if (xdtype != WOQ_F16 && xdtype != WOQ_BF16)
    return fail(WOQ_ERR_INVALID_ARGUMENT, "xdtype must be WOQ_F16 or WOQ_BF16 (got %d)", xdtype);
  if (!x || !y) return fail(WOQ_ERR_INVALID_ARGUMENT, "x and y must not be NULL");
  if (!aligned(x, 16)) return fail(WOQ_ERR_INVALID_ARGUMENT, "x must be 16-byte aligned");
  if (!aligned(y, 2)) return fail(WOQ_ERR_INVALID_ARGUMENT, "y must be 2-byte aligned");
  WOQ_TRY(check_packed_inputs(packed, scales, zeros, asymmetric));
  WOQ_TRY(check_act_scale(act_scale));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (K <= woq::gemv_max_k())
    return from_hip(woq::launch_gemv(x, xdtype, act_scale, packed, scales, zeros, N, K, bits, group_size,
                                     asymmetric != 0, y, st),
                    "gemv launch");
  return from_hip(woq::launch_gemm(x, xdtype, act_scale, packed, scales, zeros, 1, N, K, bits, group_size,
                                   asymmetric != 0, y, st),
                  "gemv (long K) launch");
  WOQ_GUARD_END
}

woq_status woq_w4a16_gemm(const void* X, int32_t xdtype, const float* act_scale, const void* packed,
                          const void* scales, const void* zeros, int64_t M, int64_t N, int64_t K, int32_t bits,
                          int32_t group_size, int32_t asymmetric, void* Y, void* workspace, size_t workspace_bytes,
                          void* stream) {
  WOQ_GUARD_BEGIN
  WOQ_TRY(check_qparams(N, K, bits, group_size));
  if (M < 1) return fail(WOQ_ERR_INVALID_ARGUMENT, "M must be >= 1 (got %lld)", (long long)M);
  if (workspace && !aligned(workspace, 256))
    return fail(WOQ_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned when given");
  if (M > INT32_MAX / 2) return fail(WOQ_ERR_UNSUPPORTED, "M too large for this library (%lld)", (long long)M);
  if (xdtype != WOQ_F16 && xdtype != WOQ_BF16)
    return fail(WOQ_ERR_INVALID_ARGUMENT, "xdtype must be WOQ_F16 or WOQ_BF16 (got %d)", xdtype);
  if (!X || !Y) return fail(WOQ_ERR_INVALID_ARGUMENT, "X and Y must not be NULL");
  if (!aligned(X, 16)) return fail(WOQ_ERR_INVALID_ARGUMENT, "X must be 16-byte aligned");
  if (!aligned(Y, 2)) return fail(WOQ_ERR_INVALID_ARGUMENT, "Y must be 2-byte aligned");
  WOQ_TRY(check_packed_inputs(packed, scales, zeros, asymmetric));
  WOQ_TRY(check_act_scale(act_scale));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (M == 1 && K <= woq::gemv_max_k())
    return from_hip(woq::launch_gemv(X, xdtype, act_scale, packed, scales, zeros, N, K, bits, group_size,
                                     asymmetric != 0, Y, st),
                    "gemm (M=1) launch");
  return from_hip(woq::launch_gemm_ws(X, xdtype, act_scale, packed, scales, zeros, M, N, K, bits, group_size,
                                      asymmetric != 0, Y, workspace, workspace_bytes, st),
                  "gemm launch");
  WOQ_GUARD_END
}

woq_status woq_dequantize(const void* packed, const void* scales, const void* zeros, int64_t N, int64_t K,
                          int32_t bits, int32_t group_size, int32_t asymmetric, float* out, void* stream) {
  WOQ_GUARD_BEGIN
  WOQ_TRY(check_qparams(N, K, bits, group_size));
  WOQ_TRY(check_packed_inputs(packed, scales, zeros, asymmetric));
  if (!out) return fail(WOQ_ERR_INVALID_ARGUMENT, "out must not be NULL");
  if (!aligned(out, 16)) return fail(WOQ_ERR_INVALID_ARGUMENT, "out must be 16-byte aligned");
  return from_hip(woq::launch_dequantize(packed, scales, zeros, N, K, bits, group_size, asymmetric != 0, out,
                                         static_cast<hipStream_t>(stream)),
                  "dequantize launch");
  WOQ_GUARD_END
}

size_t woq_awq_search_workspace_bytes(int64_t T, int64_t N, int64_t K, int32_t bits, int32_t group_size,
                                      int32_t asymmetric) {
  if (T < 1 || check_qparams(N, K, bits, group_size) != WOQ_OK) return 0;
  return woq::awq_search_workspace_bytes(T, N, K, bits, group_size, asymmetric != 0);
}

woq_status woq_awq_search(const void* X, const void* W, int64_t T, int64_t N, int64_t K, int32_t bits,
                          int32_t group_size, int32_t asymmetric, int32_t n_grid, double* losses, float* best_scale,
                          int32_t* best_index, void* workspace, size_t workspace_bytes, void* stream) {
  WOQ_GUARD_BEGIN
  WOQ_TRY(check_awq_args(X, W, T, N, K, bits, group_size, n_grid, losses, best_scale, best_index));
  const size_t need = woq::awq_search_workspace_bytes(T, N, K, bits, group_size, asymmetric != 0);
  if (!workspace || !aligned(workspace, 256))
    return fail(WOQ_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < need)
    return fail(WOQ_ERR_INVALID_ARGUMENT, "workspace too small (%zu bytes, need %zu)", workspace_bytes, need);
  return from_hip(woq::launch_awq_search(X, W, T, N, K, bits, group_size, asymmetric != 0, n_grid, losses,
                                         best_scale, best_index, workspace, static_cast<hipStream_t>(stream)),
                  "awq_search launch");
  WOQ_GUARD_END
}

woq_status woq_awq_search_noalloc(const void* X, const void* W, int64_t T, int64_t N, int64_t K, int32_t bits,
                                  int32_t group_size, int32_t asymmetric, int32_t n_grid, double* losses,
                                  float* best_scale, int32_t* best_index, void* stream) {
  WOQ_GUARD_BEGIN
  WOQ_TRY(check_awq_args(X, W, T, N, K, bits, group_size, n_grid, losses, best_scale, best_index));
  const int batch = woq::awq_noalloc_batch(T, N, K, bits, group_size, asymmetric != 0);
  if (batch < 1)
    return fail(WOQ_ERR_UNSUPPORTED,
                "awq_search_noalloc: this shape needs more scratch than the static %zu bytes "
                "(woq_awq_search with a workspace of %zu bytes takes it)",
                woq::awq_search_noalloc_max_bytes(),
                woq::awq_search_workspace_bytes(T, N, K, bits, group_size, asymmetric != 0));
  void* scratch = nullptr;
  const hipError_t e = woq::awq_noalloc_scratch(&scratch);
  if (e != hipSuccess) return from_hip(e, "awq_search_noalloc scratch address");
  return from_hip(woq::launch_awq_search(X, W, T, N, K, bits, group_size, asymmetric != 0, n_grid, losses, best_scale,
                                         best_index, scratch, static_cast<hipStream_t>(stream), batch),
                  "awq_search_noalloc launch");
  WOQ_GUARD_END
}

size_t woq_awq_search_noalloc_max_bytes(void) { return woq::awq_search_noalloc_max_bytes(); }

size_t woq_gptq_workspace_bytes(int64_t T, int64_t N, int64_t K, int32_t bits, int32_t group_size) {
  if (check_gptq(T, N, K, bits, group_size) != WOQ_OK) return 0;
  return woq::gptq_workspace_bytes(T, N, K);
}

woq_status woq_gptq_quantize_pack(const void* X, const void* W, int64_t T, int64_t N, int64_t K, int32_t bits,
                                  int32_t group_size, int32_t asymmetric, double damp, void* packed, void* scales,
                                  void* zeros, void* workspace, size_t workspace_bytes, void* stream) {
  WOQ_GUARD_BEGIN
  WOQ_TRY(check_gptq(T, N, K, bits, group_size));
  if (!(damp > 0.0) || !(damp <= 1e6)) return fail(WOQ_ERR_INVALID_ARGUMENT, "damp must be in (0, 1e6] (got %g)", damp);
  if (!X || !W) return fail(WOQ_ERR_INVALID_ARGUMENT, "X and W must not be NULL");
  if (!aligned(X, 16) || !aligned(W, 16)) return fail(WOQ_ERR_INVALID_ARGUMENT, "X and W must be 16-byte aligned");
  if (!packed || !aligned(packed, 16)) return fail(WOQ_ERR_INVALID_ARGUMENT, "packed must be non-NULL, 16-byte aligned");
  if (!scales || !aligned(scales, 2)) return fail(WOQ_ERR_INVALID_ARGUMENT, "scales must be non-NULL, 2-byte aligned");
  if (asymmetric && (!zeros || !aligned(zeros, 2)))
    return fail(WOQ_ERR_INVALID_ARGUMENT, "zeros must be non-NULL and 2-byte aligned when asymmetric");
  if (!asymmetric && zeros) return fail(WOQ_ERR_INVALID_ARGUMENT, "zeros must be NULL when symmetric");
  const size_t need = woq::gptq_workspace_bytes(T, N, K);
  if (!workspace || !aligned(workspace, 256))
    return fail(WOQ_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < need)
    return fail(WOQ_ERR_INVALID_ARGUMENT, "workspace too small (%zu bytes, need %zu)", workspace_bytes, need);
  return from_hip(woq::launch_gptq(X, W, T, N, K, bits, group_size, asymmetric != 0, damp, packed, scales,
                                   zeros, workspace, static_cast<hipStream_t>(stream)),
                  "gptq launch");
  WOQ_GUARD_END
}

woq_status woq_probe_stream_read(const void* p, size_t bytes, int32_t blocks, int32_t threads, int32_t unroll,
                                 void* sink, int32_t store, void* stream) {
  WOQ_GUARD_BEGIN
  if (!p || !aligned(p, 16)) return fail(WOQ_ERR_INVALID_ARGUMENT, "p must be non-NULL and 16-byte aligned");
  if (bytes < 16 || bytes % 16 != 0 || bytes > ((size_t)1 << 40))
    return fail(WOQ_ERR_INVALID_ARGUMENT, "bytes must be a positive multiple of 16 (got %zu)", bytes);
  if (blocks < 1 || blocks > (1 << 20)) return fail(WOQ_ERR_INVALID_ARGUMENT, "blocks must be in [1, 2^20] (got %d)", blocks);
  if (threads < 64 || threads > 1024 || threads % 64 != 0)
    return fail(WOQ_ERR_INVALID_ARGUMENT, "threads must be a multiple of 64 in [64, 1024] (got %d)", threads);
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8)
    return fail(WOQ_ERR_INVALID_ARGUMENT, "unroll must be 1, 2, 4 or 8 (got %d)", unroll);
  if (!sink || !aligned(sink, 4)) return fail(WOQ_ERR_INVALID_ARGUMENT, "sink must be non-NULL and 4-byte aligned");
  return from_hip(woq::launch_stream_read(p, (int64_t)bytes, blocks, threads, unroll, sink, store != 0,
                                          static_cast<hipStream_t>(stream)),
                  "stream_read launch");
  WOQ_GUARD_END
}

woq_status woq_probe_empty(int32_t blocks, int32_t threads, void* stream) {
  WOQ_GUARD_BEGIN
  if (blocks < 1 || blocks > (1 << 20)) return fail(WOQ_ERR_INVALID_ARGUMENT, "blocks must be in [1, 2^20] (got %d)", blocks);
  if (threads < 1 || threads > 1024) return fail(WOQ_ERR_INVALID_ARGUMENT, "threads must be in [1, 1024] (got %d)", threads);
  return from_hip(woq::launch_empty(blocks, threads, static_cast<hipStream_t>(stream)), "empty launch");
  WOQ_GUARD_END
}

woq_status woq_probe_mfma_rate(const void* src, int32_t blocks, int32_t iters, float* sink, int32_t store,
                               void* stream) {
  WOQ_GUARD_BEGIN
  if (!src || !aligned(src, 16)) return fail(WOQ_ERR_INVALID_ARGUMENT, "src must be non-NULL and 16-byte aligned");
  if (blocks < 1 || blocks > (1 << 16)) return fail(WOQ_ERR_INVALID_ARGUMENT, "blocks must be in [1, 65536] (got %d)", blocks);
  if (iters < 1 || iters > (1 << 24)) return fail(WOQ_ERR_INVALID_ARGUMENT, "iters must be in [1, 2^24] (got %d)", iters);
  if (!sink || !aligned(sink, 4)) return fail(WOQ_ERR_INVALID_ARGUMENT, "sink must be non-NULL and 4-byte aligned");
  return from_hip(woq::launch_mfma_rate(src, blocks, iters, sink, store != 0, static_cast<hipStream_t>(stream)),
                  "mfma_rate launch");
  WOQ_GUARD_END
}

woq_status woq_probe_mfma_valu(const void* src, int32_t blocks, int32_t iters, int32_t mfma_per_iter,
                               int32_t valu_per_iter, float* sink, uint64_t* clocks, int32_t store, void* stream) {
  WOQ_GUARD_BEGIN
  if (!src || !aligned(src, 16)) return fail(WOQ_ERR_INVALID_ARGUMENT, "src must be non-NULL and 16-byte aligned");
  if (blocks < 1 || blocks > (1 << 16)) return fail(WOQ_ERR_INVALID_ARGUMENT, "blocks must be in [1, 65536] (got %d)", blocks);
  if (iters < 1 || iters > (1 << 24)) return fail(WOQ_ERR_INVALID_ARGUMENT, "iters must be in [1, 2^24] (got %d)", iters);
  const bool known = (mfma_per_iter == 4 && (valu_per_iter == 0 || valu_per_iter == 16 || valu_per_iter == 32 ||
                                             valu_per_iter == 64)) ||
                     (mfma_per_iter == 0 && (valu_per_iter == 32 || valu_per_iter == 64));
  if (!known)
    return fail(WOQ_ERR_INVALID_ARGUMENT,
                "(mfma_per_iter, valu_per_iter) must be (4, 0|16|32|64) or (0, 32|64) (got (%d, %d))", mfma_per_iter,
                valu_per_iter);
  if (!sink || !aligned(sink, 4)) return fail(WOQ_ERR_INVALID_ARGUMENT, "sink must be non-NULL and 4-byte aligned");
  if (!clocks || !aligned(clocks, 8)) return fail(WOQ_ERR_INVALID_ARGUMENT, "clocks must be non-NULL and 8-byte aligned");
  return from_hip(woq::launch_mfma_valu(src, blocks, iters, mfma_per_iter, valu_per_iter, sink, clocks, store != 0,
                                        static_cast<hipStream_t>(stream)),
                  "mfma_valu launch");
  WOQ_GUARD_END
}

size_t woq_probe_gemv_timeline_words(int64_t N) { return N >= 1 && N <= (INT64_C(1) << 31) ? woq::gemv_timeline_words(N) : 0; }

woq_status woq_probe_gemv_timeline(const void* x, const void* packed, const void* scales, const void* zeros,
                                   int64_t N, void* y, uint64_t* timeline, size_t timeline_words, void* stream) {
  WOQ_GUARD_BEGIN
  if (N < 1 || N > (INT64_C(1) << 31)) return fail(WOQ_ERR_INVALID_ARGUMENT, "N must be in [1, 2^31] (got %lld)", (long long)N);
  if (!x || !aligned(x, 16)) return fail(WOQ_ERR_INVALID_ARGUMENT, "x must be non-NULL and 16-byte aligned");
  if (!packed || !aligned(packed, 16)) return fail(WOQ_ERR_INVALID_ARGUMENT, "packed must be non-NULL and 16-byte aligned");
  if (!scales || !aligned(scales, 2)) return fail(WOQ_ERR_INVALID_ARGUMENT, "scales must be non-NULL and 2-byte aligned");
  if (!zeros || !aligned(zeros, 2)) return fail(WOQ_ERR_INVALID_ARGUMENT, "zeros must be non-NULL and 2-byte aligned");
  if (!y || !aligned(y, 2)) return fail(WOQ_ERR_INVALID_ARGUMENT, "y must be non-NULL and 2-byte aligned");
  if (!timeline || !aligned(timeline, 8)) return fail(WOQ_ERR_INVALID_ARGUMENT, "timeline must be non-NULL and 8-byte aligned");
  const size_t need = woq::gemv_timeline_words(N);
  if (timeline_words < need)
    return fail(WOQ_ERR_INVALID_ARGUMENT, "timeline too small (%zu words, need %zu)", timeline_words, need);
  return from_hip(woq::launch_gemv_timeline(x, packed, scales, zeros, N, y, timeline, static_cast<hipStream_t>(stream)),
                  "gemv_timeline launch");
  WOQ_GUARD_END
}

const char* woq_status_string(woq_status status) {
  switch (status) {
    case WOQ_OK:
      return "WOQ_OK";
    case WOQ_ERR_INVALID_ARGUMENT:
      return "WOQ_ERR_INVALID_ARGUMENT";
    case WOQ_ERR_UNSUPPORTED:
      return "WOQ_ERR_UNSUPPORTED";
    case WOQ_ERR_HIP:
      return "WOQ_ERR_HIP";
    case WOQ_ERR_INTERNAL:
      return "WOQ_ERR_INTERNAL";
  }
  return "WOQ_ERR_UNKNOWN";
}

const char* woq_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
