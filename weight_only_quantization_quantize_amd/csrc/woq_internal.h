// Internal interface between the C ABI layer (woq_api.cpp) and the kernel
// translation units.  Every launcher assumes its arguments were validated by
// the ABI layer and returns the HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace woq {

// Quantize + pack (one thread per 32-weight chunk; groups reduced across the
// chunk threads of the group).
hipError_t launch_quantize_pack(const void* W, const float* act_scale, int64_t N, int64_t K, int bits,
                                int group_size, bool asymmetric, void* packed, void* scales, void* zeros,
                                hipStream_t stream);

// Several matrices sharing bits, group size and symmetry: up to kQpManyMax
// per launch when the group size suits the chunk-team kernel (G / 32 divides
// 64), otherwise one launch per matrix.
constexpr int kQpManyMax = 32;
struct QpMatrix {
  const void* W;
  const float* s;
  void* packed;
  void* scales;
  void* zeros;
  int64_t N, K;
};
bool quantize_pack_many_batched(int group_size);
hipError_t launch_quantize_pack_many(const QpMatrix* mats, int count, int bits, int group_size, bool asymmetric,
                                     hipStream_t stream);

// M = 1 GEMV.  xdtype: 0 = fp16, 1 = bf16.
hipError_t launch_gemv(const void* x, int xdtype, const float* act_scale, const void* packed,
                       const void* scales, const void* zeros, int64_t N, int64_t K, int bits,
                       int group_size, bool asymmetric, void* y, hipStream_t stream);

// M >= 1 GEMM.
hipError_t launch_gemm(const void* X, int xdtype, const float* act_scale, const void* packed,
                       const void* scales, const void* zeros, int64_t M, int64_t N, int64_t K, int bits,
                       int group_size, bool asymmetric, void* Y, hipStream_t stream);

// launch_gemm with the caller's workspace: bf16 X at shapes where
// gemm_workspace_bytes is non-zero runs on the fp16 register-B kernel
// through an exact per-row power-of-two rescale (row scales in the
// workspace) when the workspace is given and large enough.
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int bits, int group_size);
hipError_t launch_gemm_ws(const void* X, int xdtype, const float* act_scale, const void* packed,
                          const void* scales, const void* zeros, int64_t M, int64_t N, int64_t K, int bits,
                          int group_size, bool asymmetric, void* Y, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

// Whether launch_gemm takes the register-B kernel for this shape.
bool gemm_uses_regb(int64_t M, int64_t N, int64_t K, int bits, int xdtype);

// Large-M GEMM: LDS-staged 256 x 256 tiles on 32x32x16 MFMA (bf16, 3-bit,
// and fp16 shapes whose tiles fill the chip).
hipError_t launch_gemm_lds(const void* X, int xdtype, const float* act_scale, const void* packed,
                           const void* scales, const void* zeros, int64_t M, int64_t N, int64_t K, int bits,
                           int group_size, bool asymmetric, void* Y, hipStream_t stream);

// Large-M GEMM for fp16 activations and 4-bit codes (K % 64 == 0): 128 x 256
// tiles, weights decoded straight into MFMA operand registers.
hipError_t launch_gemm_regb(const void* X, const float* act_scale, const void* packed, const void* scales,
                            const void* zeros, int64_t M, int64_t N, int64_t K, int group_size, bool asymmetric,
                            void* Y, hipStream_t stream);
// The same kernel for bf16 Y: X16 is the fp16 copy of bf16 X with row m
// multiplied by f_m (and by the activation scale's reciprocal, if any);
// row_scales holds f_m (M floats) then 1 / f_m, which the epilogue applies.
hipError_t launch_gemm_regb_bf16(const void* X16, const void* packed, const void* scales, const void* zeros,
                                 int64_t M, int64_t N, int64_t K, int group_size, bool asymmetric, void* Y,
                                 const float* row_scales, hipStream_t stream);
// The same for `batch` products over one X: entry b uses act_scale + b
// s_stride, packed + b packed_stride (bytes), scales / zeros + b sz_stride
// and writes Y + b y_stride (elements); one launch fills the chip where one
// product's tiles would not.
// Mid-M GEMM (fp16 X, 4-bit codes, K % 64 == 0): 64 x 128 tiles, K split
// between two halves of the workgroup that meet in LDS.
hipError_t launch_gemm_mid(const void* X, const float* act_scale, const void* packed, const void* scales,
                           const void* zeros, int64_t M, int64_t N, int64_t K, int group_size, bool asymmetric,
                           void* Y, hipStream_t stream);
// The same kernel for bf16 Y on the rescaled fp16 copy X16 (as for
// launch_gemm_regb_bf16).
hipError_t launch_gemm_mid_rescaled_bf16(const void* X16, const void* packed, const void* scales, const void* zeros,
                                         int64_t M, int64_t N, int64_t K, int group_size, bool asymmetric, void* Y,
                                         const float* row_scales, hipStream_t stream);
bool gemm_uses_mid(int64_t M, int64_t N, int64_t K, int bits, int xdtype, bool skinny_ok);
// Mid-M GEMM for bf16 X and 4-bit codes (K % 64 == 0, G a power of two >= 64,
// no AWQ scale): the same tiles with the weights kept exact as 128 + u and the
// scale applied per group in fp32.
bool gemm_mid_bf16_supported(int64_t K, int group_size);
hipError_t launch_gemm_mid_bf16(const void* X, const void* packed, const void* scales, const void* zeros, int64_t M,
                                int64_t N, int64_t K, int group_size, bool asymmetric, void* Y, hipStream_t stream);
hipError_t launch_gemm_regb_batched(const void* X, const float* act_scale, int64_t s_stride, const void* packed,
                                    int64_t packed_stride, const void* scales, const void* zeros, int64_t sz_stride,
                                    int64_t M, int64_t N, int64_t K, int group_size, bool asymmetric, void* Y,
                                    int64_t y_stride, int batch, hipStream_t stream);

// Small-batch GEMM (2 <= M <= 64, 4-bit, group 128, K = 2048 * {1, 2, 4}):
// 16 X rows stay in registers while 16-column tiles of codes stream past.
bool gemm_skinny_supported(int64_t M, int64_t N, int64_t K, int xdtype, bool act_scale, int bits, int group_size,
                           const void* scales, const void* zeros);
hipError_t launch_gemm_skinny(const void* X, int xdtype, const float* act_scale, const void* packed,
                              const void* scales, const void* zeros, int64_t M, int64_t N, int64_t K, bool asymmetric,
                              void* Y, hipStream_t stream);

// AWQ exponent search (scratch in the caller's workspace).
size_t awq_search_workspace_bytes(int64_t T, int64_t N, int64_t K, int bits, int group_size, bool asymmetric);
// max_batch caps the exponents per batched GEMM launch (and with it the
// workspace layout); it changes no output.
hipError_t launch_awq_search(const void* X, const void* W, int64_t T, int64_t N, int64_t K, int bits,
                             int group_size, bool asymmetric, int n_grid, double* losses, float* best_scale,
                             int32_t* best_index, void* workspace, hipStream_t stream, int max_batch = 8);
// The allocation-free search: its scratch is a static device array of
// awq_search_noalloc_max_bytes() bytes; awq_noalloc_batch gives the batch
// that fits it (0: the shape does not fit); awq_noalloc_scratch the array's
// address on the current device.
size_t awq_search_noalloc_max_bytes();
int awq_noalloc_batch(int64_t T, int64_t N, int64_t K, int bits, int group_size, bool asymmetric);
hipError_t awq_noalloc_scratch(void** ptr);

// Y[m, n] = sum_k A[m, k] B[n, k] in fp32 for fp16 A [M, K], B [N, K]
// (K % 16 == 0): the dense MFMA product the AWQ search uses for its
// reference output.
hipError_t launch_dense_ref(const void* A, const void* B, int64_t M, int64_t N, int64_t K, float* Y,
                            hipStream_t stream);

// GPTQ into layout v2 (scratch in the caller's workspace).
size_t gptq_workspace_bytes(int64_t T, int64_t N, int64_t K);
hipError_t launch_gptq(const void* X, const void* W, int64_t T, int64_t N, int64_t K, int bits, int group_size,
                       bool asymmetric, double damp, void* packed, void* scales, void* zeros, void* workspace,
                       hipStream_t stream);

// Measurement aids (no quantization): a read-only stream over `bytes` bytes
// with a given launch shape, an empty kernel, and back-to-back fp16 MFMAs.
hipError_t launch_stream_read(const void* p, int64_t bytes, int blocks, int threads, int unroll, void* sink,
                              int store, hipStream_t stream);
hipError_t launch_empty(int blocks, int threads, hipStream_t stream);
hipError_t launch_mfma_rate(const void* src, int blocks, int iters, float* sink, int store, hipStream_t stream);
size_t gemv_timeline_words(int64_t N);
hipError_t launch_gemv_timeline(const void* x, const void* packed, const void* scales, const void* zeros, int64_t N,
                                void* y, uint64_t* tl, hipStream_t stream);
hipError_t launch_mfma_valu(const void* src, int blocks, int iters, int mfma_per_iter, int valu_per_iter, float* sink,
                            uint64_t* clocks, int store, hipStream_t stream);

// Dequantize to fp32 (test aid).
hipError_t launch_dequantize(const void* packed, const void* scales, const void* zeros, int64_t N,
                             int64_t K, int bits, int group_size, bool asymmetric, float* out,
                             hipStream_t stream);

}  // namespace woq
