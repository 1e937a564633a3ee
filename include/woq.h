/*
 * woq.h -- C ABI of libwoq: group-wise weight-only 3/4-bit quantization and
 * the fused dequantize + GEMV/GEMM that consumes it, for AMD MI355X (gfx950).
 *
 * What is computed (the pages this library implements):
 *
 *  - Group-wise round-to-nearest quantization of a weight row, one scale (and
 *    zero point) per group of consecutive weights along K ("Quantising Large
 *    Language Models for Efficient Inference", section "Post-training methods
 *    for 4-bit weights"); symmetric absmax and asymmetric zero-point forms
 *    ("CMU 11-868 L19-L20 Model Quantization", section "absmax and
 *    zero-point"; "LLM Quantization: 160GB Model on a Laptop", sections
 *    "Symmetric Quantization" and "Asymmetric Quantization"); AutoGPTQ-style
 *    parameters bits and group_size ("CMU 11-868 ...", section "Setup and
 *    results").
 *  - An optional per-input-channel AWQ scale s: weights are multiplied by s
 *    before quantization and activations divided by s in the matmul
 *    ("Quantising ...", section "Why LLMs are hard to quantise":
 *    Y = (X diag(s)^-1)(diag(s) W); "MIT 6.5940 Lab 4 + Lab 5", Lab 4
 *    Question 2).
 *  - A W4A16 matmul whose weights are dequantized on the fly inside the
 *    kernel ("Quantising ...", section "Weight-only vs weight-and-activation
 *    quantisation"), with fp16 or bf16 activations and fp32 accumulation.
 *
 * Quantization of one group of G weights w (fp32 after the optional fold
 * w = fl32(W * s[k]); every step one correctly rounded binary32 operation,
 * rne = round half to even, f16() = binary16 round-to-nearest-even):
 *
 *   symmetric : S = f16(max|w| / (2^(b-1)-1));
 *               u = clip(rne(w / S), -2^(b-1), 2^(b-1)-1) + 2^(b-1);
 *               S == 0 -> u = 2^(b-1).  zeros are implied (2^(b-1)).
 *   asymmetric: r = max - min, r := 1 if r == 0;  S = f16(r / (2^b-1));
 *               Z = clip(rne(-min / S), 0, 2^b-1);
 *               u = clip(rne(w / S) + Z, 0, 2^b-1);  S == 0 -> Z = u = 0.
 *   dequantized weight: w_hat = (u - Z) * S.
 *
 * Packed layout v2 (WOQ_LAYOUT_V2).  Rows n = 0..N-1 back to back, each
 * K*bits/8 bytes; groups are contiguous along K starting at k = 0.  Words are
 * little-endian 32-bit.
 *   4-bit (unchanged from layout v1): word j of a row holds k in [8j, 8j+8);
 *          the code of k = 8j + 2t + h (t = 0..3, h = 0..1) is at bits
 *          [16h+4t, 16h+4t+4).  (w >> 4t) & 0x000F000F therefore yields the
 *          pair (k, k+1) in the two 16-bit halves of a register.
 *   3-bit: a 12-byte unit j (words w0, w1, w2) holds k in [32j, 32j+32); for
 *          i = k - 32j = 2t + h (t = 0..15, h = 0..1) the whole code of pair
 *          t < 15 is in w_(t/5) at bits [16h + 3(t%5), +3), so
 *          (w >> 3(t%5)) & 0x00070007 yields pair t; the code of pair 15 is
 *          split, its bit b (b = 0..2) at bit 16h + 15 of w_b.  (Layout v1
 *          kept two low bits and the high bit of a pair in different words.)
 *   scales: fp16 [N, K/G] row-major.  zeros: fp16 [N, K/G] row-major holding
 *          the integer Z (asymmetric only).
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller (the library
 *    never allocates, frees or synchronizes).  act_scale may be NULL.
 *  - stream is a hipStream_t passed as void* (NULL = the default stream); all
 *    work is enqueued asynchronously on it.  Errors detected before launch are
 *    returned; faults during execution surface at the caller's next sync.
 *  - Arguments are validated before any HIP call.  Invalid arguments return
 *    WOQ_ERR_INVALID_ARGUMENT, valid but unimplemented combinations
 *    WOQ_ERR_UNSUPPORTED, a failing HIP launch WOQ_ERR_HIP.  woq_last_error()
 *    gives a thread-local message for the last failing call on this thread.
 *  - Constraints: bits in {3, 4}; group_size % 32 == 0; K % group_size == 0;
 *    N >= 1, K >= 32, M >= 1; packed, X/x and Y/y 16-byte aligned; scales and
 *    zeros 2-byte aligned; zeros != NULL exactly when asymmetric != 0.
 *  - Inputs must be finite.  Weights whose fp16 scale would overflow give
 *    unspecified results.  No C++ exception crosses this boundary.
 *  - Calls are thread-safe; the library keeps no state besides a cached
 *    device-property query and the per-thread error message.
 */
#ifndef WOQ_H_
#define WOQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WOQ_LAYOUT_V2 2

typedef enum woq_status {
  WOQ_OK = 0,
  WOQ_ERR_INVALID_ARGUMENT = 1,
  WOQ_ERR_UNSUPPORTED = 2,
  WOQ_ERR_HIP = 3,
  WOQ_ERR_INTERNAL = 4
} woq_status;

/* Activation / output element type. */
typedef enum woq_dtype { WOQ_F16 = 0, WOQ_BF16 = 1 } woq_dtype;

/* Layout version produced and consumed by this library (WOQ_LAYOUT_V2). */
int32_t woq_layout_version(void);

/* Bytes of the packed code array for an [N, K] matrix: N * K * bits / 8.
 * Returns 0 for invalid arguments. */
size_t woq_packed_bytes(int64_t N, int64_t K, int32_t bits);

/* Bytes of one scale (or zero) array: N * (K / group_size) * 2.
 * Returns 0 for invalid arguments. */
size_t woq_scales_bytes(int64_t N, int64_t K, int32_t group_size);

/* Workspace bytes woq_w4a16_gemm can use for this shape (0 for invalid
 * arguments).  Non-zero (8 M bytes rounded up to 256, plus 2 M K bytes) for
 * M >= 33, 4-bit codes, K % 64 == 0 and K < 65536: there, bf16 X given a workspace at
 * least this large (256-byte aligned, device memory the call may overwrite)
 * runs on the fp16 mid-M (33..127 rows, where fp16 X would take it) or
 * register-B (M >= 128) kernel through an exact per-row power-of-two rescale:
 * the call writes each row's factors and the rescaled fp16 copy of X into the
 * workspace; without one it takes the slower bf16 kernels.
 * fp16 X and woq_w4a16_gemv never use a workspace, and workspace = NULL is
 * always valid. */
size_t woq_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t bits, int32_t group_size);

/* Quantize fp16 weights W [N, K] (row-major, output channel n, input channel
 * k) group-wise and write the packed codes, scales and zeros.
 *   W         : fp16 [N, K]
 *   act_scale : fp32 [K] AWQ scale s multiplied into column k before the
 *               group statistics, or NULL
 *   packed    : out, uint8 [N, K*bits/8] in layout v2
 *   scales    : out, fp16 [N, K/group_size]
 *   zeros     : out, fp16 [N, K/group_size] when asymmetric, else NULL
 * Bit-exact with the definition above (IEEE division, RNE everywhere). */
woq_status woq_quantize_pack(const void* W, const float* act_scale, int64_t N, int64_t K,
                             int32_t bits, int32_t group_size, int32_t asymmetric,
                             void* packed, void* scales, void* zeros, void* stream);

/* One matrix of woq_quantize_pack_many: the per-matrix arguments of
 * woq_quantize_pack (device pointers owned by the caller). */
typedef struct woq_qmatrix {
  const void* W;          /* fp16 [N, K] */
  const float* act_scale; /* fp32 [K] or NULL, per matrix */
  void* packed;           /* out, uint8 [N, K*bits/8] in layout v2 */
  void* scales;           /* out, fp16 [N, K/group_size] */
  void* zeros;            /* out, fp16 [N, K/group_size] when asymmetric, else NULL */
  int64_t N, K;
} woq_qmatrix;

/* woq_quantize_pack over `count` matrices that share bits, group_size and
 * asymmetric -- e.g. every linear of a model, which a model conversion
 * quantizes and packs once, offline ("MIT 6.5940 Lab 4 + Lab 5", section
 * "Background: why the 4-bit weights get reordered first").  Each matrix's
 * packed, scales and zeros are byte-equal to what woq_quantize_pack writes
 * for the same arguments.  When group_size / 32 divides 64 up to 32 matrices
 * share one launch, so one matrix's tail overlaps the next one's start;
 * other group sizes take one launch per matrix.
 *   mats  : HOST array of `count` descriptors (count >= 1), read during the
 *           call only.
 * Every descriptor is checked as woq_quantize_pack checks its arguments
 * before anything is enqueued; an invalid one fails the whole call with
 * WOQ_ERR_INVALID_ARGUMENT and woq_last_error() names its index.  Outputs
 * of different matrices must not overlap one another or any input. */
woq_status woq_quantize_pack_many(const woq_qmatrix* mats, int32_t count, int32_t bits, int32_t group_size,
                                  int32_t asymmetric, void* stream);

/* y[n] = sum_k (x[k] / s[k]) * w_hat[n, k]  (M = 1 decode GEMV).
 *   x         : [K] of xdtype (WOQ_F16 or WOQ_BF16)
 *   act_scale : fp32 [K] (the same s given to woq_quantize_pack) or NULL
 *   packed, scales, zeros : as written by woq_quantize_pack
 *   y         : out, [N] of xdtype
 * Accumulates in fp32.  x * r(s) (r(s): the hardware reciprocal, within
 * 1 ulp of 1 / s) is rounded once to xdtype before use (a bf16 pair hi + lo
 * for bf16 x); the integer (u - Z) is multiplied exactly and S is applied in
 * fp32 per group. */
woq_status woq_w4a16_gemv(const void* x, int32_t xdtype, const float* act_scale,
                          const void* packed, const void* scales, const void* zeros,
                          int64_t N, int64_t K, int32_t bits, int32_t group_size, int32_t asymmetric,
                          void* y, void* workspace, size_t workspace_bytes, void* stream);

/* Y[m, n] = sum_k (X[m, k] / s[k]) * w_hat[n, k]  for M >= 1.
 *   X : [M, K] row-major of xdtype;  Y : out, [M, N] row-major of xdtype.
 * Small M decodes weights in registers and feeds MFMA with an exact integer
 * (u - Z) and per-group fp32 scaling.  Large M (M >= 128 and, for fp16,
 * K % 64 == 0), and fp16 X with 4-bit codes, K % 64 == 0 and K < 65536 at 33..127 rows
 * (always above 64 rows; at 33..64 rows when N >= 16384 or the small-batch
 * kernel does not take the shape), feed MFMA with dequantized weights: for
 * fp16, w_hat rounded once to fp16 (decoded straight into operand registers
 * for 4-bit codes, or staged in LDS) with X * r(s) rounded once to fp16
 * (r(s): the hardware reciprocal, within 1 ulp of 1 / s); for bf16, X used
 * as given and w_hat * r(s) kept as a bf16 pair
 * hi + lo (about 16 significant bits), or, for bf16 X at 33..127 rows without
 * an AWQ scale (group size a power of two >= 64), the exact 128 + u with the
 * scale applied per group in fp32.  bf16 X given a workspace of
 * woq_workspace_bytes(M, N, K, bits, group_size) > 0 bytes instead runs as
 * fp16: each row, X * r(s) with an AWQ scale, is multiplied by the power of
 * two f_m that puts its largest magnitude in [2^14, 2^15) and converted to
 * fp16 (exact without an AWQ scale, for every value above 2^-31 of the row's
 * largest), the product uses w_hat rounded once to fp16, and the result is
 * multiplied by 1 / f_m and rounded once to bf16.  fp32 accumulation
 * throughout; the order of the K sum inside an MFMA step is the kernel's.
 * workspace may be NULL; when given it must be 256-byte aligned. */
woq_status woq_w4a16_gemm(const void* X, int32_t xdtype, const float* act_scale,
                          const void* packed, const void* scales, const void* zeros,
                          int64_t M, int64_t N, int64_t K, int32_t bits, int32_t group_size,
                          int32_t asymmetric, void* Y, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Test aid: w_hat = (u - Z) * S as fp32 [N, K] (exact: |u - Z| < 16 and S has
 * 11 significant bits).  Pseudo-quantization's dequantize step ("MIT 6.5940
 * Lab 4 + Lab 5", Lab 4 setup). */
woq_status woq_dequantize(const void* packed, const void* scales, const void* zeros,
                          int64_t N, int64_t K, int32_t bits, int32_t group_size, int32_t asymmetric,
                          float* out, void* stream);

/* AWQ exponent search over one layer ("MIT 6.5940 Lab 4 + Lab 5", Question 2:
 * compute the scale, scale the weight channels up, quantize, divide the
 * activations; the layer-wise reconstruction objective of "Quantising Large
 * Language Models ...", section "Post-training methods for 4-bit weights").
 *   X          : fp16 [T, K] row-major calibration activations (device)
 *   W          : fp16 [N, K] row-major weights (device)
 *   bits, group_size, asymmetric : the quantizer to search for (as above)
 *   n_grid     : number of exponents, 1 .. 64; alpha_i = i / n_grid
 *   losses     : out, fp64 [n_grid] (device): || X W^T - (X / s_i) Q(W s_i)^T ||_F^2
 *                with s_i[k] = fl32(max(mean_t |X[t, k]|, 1e-4)^alpha_i)
 *   best_scale : out, fp32 [K] (device, 16-byte aligned): s of the first
 *                alpha with the smallest loss, ready to pass as act_scale
 *   best_index : out, int32 [1] (device): that alpha's index
 *   workspace  : device scratch of woq_awq_search_workspace_bytes(...) bytes,
 *                256-byte aligned, owned by the caller; holds the reference
 *                output X W^T (fp32) and, for each exponent of one batched
 *                GEMM launch (up to 8 where the GEMM is the register-B
 *                kernel, else 1), a scale vector, a packed set and the
 *                quantized output.
 * The loss uses the library's own quantize_pack and GEMM (so the quantized
 * output is rounded to fp16 as any other call's), an fp32 reference output
 * and an fp64 sum.  Asynchronous on stream; returns WOQ_ERR_INVALID_ARGUMENT
 * for bad sizes, pointers or a short workspace. */
size_t woq_awq_search_workspace_bytes(int64_t T, int64_t N, int64_t K, int32_t bits,
                                      int32_t group_size, int32_t asymmetric);
woq_status woq_awq_search(const void* X, const void* W, int64_t T, int64_t N, int64_t K,
                          int32_t bits, int32_t group_size, int32_t asymmetric, int32_t n_grid,
                          double* losses, float* best_scale, int32_t* best_index,
                          void* workspace, size_t workspace_bytes, void* stream);

/* The AWQ exponent search above without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Arguments, outputs and results
 * are those of woq_awq_search; the scratch is a static device array of
 * woq_awq_search_noalloc_max_bytes() bytes (32 MiB) inside the library, one
 * per GPU, held until the process ends.  Every call on a GPU uses that GPU's
 * one array, so calls that overlap on one GPU (other streams or threads)
 * race and must be serialized by the caller.  No allocation, free or
 * allocating library routine is called.  Shapes whose search does not fit
 * the array return WOQ_ERR_UNSUPPORTED (e.g. T x N fp32 reference output
 * plus one packed set, scale and fp16 output must fit: 512 tokens of a
 * 4096 x 4096 layer do). */
size_t woq_awq_search_noalloc_max_bytes(void);
woq_status woq_awq_search_noalloc(const void* X, const void* W, int64_t T, int64_t N, int64_t K,
                                  int32_t bits, int32_t group_size, int32_t asymmetric, int32_t n_grid,
                                  double* losses, float* best_scale, int32_t* best_index, void* stream);

/* GPTQ into layout v2 ("CMU 11-868 L19-L20 Model Quantization", section
 * "The algorithm in four steps"; the layer-wise objective of "Quantising
 * Large Language Models ...", section "Post-training methods for 4-bit
 * weights").
 *   X          : fp16 [T, K] row-major calibration activations (device)
 *   W          : fp16 [N, K] row-major weights (device)
 *   bits, group_size, asymmetric : the quantizer (as above); K % 128 == 0 and
 *                group_size divides 128 or is a multiple of 128, else
 *                WOQ_ERR_UNSUPPORTED
 *   damp       : > 0; lambda = damp * mean(diag H) is added to the diagonal
 *                of H = 2 X^T X (0.01 is the usual value)
 *   packed, scales, zeros : out, exactly as woq_quantize_pack writes them
 *                (zeros only when asymmetric), ready for the GEMV / GEMM with
 *                act_scale = NULL
 *   workspace  : device scratch of woq_gptq_workspace_bytes(...) bytes,
 *                256-byte aligned, owned by the caller (two K x K fp64
 *                matrices, an fp64 copy of W and 128 fp64 errors per row).
 * A channel with H[k, k] == 0 (never active in X) gets H[k, k] = 1 and its
 * weights set to 0 before quantization.  U (upper, U^T U = (H + lambda I)^-1)
 * comes from a Cholesky factorization and triangular inverse in fp64; columns
 * are quantized in order, each rounding error divided by U[k, k] and
 * subtracted, times U[k, j], from every later column j (fp64).  The
 * parameters of a group come from its current weights when its first column
 * is reached, and every rounding decision (group statistic, scale, zero
 * point, code) is made on the fp32 value of the current weight by the rules
 * above.  Non-finite X or W give unspecified codes.  Asynchronous on stream;
 * returns WOQ_ERR_INVALID_ARGUMENT for bad sizes, pointers or a short
 * workspace. */
size_t woq_gptq_workspace_bytes(int64_t T, int64_t N, int64_t K, int32_t bits, int32_t group_size);
woq_status woq_gptq_quantize_pack(const void* X, const void* W, int64_t T, int64_t N, int64_t K,
                                  int32_t bits, int32_t group_size, int32_t asymmetric, double damp,
                                  void* packed, void* scales, void* zeros,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Measurement aids.  Not part of the method: they measure the ceilings the
 * quantized kernels are compared with.  A decode GEMV reads its weights once
 * and does about one flop per byte, so its floor is the time to stream those
 * bytes ("MIT 6.5940 Lab 4 + Lab 5", Lab 4 "Starting point and setup"); a
 * large-batch GEMM is bound by the matrix units ("CMU 11-868 L19-L20",
 * section "Back to the question: where does the speed come from?").
 *
 * woq_probe_stream_read: reads `bytes` bytes (a multiple of 16) at p (device,
 *   16-byte aligned) once, as 16-byte nontemporal loads: blocks x threads
 *   threads (threads a multiple of 64, at most 1024), each with `unroll`
 *   (1, 2, 4 or 8) loads in flight per round.  The XOR of the words each
 *   thread read is written to sink[thread] (device, blocks * threads uint32)
 *   only when store != 0; with store == 0 sink is never written.
 * woq_probe_empty: launches an empty kernel of blocks x threads threads.
 * woq_probe_mfma_rate: blocks workgroups of 4 waves, each running `iters`
 *   steps of 4 independent v_mfma_f32_32x32x16_f16 chains (2 * 32 * 32 * 16
 *   flop each) on operands read from src (device, at least 1 MiB of fp16
 *   data, 16-byte aligned); the sums go to sink (device, blocks * 256 floats)
 *   only when store != 0.
 * woq_probe_mfma_valu: whether VALU work hides under MFMAs, and the clock
 *   the SIMDs run at.  blocks workgroups of 4 waves, each running `iters`
 *   steps of mfma_per_iter v_mfma_f32_32x32x16_f16 (4 independent chains)
 *   and valu_per_iter independent 32-bit integer VALU operations;
 *   (mfma_per_iter, valu_per_iter) is (4, 0|16|32|64) or (0, 32|64).  src
 *   and sink as for woq_probe_mfma_rate.  Wave 0 of workgroup b writes the
 *   shader clock counter (s_memtime) at its start and end to clocks[4b] and
 *   clocks[4b + 1], and the 100 MHz real-time counter (s_memrealtime) to
 *   clocks[4b + 2] and clocks[4b + 3] (device, 4 * blocks uint64).
 * woq_probe_gemv_timeline: the decode GEMV (woq_w4a16_gemv with K = 8192,
 *   group 128, 4-bit asymmetric codes, fp16 x, no activation scale; N rows,
 *   the same launch shape and result y) with a per-wave timeline: 8 uint64
 *   words per wave in timeline (device), the 100 MHz real-time counter at the
 *   wave's start, after x is staged, after its first row step, after the
 *   stream, and at its end, then the XCD id and two zero words.
 *   timeline_words must be at least woq_probe_gemv_timeline_words(N) (0 for
 *   N outside [1, 2^31]).
 * Asynchronous on stream; invalid arguments return WOQ_ERR_INVALID_ARGUMENT. */
woq_status woq_probe_stream_read(const void* p, size_t bytes, int32_t blocks, int32_t threads, int32_t unroll,
                                 void* sink, int32_t store, void* stream);
woq_status woq_probe_empty(int32_t blocks, int32_t threads, void* stream);
woq_status woq_probe_mfma_rate(const void* src, int32_t blocks, int32_t iters, float* sink, int32_t store,
                               void* stream);
woq_status woq_probe_mfma_valu(const void* src, int32_t blocks, int32_t iters, int32_t mfma_per_iter,
                               int32_t valu_per_iter, float* sink, uint64_t* clocks, int32_t store, void* stream);
size_t woq_probe_gemv_timeline_words(int64_t N);
woq_status woq_probe_gemv_timeline(const void* x, const void* packed, const void* scales, const void* zeros,
                                   int64_t N, void* y, uint64_t* timeline, size_t timeline_words, void* stream);

/* Static text for a status code. */
const char* woq_status_string(woq_status status);

/* Thread-local message describing the last failing call on this thread
 * ("" if none).  Valid until the next library call on this thread. */
const char* woq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WOQ_H_ */
