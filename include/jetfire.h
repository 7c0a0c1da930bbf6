/*
 * jetfire.h -- C ABI of the MI355X (gfx950) per-block INT8 data-flow library
 * (libjetfire.so).
 *
 * Method: "Jetfire: Efficient and Accurate Transformer Pretraining with INT8
 * Data Flow and Per-Block Quantization" (scime.ai summary of arXiv
 * 2403.12422).  Its one-line summary and "Approach" section describe the
 * data flow implemented here: every linear and non-linear operator reads and
 * writes INT8 tensors that carry one scale factor per 32x32 block, the
 * quantization is done on-chip by the producing kernel, and the weight
 * gradient is an INT8 GEMM with per-block scales as well.  Its "Problem"
 * section names the non-linear operators as memory-bound.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Matrices are row-major.  A "leading dimension" (ld*) is the distance,
 *    in elements, between the starts of consecutive stored rows.
 *  - Every row and column count is a multiple of 32.  Block (bi, bj) covers
 *    rows 32bi..32bi+31 and columns 32bj..32bj+31 of the stored matrix.
 *  - A scale grid of a stored R x C matrix is binary32 [R/32][C/32],
 *    row-major and contiguous (its leading dimension is C/32).
 *  - Per-block rule (the readings of the pages used throughout):
 *        s = fl(max|x| / 127)               one IEEE binary32 division
 *        q = clamp(rne(fl(x / s)), -127, 127)
 *    and a block whose s is zero (all zeros, or max|x|/127 underflows) has
 *    q = 0 everywhere.  Dequantized value: fl(s * q).
 *  - Pointers are DEVICE pointers (hipMalloc'd or any device-accessible
 *    allocation), except that nothing is dereferenced before validation.
 *    The caller owns every buffer; the library never allocates, frees,
 *    copies to the host or synchronizes.  Work is enqueued on `stream`
 *    (0 = the null stream) and is asynchronous; outputs are fully written.
 *  - Validation runs on the host before any HIP call and reports the first
 *    failing condition:
 *        JF_ERR_NULL   a required pointer is NULL (the pointers of an empty
 *                      matrix may be NULL)
 *        JF_ERR_SHAPE  a size is negative or not a multiple of 32
 *        JF_ERR_LD     a leading dimension is below the row length, or its
 *                      row pitch is not a multiple of 16 bytes
 *        JF_ERR_ALIGN  a matrix base is not 16-byte aligned, a scale grid
 *                      base is not 4-byte aligned, or a binary64 sum is not
 *                      8-byte aligned
 *        JF_ERR_DTYPE  an unknown element type / output kind
 *        JF_ERR_ARG    a transpose flag other than 0 or 1, an unknown scale
 *                      granularity, or a negative or non-finite epsilon
 *        JF_ERR_ALIAS  an output overlaps an input or another output
 *        JF_ERR_HIP    the kernel launch failed (hipGetLastError)
 *    A size of zero is valid: nothing is launched for an empty output, and a
 *    GEMM with K = 0 writes zeros (binary32) or zero codes and scales.  (This
 *    departs on purpose from treating an empty size as a shape error: torch
 *    hands out empty tensors, and an empty output or a K = 0 contraction has
 *    a well-defined result.  JF_ERR_ARG, for flags and granularities out of
 *    range, is likewise an addition to the shape and pointer codes.)
 *  - Inputs must be finite; NaN or Inf inputs give unspecified outputs, and
 *    so do finite inputs whose binary32 results overflow (a GEMM sum, a
 *    residual add or a dequantized value beyond the binary32 range; the
 *    bfloat16 dequantized copy rounds such values to infinity).
 *  - Entry points keep no state and are safe to call from several threads.
 */
#ifndef JETFIRE_H
#define JETFIRE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define JF_ABI_VERSION 5

#ifndef JF_API
#define JF_API __attribute__((visibility("default")))
#endif

typedef enum jf_status {
    JF_OK = 0,
    JF_ERR_NULL = 1,
    JF_ERR_SHAPE = 2,
    JF_ERR_LD = 3,
    JF_ERR_ALIGN = 4,
    JF_ERR_DTYPE = 5,
    JF_ERR_ARG = 6,
    JF_ERR_ALIAS = 7,
    JF_ERR_HIP = 8
} jf_status;

/* Element type of a high-precision input. */
typedef enum jf_dtype { JF_F32 = 0, JF_BF16 = 1 } jf_dtype;

/* Output kind of the GEMM. */
typedef enum jf_out { JF_OUT_I8 = 0, JF_OUT_F32 = 1 } jf_out;

/* Scale granularity of jf_quant_error: one scale per 32x32 block, per row
 * (token), per column (channel) or for the whole matrix (tensor). */
typedef enum jf_gran { JF_GRAN_BLOCK = 0, JF_GRAN_TOKEN = 1, JF_GRAN_CHANNEL = 2, JF_GRAN_TENSOR = 3 } jf_gran;

/*
 * jf_quantize_block -- per-block INT8 quantization of a high-precision matrix.
 * Pages: one-line summary and "Approach" (INT8 tensors with one scale per
 * 32x32 block, quantization on-chip).
 *
 *   xt    JF_F32 (binary32) or JF_BF16 (bfloat16; each value is widened
 *         exactly to binary32 first)
 *   x     rows x cols input, leading dimension ldx (elements of xt)
 *   q     rows x cols int8 codes, leading dimension ldq
 *   s     (rows/32) x (cols/32) binary32 scales, contiguous
 * Codes and scales are bit-exact with the per-block rule above.
 */
JF_API jf_status jf_quantize_block(jf_dtype xt, const void *x, int64_t ldx, int64_t rows, int64_t cols,
                            int8_t *q, int64_t ldq, float *s, hipStream_t stream);

/*
 * jf_dequantize_block -- per-block INT8 codes back to high precision.
 * Pages: "Approach" (INT8 tensors with one scale per 32x32 block); the
 * dequantized value of code q under block scale s is fl(s*q).
 *
 *   q, s  rows x cols codes (ldq) and their scale grid
 *   yt    JF_F32: y is binary32, y = fl(s*q) exactly as the convention above;
 *         JF_BF16: y is bfloat16, that binary32 value rounded to the nearest
 *         bfloat16, ties to even
 *   y     rows x cols output, leading dimension ldy (elements of yt)
 * y may not overlap q or s.
 */
JF_API jf_status jf_dequantize_block(const int8_t *q, int64_t ldq, const float *s, int64_t rows, int64_t cols,
                                     jf_dtype yt, void *y, int64_t ldy, hipStream_t stream);

/*
 * jf_gemm_i8_blockscaled -- C[M x N] = op(A)[M x K] . op(B)[K x N] on INT8
 * codes with per-block scales.  Pages: "Approach" (linear operators in the
 * INT8 data flow; the weight gradient is also INT8 with per-block scales).
 *
 *   transA  0: A stored M x K (lda >= K);  1: A stored K x M (lda >= M)
 *   transB  0: B stored K x N (ldb >= N);  1: B stored N x K (ldb >= K)
 *   sA, sB  scale grids of A and B in their STORED orientation
 *           (e.g. transA = 1: sA is [K/32][M/32])
 *   out     JF_OUT_F32: C is binary32, ldc >= N, sC ignored (may be NULL)
 *           JF_OUT_I8:  C is int8 codes, ldc >= N, sC is [M/32][N/32]
 * Numerics.  For each output block (I, J) and each 32-deep k-block kappa in
 * ascending order: P = exact int32 sum of 32 code products; sigma =
 * fl(sA[I,kappa] * sB[kappa,J]); acc = fma(sigma, (float)P, acc) in binary32,
 * starting from +0.  JF_OUT_F32 stores acc; JF_OUT_I8 requantizes each
 * 32x32 output block with the per-block rule before it leaves the chip.
 * For a linear layer with W stored K x N (in x out features):
 *   forward Y = X W (0,0);  dgrad dX = dY W^T (0,1);  wgrad dW = X^T dY (1,0).
 */
JF_API jf_status jf_gemm_i8_blockscaled(int transA, int transB, int64_t M, int64_t N, int64_t K,
                                 const int8_t *A, int64_t lda, const float *sA,
                                 const int8_t *B, int64_t ldb, const float *sB,
                                 jf_out out, void *C, int64_t ldc, float *sC,
                                 hipStream_t stream);

/*
 * jf_requant_block -- per-block requantization of a binary32 matrix: the
 * stand-alone form of the GEMM's requantizing epilogue (pages: "Approach",
 * quantization applied on-chip by the producer).  Same rule, same layout as
 * jf_quantize_block with xt = JF_F32.
 */
JF_API jf_status jf_requant_block(const float *x, int64_t ldx, int64_t rows, int64_t cols,
                           int8_t *q, int64_t ldq, float *s, hipStream_t stream);

/*
 * jf_gelu_i8 -- INT8-in / INT8-out GELU.  Pages: "Problem" (non-linear
 * operators are memory-bound) and "Approach" (they too read and write INT8
 * with per-block scales).
 *
 *   q, s    rows x cols input codes (ldq) and their scale grid
 *   qo, so  rows x cols output codes (ldqo) and their scale grid
 * Per block: x = fl(s*q); g = x * Phi(x) with Phi the standard normal CDF
 * (erf form of GELU), evaluated in binary64 and rounded once to binary32;
 * then the per-block rule on g.  (The kernel evaluates g per code value in
 * binary32 and redoes in binary64 every entry whose output code it cannot
 * decide, so codes and scales match the binary64 definition.)  In-place
 * operation is rejected.
 */
JF_API jf_status jf_gelu_i8(const int8_t *q, int64_t ldq, const float *s, int64_t rows, int64_t cols,
                     int8_t *qo, int64_t ldqo, float *so, hipStream_t stream);

/*
 * jf_gelu_bwd_i8 -- INT8 GELU backward: dX = dY * GELU'(X).  Pages:
 * "Approach" (every operator of the INT8 data flow reads and writes INT8
 * with per-block scales; the backward pass is part of that data flow).
 *
 *   qdy, sdy  rows x cols incoming gradient codes (lddy) and scale grid
 *   qx, sx    rows x cols forward input codes (ldx) and scale grid, same
 *             32x32 blocking
 *   qo, so    rows x cols output gradient codes (ldo) and scale grid
 * Per element: dy = fl(sdy*qdy), x = fl(sx*qx), y = fl(dy * GELU'(x)) with
 * GELU'(x) = Phi(x) + x phi(x) evaluated in binary64 and rounded once to
 * binary32; then the per-block rule on y.  Outputs may not overlap inputs.
 */
JF_API jf_status jf_gelu_bwd_i8(const int8_t *qdy, int64_t lddy, const float *sdy, const int8_t *qx, int64_t ldx,
                                const float *sx, int64_t rows, int64_t cols, int8_t *qo, int64_t ldo, float *so,
                                hipStream_t stream);

/*
 * jf_add_i8 -- residual add of two per-block INT8 tensors.  Pages: "Jetfire"
 * summary, "Approach" (every operator of the data flow reads and writes INT8
 * with one scale per 32x32 block; the add itself is this library's reading).
 *
 *   qa, sa    rows x cols codes (lda) and scale grid of the first operand
 *   qb, sb    the second operand, same 32x32 blocking (ldb)
 *   qo, so    rows x cols output codes (ldo) and scale grid
 * Per element z = fl(fl(sa*qa) + fl(sb*qb)); then the per-block rule on z.
 * Outputs may not overlap inputs.
 */
JF_API jf_status jf_add_i8(const int8_t *qa, int64_t lda, const float *sa, const int8_t *qb, int64_t ldb,
                           const float *sb, int64_t rows, int64_t cols, int8_t *qo, int64_t ldo, float *so,
                           hipStream_t stream);

/*
 * jf_layernorm_i8 -- LayerNorm over each row (the hidden dimension) of a
 * per-block INT8 tensor, INT8 out.  Pages: "Jetfire" summary, "Approach"
 * (every operator of the data flow reads and writes per-block INT8; the
 * normalization itself is this library's reading).
 *
 *   q, s         rows x cols input codes (ldq) and scale grid
 *   gamma, beta  cols binary32 values each (16-byte aligned)
 *   eps          added to the variance; finite and >= 0 (rows of zero
 *                variance need eps > 0)
 *   qo, so       rows x cols output codes (ldo) and scale grid
 *   mean, rstd   optional (NULL to skip): rows binary64 values each, the
 *                row means and 1/sqrt(v + eps) (8-byte aligned)
 * Per row: x = fl(s*q); m = sum(x)/n and v = sum((x - m)^2)/n in binary64;
 * r = 1/sqrt(v + eps) in binary64; y = ((x - m)*r)*gamma + beta in binary64
 * rounded once to binary32; then the per-block rule on y.  The binary64 sums
 * are formed in an unspecified order.  Outputs may not overlap inputs or
 * each other.
 */
JF_API jf_status jf_layernorm_i8(const int8_t *q, int64_t ldq, const float *s, int64_t rows, int64_t cols,
                                 const float *gamma, const float *beta, float eps, int8_t *qo, int64_t ldo,
                                 float *so, double *mean, double *rstd, hipStream_t stream);

/*
 * jf_quant_error -- quantization error of one binary32 matrix under one scale
 * granularity.  Pages: "Jetfire" summary, "Measured effects" (per-block
 * quantization keeps the error of activations with channel-wise outliers
 * below per-token and per-channel quantization).
 *
 *   x, ldx       rows x cols binary32 matrix (16-byte aligned rows)
 *   granularity  a jf_gran value
 *   s            group scales, written: (rows/32) x (cols/32) row-major for
 *                JF_GRAN_BLOCK, rows for TOKEN, cols for CHANNEL, 1 for
 *                TENSOR (4-byte aligned)
 *   sse          one binary64, written: sum over all elements of
 *                (x - fl(s*q))^2, each term in binary64 (8-byte aligned)
 * Each group takes the per-block rule: s = fl(max|x|/127),
 * q = clamp(rne(fl(x/s)), -127, 127), fl(s*q) = 0 when s = 0.  Scales are
 * exact; sse is summed in an unspecified order (binary64 rounding only).
 * The codes are not stored.  sse is required; with rows or cols zero the
 * scales that exist are set to zero and sse to 0.  s and sse may not overlap
 * x or each other.
 */
JF_API jf_status jf_quant_error(const float *x, int64_t ldx, int64_t rows, int64_t cols, int granularity,
                                float *s, double *sse, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
JF_API const char *jf_status_str(jf_status status);

/* JF_ABI_VERSION of the built library. */
JF_API int jf_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* JETFIRE_H */
