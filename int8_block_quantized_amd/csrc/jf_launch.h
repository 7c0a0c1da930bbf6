// jf_launch.h -- internal launchers behind the C ABI (include/jetfire.h).
// Arguments are validated by the ABI layer before these are called; each
// launcher only enqueues kernels on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jf {

hipError_t launch_quantize_f32(const float *x, int64_t ldx, int64_t rows, int64_t cols,
                               int8_t *q, int64_t ldq, float *s, hipStream_t stream);
hipError_t launch_quantize_bf16(const uint16_t *x, int64_t ldx, int64_t rows, int64_t cols,
                                int8_t *q, int64_t ldq, float *s, hipStream_t stream);
hipError_t launch_dequantize(const int8_t *q, int64_t ldq, const float *s, int64_t rows, int64_t cols, bool bf16,
                             void *y, int64_t ldy, hipStream_t stream);
hipError_t launch_gemm(int transA, int transB, int64_t M, int64_t N, int64_t K,
                       const int8_t *A, int64_t lda, const float *sA,
                       const int8_t *B, int64_t ldb, const float *sB,
                       bool out_i8, void *C, int64_t ldc, float *sC, hipStream_t stream);
hipError_t launch_gelu(const int8_t *q, int64_t ldq, const float *s, int64_t rows, int64_t cols,
                       int8_t *qo, int64_t ldqo, float *so, hipStream_t stream);

hipError_t launch_gelu_bwd(const int8_t *qdy, int64_t lddy, const float *sdy, const int8_t *qx, int64_t ldx,
                           const float *sx, int64_t rows, int64_t cols, int8_t *qo, int64_t ldo, float *so,
                           hipStream_t stream);

hipError_t launch_add(const int8_t *qa, int64_t lda, const float *sa, const int8_t *qb, int64_t ldb,
                      const float *sb, int64_t rows, int64_t cols, int8_t *qo, int64_t ldo, float *so,
                      hipStream_t stream);
hipError_t launch_layernorm(const int8_t *q, int64_t ldq, const float *s, int64_t rows, int64_t cols,
                            const float *gamma, const float *beta, float eps, int8_t *qo, int64_t ldo, float *so,
                            double *mean, double *rstd, hipStream_t stream);

// granularity: 0 block, 1 token (row), 2 channel (column), 3 tensor
hipError_t launch_quant_error(const float *x, int64_t ldx, int64_t rows, int64_t cols, int granularity, float *s,
                              double *sse, hipStream_t stream);

}  // namespace jf
