/*
 * jfo.c -- CPU oracle for the per-block (32x32) INT8 data flow.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * reference that the HIP kernels are checked against.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never links, loads or calls it, and it shares no code,
 * header, table or constant with the HIP path.
 *
 * Source of the method: "Jetfire: Efficient and Accurate Transformer
 * Pretraining with INT8 Data Flow and Per-Block Quantization" (scime.ai
 * summary page of arXiv 2403.12422):
 *   - one-line summary and "Approach": every linear and non-linear operator
 *     reads and writes INT8 tensors with one scale factor per 32x32 block
 *     (B = 32), quantization happens on-chip, and the weight gradient is also
 *     an INT8 GEMM with per-block scales;
 *   - "Problem": non-linear operators are memory-bound.
 * The pages give no formula.  The readings taken here (all listed with their
 * reasons in the design notes):
 *   - scale  s = fl(max|x| / 127) in binary32, one IEEE division;
 *   - code   q = clamp(round_half_even(fl(x / s)), -127, 127);
 *   - a block whose s is zero (all zeros, or max|x|/127 underflows) gets
 *     s = 0 and q = 0 everywhere;
 *   - GEMM: per output block and per 32-deep k-block kappa (ascending) the
 *     exact int32 partial P is formed, sigma = fl(sA * sB), and the fp32
 *     accumulator becomes fmaf(sigma, (float)P, acc);
 *   - GELU: x = fl(s * q), g = x * Phi(x) with Phi(x) = erfc(-x/sqrt 2)/2
 *     evaluated in binary64 and rounded once to binary32, then the block
 *     is requantized with the same scale/code rule;
 *   - GELU backward: dy = fl(s_dy * q_dy), x = fl(s_x * q_x),
 *     g' = Phi(x) + x phi(x) in binary64 rounded once, y = fl(dy * g'),
 *     then the same per-block requantization;
 *   - residual add of two tensors with the same blocking:
 *     z = fl(fl(s_a * q_a) + fl(s_b * q_b)), then the per-block rule;
 *   - dequantized value fl(s * q) in binary32; its bfloat16 copy is that
 *     binary32 value rounded to the nearest bfloat16, ties to even;
 *   - LayerNorm over each row (the hidden dimension): x = fl(s * q);
 *     mean m = (sum x) / n and variance v = (sum (x - m)^2) / n in binary64,
 *     summed in column order; r = 1 / sqrt(v + eps) in binary64;
 *     y = ((x - m) * r) * gamma + beta in binary64, rounded once to binary32;
 *     then the per-block rule on y.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off (no contraction, no fast-math),
 * so every rounding below is the one written.  All matrices are dense,
 * row-major and contiguous; all sizes are multiples of 32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define JFO_B 32

/* ------------------------------------------------------------------ */
/* Per-block quantization (Approach: per-block scale factors, B = 32). */
/* ------------------------------------------------------------------ */

/* Quantize one 32x32 block of binary32 values.  x has row stride ldx,
 * q has row stride ldq. */
static void quantize_one_block(const float *x, int64_t ldx, int8_t *q, int64_t ldq, float *s_out)
{
    float m = 0.0f;
    for (int r = 0; r < JFO_B; ++r)
        for (int c = 0; c < JFO_B; ++c) {
            float a = fabsf(x[r * ldx + c]);
            if (a > m) m = a;
        }
    float s = m / 127.0f;
    *s_out = s;
    for (int r = 0; r < JFO_B; ++r)
        for (int c = 0; c < JFO_B; ++c) {
            int8_t code = 0;
            if (s != 0.0f) {
                float t = x[r * ldx + c] / s;   /* one IEEE binary32 division */
                float v = rintf(t);             /* ties to even (default mode) */
                if (v > 127.0f) v = 127.0f;
                if (v < -127.0f) v = -127.0f;
                code = (int8_t)v;
            }
            q[r * ldq + c] = code;
        }
}

static int shape_ok(int64_t rows, int64_t cols)
{
    return rows > 0 && cols > 0 && rows % JFO_B == 0 && cols % JFO_B == 0;
}

/* x: rows x cols binary32 -> q: rows x cols int8, s: (rows/32) x (cols/32). */
int jfo_quantize_f32(const float *x, int64_t rows, int64_t cols, int8_t *q, float *s)
{
    if (!shape_ok(rows, cols)) return -1;
    const int64_t br = rows / JFO_B, bc = cols / JFO_B;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < br * bc; ++b) {
        int64_t bi = b / bc, bj = b % bc;
        quantize_one_block(x + bi * JFO_B * cols + bj * JFO_B, cols,
                           q + bi * JFO_B * cols + bj * JFO_B, cols, &s[b]);
    }
    return 0;
}

/* bfloat16 input: each value is widened exactly (its 16 bits become the high
 * half of a binary32) and then quantized as above. */
int jfo_quantize_bf16(const uint16_t *x, int64_t rows, int64_t cols, int8_t *q, float *s)
{
    if (!shape_ok(rows, cols)) return -1;
    const int64_t br = rows / JFO_B, bc = cols / JFO_B;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < br * bc; ++b) {
        int64_t bi = b / bc, bj = b % bc;
        float tile[JFO_B * JFO_B];
        for (int r = 0; r < JFO_B; ++r)
            for (int c = 0; c < JFO_B; ++c) {
                uint32_t bits = (uint32_t)x[(bi * JFO_B + r) * cols + bj * JFO_B + c] << 16;
                float v;
                memcpy(&v, &bits, sizeof v);
                tile[r * JFO_B + c] = v;
            }
        quantize_one_block(tile, JFO_B, q + bi * JFO_B * cols + bj * JFO_B, cols, &s[b]);
    }
    return 0;
}

/* Requantization of a binary32 tensor: the same rule as quantization.  This
 * is the stand-alone form of the GEMM's requantizing epilogue. */
int jfo_requant(const float *x, int64_t rows, int64_t cols, int8_t *q, float *s)
{
    return jfo_quantize_f32(x, rows, cols, q, s);
}

/* Dequantization x = fl(s * q), binary32. */
int jfo_dequantize(const int8_t *q, const float *s, int64_t rows, int64_t cols, float *x)
{
    if (!shape_ok(rows, cols)) return -1;
    const int64_t bc = cols / JFO_B;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j)
            x[i * cols + j] = s[(i / JFO_B) * bc + j / JFO_B] * (float)q[i * cols + j];
    return 0;
}

/* The bfloat16 nearest to a finite binary32 value f, ties to the even
 * significand: the two bfloat16 magnitudes around |f| are |f| with its low 16
 * bits cleared and the next one up (0x7F800000, infinity, past the largest
 * finite one, which counts as 2^128 for the distance); the closer one is
 * taken, and on a tie the one whose last kept bit is 0.  Distances are exact
 * in binary64. */
static uint16_t bf16_nearest_even(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    const uint32_t sign = u & 0x80000000u, mag = u & 0x7FFFFFFFu;
    const uint32_t lo = mag & 0xFFFF0000u, hi = lo + 0x10000u;
    if (lo == mag) return (uint16_t)((sign | lo) >> 16);
    float flo, fhi;
    memcpy(&flo, &lo, sizeof flo);
    memcpy(&fhi, &hi, sizeof fhi);
    const double a = fabs((double)f);
    const double dlo = a - (double)flo;
    const double dhi = (hi == 0x7F800000u ? ldexp(1.0, 128) : (double)fhi) - a;
    uint32_t r;
    if (dlo < dhi)
        r = lo;
    else if (dhi < dlo)
        r = hi;
    else
        r = (lo & 0x10000u) ? hi : lo;
    return (uint16_t)((sign | r) >> 16);
}

/* bfloat16 copy of the dequantized values: nearest-even of fl(s * q). */
int jfo_dequantize_bf16(const int8_t *q, const float *s, int64_t rows, int64_t cols, uint16_t *x)
{
    if (!shape_ok(rows, cols)) return -1;
    const int64_t bc = cols / JFO_B;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j)
            x[i * cols + j] = bf16_nearest_even(s[(i / JFO_B) * bc + j / JFO_B] * (float)q[i * cols + j]);
    return 0;
}

/* Single binary32 -> bfloat16 conversions (for the pins of the rule above). */
int jfo_bf16_round(const float *f, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_nearest_even(f[i]);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Block-scaled GEMM  C[MxN] = op(A)[MxK] * op(B)[KxN]                 */
/* (Approach: linear operators, incl. the weight gradient, in INT8     */
/*  with per-block scales).                                            */
/* A is stored MxK (ta = 0) or KxM (ta = 1); B is stored KxN (tb = 0)   */
/* or NxK (tb = 1).  Scale grids follow the stored orientation.        */
/* ------------------------------------------------------------------ */

typedef struct {
    int ta, tb;
    int64_t M, N, K;
    const int8_t *A, *B;
    const float *sA, *sB;
} gemm_args;

static inline int32_t a_at(const gemm_args *g, int64_t i, int64_t k)
{
    return g->ta ? g->A[k * g->M + i] : g->A[i * g->K + k];
}
static inline int32_t b_at(const gemm_args *g, int64_t k, int64_t j)
{
    return g->tb ? g->B[j * g->K + k] : g->B[k * g->N + j];
}
static inline float sa_at(const gemm_args *g, int64_t I, int64_t kb)
{
    return g->ta ? g->sA[kb * (g->M / JFO_B) + I] : g->sA[I * (g->K / JFO_B) + kb];
}
static inline float sb_at(const gemm_args *g, int64_t kb, int64_t J)
{
    return g->tb ? g->sB[J * (g->K / JFO_B) + kb] : g->sB[kb * (g->N / JFO_B) + J];
}

/* Exact int32 partial of output element (i, j) over k-block kb. */
static inline int32_t partial(const gemm_args *g, int64_t i, int64_t j, int64_t kb)
{
    int32_t p = 0;
    for (int t = 0; t < JFO_B; ++t)
        p += a_at(g, i, kb * JFO_B + t) * b_at(g, kb * JFO_B + t, j);
    return p;
}

/* One output element: k-blocks in ascending order, sigma = fl(sA*sB), one
 * fused multiply-add per k-block into a binary32 accumulator. */
static float gemm_element(const gemm_args *g, int64_t i, int64_t j)
{
    float acc = 0.0f;
    for (int64_t kb = 0; kb < g->K / JFO_B; ++kb) {
        int32_t p = partial(g, i, j, kb);
        float sigma = sa_at(g, i / JFO_B, kb) * sb_at(g, kb, j / JFO_B);
        acc = fmaf(sigma, (float)p, acc);
    }
    return acc;
}

static int gemm_shape_ok(int ta, int tb, int64_t M, int64_t N, int64_t K)
{
    return (ta == 0 || ta == 1) && (tb == 0 || tb == 1) && shape_ok(M, N) && shape_ok(K, K);
}

/* Full binary32 output, C row-major MxN. */
int jfo_gemm_f32(int ta, int tb, int64_t M, int64_t N, int64_t K,
                 const int8_t *A, const float *sA, const int8_t *B, const float *sB, float *C)
{
    if (!gemm_shape_ok(ta, tb, M, N, K)) return -1;
    gemm_args g = {ta, tb, M, N, K, A, B, sA, sB};
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            C[i * N + j] = gemm_element(&g, i, j);
    return 0;
}

/* Selected output blocks only.  blocks holds nblk pairs (I, J); block b's
 * 32x32 binary32 result goes to out[b*1024 ...] row-major. */
int jfo_gemm_f32_blocks(int ta, int tb, int64_t M, int64_t N, int64_t K,
                        const int8_t *A, const float *sA, const int8_t *B, const float *sB,
                        const int64_t *blocks, int64_t nblk, float *out)
{
    if (!gemm_shape_ok(ta, tb, M, N, K)) return -1;
    gemm_args g = {ta, tb, M, N, K, A, B, sA, sB};
    for (int64_t b = 0; b < nblk; ++b)
        if (blocks[2 * b] < 0 || blocks[2 * b] >= M / JFO_B ||
            blocks[2 * b + 1] < 0 || blocks[2 * b + 1] >= N / JFO_B) return -2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b) {
        int64_t I = blocks[2 * b], J = blocks[2 * b + 1];
        for (int r = 0; r < JFO_B; ++r)
            for (int c = 0; c < JFO_B; ++c)
                out[b * JFO_B * JFO_B + r * JFO_B + c] =
                    gemm_element(&g, I * JFO_B + r, J * JFO_B + c);
    }
    return 0;
}

/* The int32 partial of output block (I, J) at k-block kb, 32x32 row-major. */
int jfo_gemm_partial(int ta, int tb, int64_t M, int64_t N, int64_t K,
                     const int8_t *A, const int8_t *B, int64_t I, int64_t J, int64_t kb,
                     int32_t *P)
{
    if (!gemm_shape_ok(ta, tb, M, N, K)) return -1;
    if (I < 0 || I >= M / JFO_B || J < 0 || J >= N / JFO_B || kb < 0 || kb >= K / JFO_B) return -2;
    gemm_args g = {ta, tb, M, N, K, A, B, NULL, NULL};
    for (int r = 0; r < JFO_B; ++r)
        for (int c = 0; c < JFO_B; ++c)
            P[r * JFO_B + c] = partial(&g, I * JFO_B + r, J * JFO_B + c, kb);
    return 0;
}

/* INT8 output: the binary32 result of each output block, requantized with
 * the per-block rule (the GEMM's on-chip requantization). */
int jfo_gemm_i8(int ta, int tb, int64_t M, int64_t N, int64_t K,
                const int8_t *A, const float *sA, const int8_t *B, const float *sB,
                int8_t *Cq, float *sC)
{
    if (!gemm_shape_ok(ta, tb, M, N, K)) return -1;
    gemm_args g = {ta, tb, M, N, K, A, B, sA, sB};
    const int64_t bc = N / JFO_B;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < (M / JFO_B) * bc; ++b) {
        int64_t I = b / bc, J = b % bc;
        float tile[JFO_B * JFO_B];
        for (int r = 0; r < JFO_B; ++r)
            for (int c = 0; c < JFO_B; ++c)
                tile[r * JFO_B + c] = gemm_element(&g, I * JFO_B + r, J * JFO_B + c);
        quantize_one_block(tile, JFO_B, Cq + I * JFO_B * N + J * JFO_B, N, &sC[b]);
    }
    return 0;
}

/* Selected blocks, INT8 output: codes to outq[b*1024 ...], scale to outs[b]. */
int jfo_gemm_i8_blocks(int ta, int tb, int64_t M, int64_t N, int64_t K,
                       const int8_t *A, const float *sA, const int8_t *B, const float *sB,
                       const int64_t *blocks, int64_t nblk, int8_t *outq, float *outs)
{
    if (!gemm_shape_ok(ta, tb, M, N, K)) return -1;
    gemm_args g = {ta, tb, M, N, K, A, B, sA, sB};
    for (int64_t b = 0; b < nblk; ++b)
        if (blocks[2 * b] < 0 || blocks[2 * b] >= M / JFO_B ||
            blocks[2 * b + 1] < 0 || blocks[2 * b + 1] >= N / JFO_B) return -2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b) {
        int64_t I = blocks[2 * b], J = blocks[2 * b + 1];
        float tile[JFO_B * JFO_B];
        for (int r = 0; r < JFO_B; ++r)
            for (int c = 0; c < JFO_B; ++c)
                tile[r * JFO_B + c] = gemm_element(&g, I * JFO_B + r, J * JFO_B + c);
        quantize_one_block(tile, JFO_B, outq + b * JFO_B * JFO_B, JFO_B, &outs[b]);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* INT8 -> INT8 GELU (Problem: memory-bound non-linear operators;     */
/* Approach: non-linear operators also read and write INT8 + scales). */
/* ------------------------------------------------------------------ */

/* g(x) = x * Phi(x), Phi the standard normal CDF written through erfc so the
 * negative tail keeps its relative accuracy; binary64, rounded once. */
float jfo_gelu_value(float x)
{
    double xd = (double)x;
    double g = xd * (0.5 * erfc(-xd * M_SQRT1_2));
    return (float)g;
}

int jfo_gelu(const int8_t *q, const float *s, int64_t rows, int64_t cols, int8_t *qo, float *so)
{
    if (!shape_ok(rows, cols)) return -1;
    const int64_t bc = cols / JFO_B;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < (rows / JFO_B) * bc; ++b) {
        int64_t bi = b / bc, bj = b % bc;
        float tile[JFO_B * JFO_B];
        for (int r = 0; r < JFO_B; ++r)
            for (int c = 0; c < JFO_B; ++c) {
                float x = s[b] * (float)q[(bi * JFO_B + r) * cols + bj * JFO_B + c];
                tile[r * JFO_B + c] = jfo_gelu_value(x);
            }
        quantize_one_block(tile, JFO_B, qo + bi * JFO_B * cols + bj * JFO_B, cols, &so[b]);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* INT8 GELU backward (Approach: every operator of the data flow,     */
/* the backward pass included, reads and writes INT8 with per-block   */
/* scales).  dX = dY * GELU'(X) elementwise, both inputs INT8 + 32x32 */
/* block scales over the same blocking, the product requantized per   */
/* block with the same scale/code rule.                               */
/* ------------------------------------------------------------------ */

/* GELU'(x) = Phi(x) + x * phi(x), phi(x) = exp(-x^2/2) / sqrt(2 pi);
 * binary64, rounded once to binary32. */
float jfo_gelu_grad_value(float x)
{
    double xd = (double)x;
    double cdf = 0.5 * erfc(-xd * M_SQRT1_2);
    double pdf = exp(-0.5 * xd * xd) * 0.39894228040143267794;
    return (float)(cdf + xd * pdf);
}

int jfo_gelu_bwd(const int8_t *qdy, const float *sdy, const int8_t *qx, const float *sx,
                 int64_t rows, int64_t cols, int8_t *qo, float *so)
{
    if (!shape_ok(rows, cols)) return -1;
    const int64_t bc = cols / JFO_B;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < (rows / JFO_B) * bc; ++b) {
        int64_t bi = b / bc, bj = b % bc;
        float tile[JFO_B * JFO_B];
        for (int r = 0; r < JFO_B; ++r)
            for (int c = 0; c < JFO_B; ++c) {
                int64_t at = (bi * JFO_B + r) * cols + bj * JFO_B + c;
                float dy = sdy[b] * (float)qdy[at];
                float x = sx[b] * (float)qx[at];
                tile[r * JFO_B + c] = dy * jfo_gelu_grad_value(x);
            }
        quantize_one_block(tile, JFO_B, qo + bi * JFO_B * cols + bj * JFO_B, cols, &so[b]);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Residual add and LayerNorm with INT8 in and out ("Approach": every   */
/* operator of the data flow reads and writes per-block INT8).          */
/* ------------------------------------------------------------------ */

int jfo_add(const int8_t *qa, const float *sa, const int8_t *qb, const float *sb,
            int64_t rows, int64_t cols, int8_t *qo, float *so)
{
    if (!shape_ok(rows, cols)) return -1;
    const int64_t bc = cols / JFO_B;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < (rows / JFO_B) * bc; ++b) {
        int64_t bi = b / bc, bj = b % bc;
        float tile[JFO_B * JFO_B];
        for (int r = 0; r < JFO_B; ++r)
            for (int c = 0; c < JFO_B; ++c) {
                int64_t at = (bi * JFO_B + r) * cols + bj * JFO_B + c;
                float a = sa[b] * (float)qa[at];
                float bv = sb[b] * (float)qb[at];
                tile[r * JFO_B + c] = a + bv;
            }
        quantize_one_block(tile, JFO_B, qo + bi * JFO_B * cols + bj * JFO_B, cols, &so[b]);
    }
    return 0;
}

/* mean and rstd (optional, may be NULL) receive m and r of every row. */
int jfo_layernorm(const int8_t *q, const float *s, int64_t rows, int64_t cols, const float *gamma,
                  const float *beta, float eps, int8_t *qo, float *so, double *mean, double *rstd)
{
    if (!shape_ok(rows, cols)) return -1;
    const int64_t bc = cols / JFO_B;
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (int64_t bi = 0; bi < rows / JFO_B; ++bi) {
        float *y = (float *)malloc((size_t)(JFO_B * cols) * sizeof(float));
        if (!y) { bad = 1; continue; }
        for (int r = 0; r < JFO_B; ++r) {
            const int64_t row = bi * JFO_B + r;
            double sum = 0.0;
            for (int64_t c = 0; c < cols; ++c)
                sum += (double)(s[bi * bc + c / JFO_B] * (float)q[row * cols + c]);
            const double m = sum / (double)cols;
            double sq = 0.0;
            for (int64_t c = 0; c < cols; ++c) {
                double d = (double)(s[bi * bc + c / JFO_B] * (float)q[row * cols + c]) - m;
                sq += d * d;
            }
            const double v = sq / (double)cols;
            const double rs = 1.0 / sqrt(v + (double)eps);
            if (mean) mean[row] = m;
            if (rstd) rstd[row] = rs;
            for (int64_t c = 0; c < cols; ++c) {
                double x = (double)(s[bi * bc + c / JFO_B] * (float)q[row * cols + c]);
                y[r * cols + c] = (float)(((x - m) * rs) * (double)gamma[c] + (double)beta[c]);
            }
        }
        for (int64_t bj = 0; bj < bc; ++bj)
            quantize_one_block(y + bj * JFO_B, cols, qo + bi * JFO_B * cols + bj * JFO_B, cols, &so[bi * bc + bj]);
        free(y);
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------ */
/* Quantization error by scale granularity ("Measured effects": the   */
/* per-block vs per-token and per-channel quantization-error          */
/* ablations).  The same scale/code rule on four group shapes:        */
/*   0: 32x32 blocks, 1: per token (one scale per row),               */
/*   2: per channel (one per column), 3: per tensor (one scale).      */
/* Returns the group scales (row-major over the group grid) and the   */
/* sum of squared errors sum (x - fl(s*q))^2, accumulated in binary64 */
/* (the difference of two binary32 values is exact in binary64).      */
/* ------------------------------------------------------------------ */

static int64_t group_of(int gran, int64_t rows, int64_t cols, int64_t r, int64_t c)
{
    switch (gran) {
    case 0: return (r / JFO_B) * (cols / JFO_B) + c / JFO_B;
    case 1: return r;
    case 2: return c;
    default: return 0;
    }
}

int64_t jfo_quant_groups(int gran, int64_t rows, int64_t cols)
{
    switch (gran) {
    case 0: return (rows / JFO_B) * (cols / JFO_B);
    case 1: return rows;
    case 2: return cols;
    case 3: return 1;
    default: return -1;
    }
}

int jfo_quant_sse(const float *x, int64_t rows, int64_t cols, int gran, float *s, double *sse)
{
    if (!shape_ok(rows, cols) || gran < 0 || gran > 3) return -1;
    const int64_t ng = jfo_quant_groups(gran, rows, cols);
    for (int64_t g = 0; g < ng; ++g) s[g] = 0.0f;
    /* group maxima (exact), then s = fl(max / 127) */
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int64_t g = group_of(gran, rows, cols, r, c);
            float a = fabsf(x[r * cols + c]);
            if (a > s[g]) s[g] = a;
        }
    for (int64_t g = 0; g < ng; ++g) s[g] = s[g] / 127.0f;
    /* per-row sums in parallel, then summed in row order: deterministic */
    double *rowsum = (double *)malloc((size_t)rows * sizeof(double));
    if (!rowsum) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double row = 0.0;
        for (int64_t c = 0; c < cols; ++c) {
            float sg = s[group_of(gran, rows, cols, r, c)];
            float xv = x[r * cols + c], xh = 0.0f;
            if (sg != 0.0f) {
                float v = rintf(xv / sg);
                if (v > 127.0f) v = 127.0f;
                if (v < -127.0f) v = -127.0f;
                xh = sg * v;
            }
            double d = (double)xv - (double)xh;
            row += d * d;
        }
        rowsum[r] = row;
    }
    double total = 0.0;
    for (int64_t r = 0; r < rows; ++r) total += rowsum[r];
    free(rowsum);
    *sse = total;
    return 0;
}

/* ------------------------------------------------------------------ */
/* Thread control for the timed CPU baseline.                         */
/* ------------------------------------------------------------------ */
void jfo_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
int jfo_get_threads(void) { return omp_get_max_threads(); }
