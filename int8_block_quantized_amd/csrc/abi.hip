// abi.hip -- the C ABI of libjetfire (declared in include/jetfire.h).
//
// Every entry point validates its arguments on the host, in the order the
// header lists the status codes, before any HIP call, then enqueues its
// kernels on the caller's stream.  Nothing here allocates or synchronizes.
#include "jetfire.h"
#include "jf_launch.h"

#include <stdint.h>

namespace {

constexpr int64_t kB = 32;

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

// Bytes spanned by a rows x cols matrix of elt-byte elements with leading
// dimension ld (empty for an empty matrix).
Range span(const void *p, int64_t rows, int64_t cols, int64_t ld, int64_t elt) {
    if (rows <= 0 || cols <= 0) return {0, 0};
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, lo + (uintptr_t)(((rows - 1) * ld + cols) * elt)};
}

bool overlap(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool shape_ok(int64_t v) { return v >= 0 && v % kB == 0 && v <= (int64_t(1) << 30); }

// ld must cover the row and give a 16-byte row pitch.
bool ld_ok(int64_t ld, int64_t row_len, int64_t elt) {
    return ld >= row_len && ld <= (int64_t(1) << 36) && (ld * elt) % 16 == 0;
}

bool aligned(const void *p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }  // NULL is aligned

jf_status hip_status(hipError_t e) { return e == hipSuccess ? JF_OK : JF_ERR_HIP; }

// A pointer is required unless its matrix is empty (torch hands out NULL for
// empty tensors).  Negative sizes count as non-empty here and are rejected
// by the shape check that follows.
bool missing(const void *p, int64_t rows, int64_t cols) { return !p && !(rows == 0 || cols == 0); }

}  // namespace

extern "C" {

int jf_abi_version(void) { return JF_ABI_VERSION; }

const char *jf_status_str(jf_status st) {
    switch (st) {
        case JF_OK: return "ok";
        case JF_ERR_NULL: return "null pointer";
        case JF_ERR_SHAPE: return "size negative or not a multiple of 32";
        case JF_ERR_LD: return "leading dimension below row length or row pitch not a multiple of 16 bytes";
        case JF_ERR_ALIGN: return "pointer misaligned (matrices 16 bytes, scales 4 bytes, sums 8 bytes)";
        case JF_ERR_DTYPE: return "unknown element type or output kind";
        case JF_ERR_ARG: return "transpose flag not 0 or 1, unknown scale granularity, or bad epsilon";
        case JF_ERR_ALIAS: return "an output overlaps an input or another output";
        case JF_ERR_HIP: return "HIP kernel launch failed";
    }
    return "unknown status";
}

jf_status jf_quantize_block(jf_dtype xt, const void *x, int64_t ldx, int64_t rows, int64_t cols, int8_t *q,
                            int64_t ldq, float *s, hipStream_t stream) {
    if (missing(x, rows, cols) || missing(q, rows, cols) || missing(s, rows, cols)) return JF_ERR_NULL;
    if (!shape_ok(rows) || !shape_ok(cols)) return JF_ERR_SHAPE;
    if (xt != JF_F32 && xt != JF_BF16) return JF_ERR_DTYPE;
    const int64_t elt = xt == JF_F32 ? 4 : 2;
    if (!ld_ok(ldx, cols, elt) || !ld_ok(ldq, cols, 1)) return JF_ERR_LD;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return JF_ERR_ALIGN;
    const Range rx = span(x, rows, cols, ldx, elt), rq = span(q, rows, cols, ldq, 1);
    const Range rs = span(s, rows / kB, cols / kB, cols / kB, 4);
    if (overlap(rx, rq) || overlap(rx, rs) || overlap(rq, rs)) return JF_ERR_ALIAS;
    if (rows == 0 || cols == 0) return JF_OK;
    if (xt == JF_F32)
        return hip_status(jf::launch_quantize_f32(static_cast<const float *>(x), ldx, rows, cols, q, ldq, s, stream));
    return hip_status(jf::launch_quantize_bf16(static_cast<const uint16_t *>(x), ldx, rows, cols, q, ldq, s, stream));
}

jf_status jf_requant_block(const float *x, int64_t ldx, int64_t rows, int64_t cols, int8_t *q, int64_t ldq,
                           float *s, hipStream_t stream) {
    return jf_quantize_block(JF_F32, x, ldx, rows, cols, q, ldq, s, stream);
}

jf_status jf_dequantize_block(const int8_t *q, int64_t ldq, const float *s, int64_t rows, int64_t cols,
                              jf_dtype yt, void *y, int64_t ldy, hipStream_t stream) {
    if (missing(q, rows, cols) || missing(s, rows, cols) || missing(y, rows, cols)) return JF_ERR_NULL;
    if (!shape_ok(rows) || !shape_ok(cols)) return JF_ERR_SHAPE;
    if (yt != JF_F32 && yt != JF_BF16) return JF_ERR_DTYPE;
    const int64_t elt = yt == JF_F32 ? 4 : 2;
    if (!ld_ok(ldq, cols, 1) || !ld_ok(ldy, cols, elt)) return JF_ERR_LD;
    if (!aligned(q, 16) || !aligned(y, 16) || !aligned(s, 4)) return JF_ERR_ALIGN;
    const Range ry = span(y, rows, cols, ldy, elt);
    if (overlap(ry, span(q, rows, cols, ldq, 1)) || overlap(ry, span(s, rows / kB, cols / kB, cols / kB, 4)))
        return JF_ERR_ALIAS;
    if (rows == 0 || cols == 0) return JF_OK;
    return hip_status(jf::launch_dequantize(q, ldq, s, rows, cols, yt == JF_BF16, y, ldy, stream));
}

jf_status jf_gemm_i8_blockscaled(int transA, int transB, int64_t M, int64_t N, int64_t K, const int8_t *A,
                                 int64_t lda, const float *sA, const int8_t *B, int64_t ldb, const float *sB,
                                 jf_out out, void *C, int64_t ldc, float *sC, hipStream_t stream) {
    if (missing(A, M, K) || missing(sA, M, K) || missing(B, K, N) || missing(sB, K, N) || missing(C, M, N))
        return JF_ERR_NULL;
    if (out == JF_OUT_I8 && missing(sC, M, N)) return JF_ERR_NULL;
    if (!shape_ok(M) || !shape_ok(N) || !shape_ok(K)) return JF_ERR_SHAPE;
    if (out != JF_OUT_I8 && out != JF_OUT_F32) return JF_ERR_DTYPE;
    if ((transA != 0 && transA != 1) || (transB != 0 && transB != 1)) return JF_ERR_ARG;
    // stored shapes
    const int64_t a_rows = transA ? K : M, a_cols = transA ? M : K;
    const int64_t b_rows = transB ? N : K, b_cols = transB ? K : N;
    const int64_t c_elt = out == JF_OUT_F32 ? 4 : 1;
    if (!ld_ok(lda, a_cols, 1) || !ld_ok(ldb, b_cols, 1) || !ld_ok(ldc, N, c_elt)) return JF_ERR_LD;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(sA, 4) || !aligned(sB, 4) ||
        (out == JF_OUT_I8 && !aligned(sC, 4)))
        return JF_ERR_ALIGN;
    const Range ra = span(A, a_rows, a_cols, lda, 1), rb = span(B, b_rows, b_cols, ldb, 1);
    const Range rsa = span(sA, a_rows / kB, a_cols / kB, a_cols / kB, 4);
    const Range rsb = span(sB, b_rows / kB, b_cols / kB, b_cols / kB, 4);
    const Range rc = span(C, M, N, ldc, c_elt);
    const Range rsc = out == JF_OUT_I8 ? span(sC, M / kB, N / kB, N / kB, 4) : Range{0, 0};
    for (Range in : {ra, rb, rsa, rsb})
        if (overlap(rc, in) || overlap(rsc, in)) return JF_ERR_ALIAS;
    if (overlap(rc, rsc)) return JF_ERR_ALIAS;
    if (M == 0 || N == 0) return JF_OK;
    return hip_status(jf::launch_gemm(transA, transB, M, N, K, A, lda, sA, B, ldb, sB, out == JF_OUT_I8, C, ldc,
                                      sC, stream));
}

jf_status jf_gelu_i8(const int8_t *q, int64_t ldq, const float *s, int64_t rows, int64_t cols, int8_t *qo,
                     int64_t ldqo, float *so, hipStream_t stream) {
    if (missing(q, rows, cols) || missing(s, rows, cols) || missing(qo, rows, cols) || missing(so, rows, cols))
        return JF_ERR_NULL;
    if (!shape_ok(rows) || !shape_ok(cols)) return JF_ERR_SHAPE;
    if (!ld_ok(ldq, cols, 1) || !ld_ok(ldqo, cols, 1)) return JF_ERR_LD;
    if (!aligned(q, 16) || !aligned(qo, 16) || !aligned(s, 4) || !aligned(so, 4)) return JF_ERR_ALIGN;
    const Range rq = span(q, rows, cols, ldq, 1), rqo = span(qo, rows, cols, ldqo, 1);
    const Range rs = span(s, rows / kB, cols / kB, cols / kB, 4), rso = span(so, rows / kB, cols / kB, cols / kB, 4);
    for (Range in : {rq, rs})
        if (overlap(rqo, in) || overlap(rso, in)) return JF_ERR_ALIAS;
    if (overlap(rqo, rso)) return JF_ERR_ALIAS;
    if (rows == 0 || cols == 0) return JF_OK;
    return hip_status(jf::launch_gelu(q, ldq, s, rows, cols, qo, ldqo, so, stream));
}

jf_status jf_gelu_bwd_i8(const int8_t *qdy, int64_t lddy, const float *sdy, const int8_t *qx, int64_t ldx,
                         const float *sx, int64_t rows, int64_t cols, int8_t *qo, int64_t ldo, float *so,
                         hipStream_t stream) {
    if (missing(qdy, rows, cols) || missing(sdy, rows, cols) || missing(qx, rows, cols) ||
        missing(sx, rows, cols) || missing(qo, rows, cols) || missing(so, rows, cols))
        return JF_ERR_NULL;
    if (!shape_ok(rows) || !shape_ok(cols)) return JF_ERR_SHAPE;
    if (!ld_ok(lddy, cols, 1) || !ld_ok(ldx, cols, 1) || !ld_ok(ldo, cols, 1)) return JF_ERR_LD;
    if (!aligned(qdy, 16) || !aligned(qx, 16) || !aligned(qo, 16) || !aligned(sdy, 4) || !aligned(sx, 4) ||
        !aligned(so, 4))
        return JF_ERR_ALIGN;
    const int64_t gr = rows / kB, gc = cols / kB;
    const Range rqo = span(qo, rows, cols, ldo, 1), rso = span(so, gr, gc, gc, 4);
    for (Range in : {span(qdy, rows, cols, lddy, 1), span(qx, rows, cols, ldx, 1), span(sdy, gr, gc, gc, 4),
                     span(sx, gr, gc, gc, 4)})
        if (overlap(rqo, in) || overlap(rso, in)) return JF_ERR_ALIAS;
    if (overlap(rqo, rso)) return JF_ERR_ALIAS;
    if (rows == 0 || cols == 0) return JF_OK;
    return hip_status(jf::launch_gelu_bwd(qdy, lddy, sdy, qx, ldx, sx, rows, cols, qo, ldo, so, stream));
}

jf_status jf_add_i8(const int8_t *qa, int64_t lda, const float *sa, const int8_t *qb, int64_t ldb, const float *sb,
                    int64_t rows, int64_t cols, int8_t *qo, int64_t ldo, float *so, hipStream_t stream) {
    if (missing(qa, rows, cols) || missing(sa, rows, cols) || missing(qb, rows, cols) || missing(sb, rows, cols) ||
        missing(qo, rows, cols) || missing(so, rows, cols))
        return JF_ERR_NULL;
    if (!shape_ok(rows) || !shape_ok(cols)) return JF_ERR_SHAPE;
    if (!ld_ok(lda, cols, 1) || !ld_ok(ldb, cols, 1) || !ld_ok(ldo, cols, 1)) return JF_ERR_LD;
    if (!aligned(qa, 16) || !aligned(qb, 16) || !aligned(qo, 16) || !aligned(sa, 4) || !aligned(sb, 4) ||
        !aligned(so, 4))
        return JF_ERR_ALIGN;
    const int64_t gr = rows / kB, gc = cols / kB;
    const Range rqo = span(qo, rows, cols, ldo, 1), rso = span(so, gr, gc, gc, 4);
    for (Range in : {span(qa, rows, cols, lda, 1), span(sa, gr, gc, gc, 4), span(qb, rows, cols, ldb, 1),
                     span(sb, gr, gc, gc, 4)})
        if (overlap(rqo, in) || overlap(rso, in)) return JF_ERR_ALIAS;
    if (overlap(rqo, rso)) return JF_ERR_ALIAS;
    if (rows == 0 || cols == 0) return JF_OK;
    return hip_status(jf::launch_add(qa, lda, sa, qb, ldb, sb, rows, cols, qo, ldo, so, stream));
}

jf_status jf_layernorm_i8(const int8_t *q, int64_t ldq, const float *s, int64_t rows, int64_t cols,
                          const float *gamma, const float *beta, float eps, int8_t *qo, int64_t ldo, float *so,
                          double *mean, double *rstd, hipStream_t stream) {
    if (missing(q, rows, cols) || missing(s, rows, cols) || missing(gamma, rows, cols) ||
        missing(beta, rows, cols) || missing(qo, rows, cols) || missing(so, rows, cols))
        return JF_ERR_NULL;
    if (!shape_ok(rows) || !shape_ok(cols)) return JF_ERR_SHAPE;
    if (!ld_ok(ldq, cols, 1) || !ld_ok(ldo, cols, 1)) return JF_ERR_LD;
    if (!aligned(q, 16) || !aligned(qo, 16) || !aligned(gamma, 16) || !aligned(beta, 16) || !aligned(s, 4) ||
        !aligned(so, 4) || !aligned(mean, 8) || !aligned(rstd, 8))
        return JF_ERR_ALIGN;
    if (!(eps >= 0.0f) || !(eps < __builtin_inff())) return JF_ERR_ARG;
    const int64_t gr = rows / kB, gc = cols / kB;
    const Range rqo = span(qo, rows, cols, ldo, 1), rso = span(so, gr, gc, gc, 4);
    const Range rm = mean ? span(mean, 1, rows, rows, 8) : Range{0, 0};
    const Range rr = rstd ? span(rstd, 1, rows, rows, 8) : Range{0, 0};
    for (Range in : {span(q, rows, cols, ldq, 1), span(s, gr, gc, gc, 4), span(gamma, 1, cols, cols, 4),
                     span(beta, 1, cols, cols, 4)})
        if (overlap(rqo, in) || overlap(rso, in) || overlap(rm, in) || overlap(rr, in)) return JF_ERR_ALIAS;
    if (overlap(rqo, rso) || overlap(rqo, rm) || overlap(rqo, rr) || overlap(rso, rm) || overlap(rso, rr) ||
        overlap(rm, rr))
        return JF_ERR_ALIAS;
    if (rows == 0 || cols == 0) return JF_OK;
    return hip_status(jf::launch_layernorm(q, ldq, s, rows, cols, gamma, beta, eps, qo, ldo, so, mean, rstd,
                                           stream));
}

jf_status jf_quant_error(const float *x, int64_t ldx, int64_t rows, int64_t cols, int granularity, float *s,
                         double *sse, hipStream_t stream) {
    // number of scales; an unknown granularity needs s too (rejected below)
    const bool known = granularity >= JF_GRAN_BLOCK && granularity <= JF_GRAN_TENSOR;
    const int64_t ng = granularity == JF_GRAN_BLOCK ? (rows / kB) * (cols / kB)
                       : granularity == JF_GRAN_TOKEN ? rows
                       : granularity == JF_GRAN_CHANNEL ? cols
                                                        : 1;
    if (missing(x, rows, cols) || !sse || (!s && (ng != 0 || !known))) return JF_ERR_NULL;
    if (!shape_ok(rows) || !shape_ok(cols)) return JF_ERR_SHAPE;
    if (!ld_ok(ldx, cols, 4)) return JF_ERR_LD;
    if (!aligned(x, 16) || !aligned(s, 4) || !aligned(sse, 8)) return JF_ERR_ALIGN;
    if (!known) return JF_ERR_ARG;
    const Range rx = span(x, rows, cols, ldx, 4), rs = span(s, 1, ng, ng, 4), re = span(sse, 1, 1, 1, 8);
    if (overlap(rx, rs) || overlap(rx, re) || overlap(rs, re)) return JF_ERR_ALIAS;
    return hip_status(jf::launch_quant_error(x, ldx, rows, cols, granularity, s, sse, stream));
}

}  // extern "C"
