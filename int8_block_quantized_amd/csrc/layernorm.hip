// layernorm.hip -- LayerNorm over each row of a per-block INT8 tensor,
// requantized per block (INT8 in, INT8 out).
//
// Pages: Jetfire summary, "Approach": every operator of the data flow reads
// and writes INT8 with one scale per 32x32 block.  Per row (the hidden
// dimension, n columns): x = fl(s*q); mean m = sum(x)/n and biased variance
// v = sum((x - m)^2)/n in binary64; r = 1/sqrt(v + eps) in binary64;
// y = ((x - m)*r)*gamma + beta in binary64, rounded once to binary32; then
// the per-block rule on y (s = fl(max|y|/127), exact codes).
//
// One workgroup of 16 wavefronts per 32-row strip (one block row).  Each
// wavefront takes groups of four adjacent blocks (the jf_group.h mapping),
// group g = wave + 16k; the strip's codes stay in registers for rows of up
// to 32 groups (4096 columns) and are re-read for each pass beyond that.
// Three passes: row sums, sums of squared deviations (lane partials in
// binary64, reduced over the 8 lanes of a row with DPP and over the
// wavefronts through LDS in wavefront order), then y, block maxima, codes.
// HBM traffic: 1 byte in + 1 byte out per element, 8 bytes of scales per
// block, gamma and beta once per strip (cached).
#include "jf_group.h"
#include "jf_launch.h"

namespace jf {
namespace {

constexpr int kLnWaves = 16;

template <int CTRL>
__device__ __forceinline__ double dpp64(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = dpp<CTRL>((uint32_t)u), hi = dpp<CTRL>((uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Sum over the 8 lanes sharing l/8 (one row of the group); every one of
// them receives the same value.
__device__ __forceinline__ double row_sum8(double v) {
    v += dpp64<kDppXor1>(v);
    v += dpp64<kDppXor2>(v);
    v += dpp64<kDppHalfMirror>(v);
    return v;
}

template <int GPW>
__global__ __launch_bounds__(1024) void k_layernorm_i8(const int8_t *__restrict__ q, int64_t ldq,
                                                       const float *__restrict__ s, int nbc, int ngc, int64_t cols,
                                                       const float *__restrict__ gamma,
                                                       const float *__restrict__ beta, float eps,
                                                       int8_t *__restrict__ qo, int64_t ldo, float *__restrict__ so,
                                                       double *__restrict__ mean_out, double *__restrict__ rstd_out) {
    __shared__ double part[kLnWaves][kBlock];
    __shared__ double stat[2][kBlock];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_id_uniform();
    const int r8 = lane >> 3, b = (lane & 7) >> 1, colb = (lane & 1) * 16;
    const int64_t bi = blockIdx.x;
    const int8_t *qrow = q + (bi * kBlock + r8) * ldq + colb;

    auto load = [&](int g, u32x4 (&w)[4]) {
        const int bj = min(kGroupBlocks * g + b, nbc - 1);
        const int8_t *p = qrow + (int64_t)bj * kBlock;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = *reinterpret_cast<const u32x4 *>(p + 8 * i * ldq);
    };
    u32x4 regs[GPW > 0 ? GPW : 1][4];
    if constexpr (GPW > 0) {
#pragma unroll
        for (int k = 0; k < GPW; ++k)
            if (wave + kLnWaves * k < ngc) load(wave + kLnWaves * k, regs[k]);
    }
    // f(g, codes) over the wavefront's groups (wave-uniform control flow)
    auto for_groups = [&](auto &&f) {
        if constexpr (GPW > 0) {
#pragma unroll
            for (int k = 0; k < GPW; ++k)
                if (wave + kLnWaves * k < ngc) f(wave + kLnWaves * k, regs[k]);
        } else {
            for (int g = wave; g < ngc; g += kLnWaves) {
                u32x4 w[4];
                load(g, w);
                f(g, w);
            }
        }
    };
    auto lane_scale = [&](int g) { return s[bi * nbc + min(kGroupBlocks * g + b, nbc - 1)]; };
    auto lane_valid = [&](int g) { return kGroupBlocks * g + b < nbc; };

    // Row statistic: lane partials -> 8-lane row sums -> per-wavefront
    // partials in LDS -> 32 threads add the 16 partials in wavefront order.
    auto reduce_rows = [&](const double (&acc)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double v = row_sum8(acc[i]);
            if ((lane & 7) == 0) part[wave][8 * i + r8] = v;
        }
        __syncthreads();
    };
    auto row_total = [&](int row) {
        double t = 0.0;
#pragma unroll
        for (int w = 0; w < kLnWaves; ++w) t += part[w][row];
        return t;
    };

    // pass 1: mean
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for_groups([&](int g, const u32x4 (&w)[4]) {
        if (!lane_valid(g)) return;
        const float sc = lane_scale(g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w4[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int k = 0; k < 4; ++k) acc[i] += (double)(sc * (float)sbyte(w4[d], k));
        }
    });
    reduce_rows(acc);
    if (threadIdx.x < kBlock) stat[0][threadIdx.x] = row_total(threadIdx.x) / (double)cols;
    __syncthreads();
    double mrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mrow[i] = stat[0][8 * i + r8];

    // pass 2: biased variance -> 1/sqrt(v + eps)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = 0.0;
    for_groups([&](int g, const u32x4 (&w)[4]) {
        if (!lane_valid(g)) return;
        const float sc = lane_scale(g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w4[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const double dv = (double)(sc * (float)sbyte(w4[d], k)) - mrow[i];
                    acc[i] += dv * dv;
                }
        }
    });
    reduce_rows(acc);
    if (threadIdx.x < kBlock) {
        const double v = row_total(threadIdx.x) / (double)cols;
        const double r = 1.0 / sqrt(v + (double)eps);
        stat[1][threadIdx.x] = r;
        const int64_t row = bi * kBlock + threadIdx.x;
        if (mean_out) mean_out[row] = stat[0][threadIdx.x];
        if (rstd_out) rstd_out[row] = r;
    }
    __syncthreads();

    // pass 3: y, block maxima, codes
    for_groups([&](int g, const u32x4 (&w)[4]) {
        const float sc = lane_scale(g);
        const int bj = min(kGroupBlocks * g + b, nbc - 1);
        const int64_t c0 = (int64_t)bj * kBlock + colb;
        float y[64];
        float mx = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const f32x4 gm = *reinterpret_cast<const f32x4 *>(gamma + c0 + 4 * d);
            const f32x4 bt = *reinterpret_cast<const f32x4 *>(beta + c0 + 4 * d);
            const float gk[4] = {gm.x, gm.y, gm.z, gm.w}, bk[4] = {bt.x, bt.y, bt.z, bt.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t wd = d == 0 ? w[i].x : d == 1 ? w[i].y : d == 2 ? w[i].z : w[i].w;
                // the row's mean and 1/sqrt(v + eps), read where used
                const double mi = stat[0][8 * i + r8], ri = stat[1][8 * i + r8];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const double x = (double)(sc * (float)sbyte(wd, k));
                    const float v = (float)(((x - mi) * ri) * (double)gk[k] + (double)bk[k]);
                    y[16 * i + 4 * d + k] = v;
                    mx = fmaxf(mx, fabsf(v));
                }
            }
        }
        const float sown = block_scale(group_own_block_max(mx));   // the lane's block's output scale
        const int gj0 = kGroupBlocks * g;
        if (lane_valid(g))
            store_group_codes(y, sown, qo + (bi * kBlock + r8) * ldo + (int64_t)(gj0 + b) * kBlock + colb, ldo);
        if ((lane & 1) == 0 && lane < 2 * min(kGroupBlocks, nbc - gj0))
            so[bi * nbc + gj0 + (lane >> 1)] = sown;   // lanes 0, 2, 4, 6 hold blocks 0..3
    });
}

}  // namespace

hipError_t launch_layernorm(const int8_t *q, int64_t ldq, const float *s, int64_t rows, int64_t cols,
                            const float *gamma, const float *beta, float eps, int8_t *qo, int64_t ldo, float *so,
                            double *mean, double *rstd, hipStream_t stream) {
    const int64_t nbr = rows / kBlock, nbc = cols / kBlock;
    if (nbr == 0 || nbc == 0) return hipSuccess;
    const int64_t ngc = (nbc + kGroupBlocks - 1) / kGroupBlocks;
    const dim3 grid((unsigned)nbr), block(kWave * kLnWaves);
    if (ngc <= kLnWaves)
        hipLaunchKernelGGL(k_layernorm_i8<1>, grid, block, 0, stream, q, ldq, s, (int)nbc, (int)ngc, cols, gamma,
                           beta, eps, qo, ldo, so, mean, rstd);
    else if (ngc <= 2 * kLnWaves)
        hipLaunchKernelGGL(k_layernorm_i8<2>, grid, block, 0, stream, q, ldq, s, (int)nbc, (int)ngc, cols, gamma,
                           beta, eps, qo, ldo, so, mean, rstd);
    else
        hipLaunchKernelGGL(k_layernorm_i8<0>, grid, block, 0, stream, q, ldq, s, (int)nbc, (int)ngc, cols, gamma,
                           beta, eps, qo, ldo, so, mean, rstd);
    return hipGetLastError();
}

}  // namespace jf
