// add.hip -- residual add of two per-block INT8 tensors, requantized per block.
//
// Pages: Jetfire summary, "Approach": every operator of the data flow reads
// and writes INT8 with one scale per 32x32 block.  The add: both operands
// share the 32x32 blocking; per element z = fl(fl(sa*qa) + fl(sb*qb)), then
// s = fl(max|z|/127) per block and the exact codes of quant_codes.
// Mapping: jf_group.h (four adjacent blocks per wavefront).  HBM traffic:
// 2 bytes in + 1 byte out per element, 12 bytes of scales per block.
#include "jf_group.h"
#include "jf_launch.h"

namespace jf {
namespace {

__global__ __launch_bounds__(256) void k_add_i8(const int8_t *__restrict__ qa, int64_t lda,
                                                const float *__restrict__ sa, const int8_t *__restrict__ qb,
                                                int64_t ldb, const float *__restrict__ sb, int nbc, int ngc,
                                                int64_t ngroups, int8_t *__restrict__ qo, int64_t ldo,
                                                float *__restrict__ so) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_id_uniform();
    const int r8 = lane >> 3, b = (lane & 7) >> 1, colb = (lane & 1) * 16;
    const int64_t grp_raw = (int64_t)blockIdx.x * 4 + wave;
    const int64_t grp = min(grp_raw, ngroups - 1);           // tail: re-read, never stored
    const int64_t gi = grp / ngc;
    const int gj0 = (int)(grp - gi * ngc) * kGroupBlocks;
    const int bj = min(gj0 + b, nbc - 1);

    u32x4 wa[4], wb[4];
    {
        const int8_t *pa = qa + (gi * kBlock + r8) * lda + (int64_t)bj * kBlock + colb;
        const int8_t *pb = qb + (gi * kBlock + r8) * ldb + (int64_t)bj * kBlock + colb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wa[i] = ld_stream(reinterpret_cast<const u32x4 *>(pa + 8 * i * lda));
            wb[i] = ld_stream(reinterpret_cast<const u32x4 *>(pb + 8 * i * ldb));
        }
    }
    const float sa_l = sa[gi * nbc + bj], sb_l = sb[gi * nbc + bj];
    if (grp_raw >= ngroups) return;
    const int nb = min(kGroupBlocks, nbc - gj0);

    float y[64];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t a4[4] = {wa[i].x, wa[i].y, wa[i].z, wa[i].w};
        const uint32_t b4[4] = {wb[i].x, wb[i].y, wb[i].z, wb[i].w};
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float xa = sa_l * (float)sbyte(a4[d], k);
                const float xb = sb_l * (float)sbyte(b4[d], k);
                const float v = xa + xb;
                y[16 * i + 4 * d + k] = v;
                m = fmaxf(m, fabsf(v));
            }
    }
    const float sown = block_scale(group_own_block_max(m));   // the lane's block's output scale
    if (gj0 + b < nbc)
        store_group_codes(y, sown, qo + (gi * kBlock + r8) * ldo + (int64_t)(gj0 + b) * kBlock + colb, ldo);
    if ((lane & 1) == 0 && lane < 2 * nb) so[gi * nbc + gj0 + (lane >> 1)] = sown;   // lanes 0, 2, 4, 6
}

}  // namespace

hipError_t launch_add(const int8_t *qa, int64_t lda, const float *sa, const int8_t *qb, int64_t ldb,
                      const float *sb, int64_t rows, int64_t cols, int8_t *qo, int64_t ldo, float *so,
                      hipStream_t stream) {
    const int64_t nbr = rows / kBlock, nbc = cols / kBlock;
    if (nbr == 0 || nbc == 0) return hipSuccess;
    const int64_t ngc = (nbc + kGroupBlocks - 1) / kGroupBlocks, ngroups = nbr * ngc;
    const int64_t grid = (ngroups + 3) / 4;
    hipLaunchKernelGGL(k_add_i8, dim3((unsigned)grid), dim3(256), 0, stream, qa, lda, sa, qb, ldb, sb, (int)nbc,
                       (int)ngc, ngroups, qo, ldo, so);
    return hipGetLastError();
}

}  // namespace jf
