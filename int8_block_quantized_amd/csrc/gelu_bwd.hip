// gelu_bwd.hip -- INT8 GELU backward: dX = dY * GELU'(X), requantized per block.
//
// Pages: Jetfire summary, "Approach": every operator of the INT8 data flow,
// the backward pass included, reads and writes INT8 with one scale per
// 32x32 block; the non-linear operators are memory-bound ("Problem").
// GELU'(x) = Phi(x) + x phi(x) (derivative of the erf form x Phi(x)).
//
// Memory mapping as in the forward GELU: a wavefront covers a group of four
// horizontally adjacent blocks, lane l holding rows 8i + l/8 (i = 0..3),
// bytes 16(l%8)..+15 of the group row (block (l%8)/2), so every 16-byte
// load and store spans eight whole 128-byte rows.
//
// Per block, x takes at most 256 values (one per code), so GELU'(x) is
// evaluated once per code: the four blocks' 256-entry derivative tables are
// built in binary64 (rounded once to binary32: the definition), x and -x
// together from one evaluation of the normal tail (jf_gelu.h), and kept in
// LDS, 1 KiB each.
// Then per element: dy = fl(sdy*qdy), y = fl(dy * table[qx]), the block max
// |y| (DPP within rows of 16 lanes, row-swapping permutes across them),
// s = fl(max/127) and the exact codes of quant_codes.
// HBM traffic: 2 bytes in + 1 byte out per element, 12 bytes per block.
#include "jf_gelu.h"
#include "jf_group.h"
#include "jf_launch.h"

namespace jf {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const float lds_f32;

constexpr int kGroup = kGroupBlocks;   // horizontally adjacent blocks per wavefront

// GELU' at x and -x (x >= 0) in binary64, each rounded once: the scaled
// normal-tail expansion (one exp and one division; a library erfc and exp
// cost about three times as many instructions).
__device__ __forceinline__ float2 gelu_grad_pair(float x) { return gelu_grad_pair_tail(x); }

__global__ __launch_bounds__(256) void k_gelu_bwd_i8(const int8_t *__restrict__ qdy, int64_t lddy,
                                                     const float *__restrict__ sdy,
                                                     const int8_t *__restrict__ qx, int64_t ldx,
                                                     const float *__restrict__ sx, int nbc, int ngc,
                                                     int64_t ngroups, int8_t *__restrict__ qo, int64_t ldo,
                                                     float *__restrict__ so) {
    // Per wavefront: four 256-entry derivative tables (1 KiB each, 1 KiB aligned).
    __shared__ __attribute__((aligned(1024))) float tables[4][kGroup][256];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_id_uniform();
    const int r8 = lane >> 3, b = (lane & 7) >> 1, colb = (lane & 1) * 16;
    const int64_t grp_raw = (int64_t)blockIdx.x * 4 + wave;
    const int64_t grp = min(grp_raw, ngroups - 1);           // tail: re-read, never stored
    const int64_t gi = grp / ngc;
    const int gj0 = (int)(grp - gi * ngc) * kGroup;
    const int bj = min(gj0 + b, nbc - 1);

    u32x4 wy[4], wx[4];
    {
        const int8_t *py = qdy + (gi * kBlock + r8) * lddy + (int64_t)bj * kBlock + colb;
        const int8_t *px = qx + (gi * kBlock + r8) * ldx + (int64_t)bj * kBlock + colb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wy[i] = ld_stream(reinterpret_cast<const u32x4 *>(py + 8 * i * lddy));
            wx[i] = ld_stream(reinterpret_cast<const u32x4 *>(px + 8 * i * ldx));
        }
    }
    const float sdy_l = sdy[gi * nbc + bj], sx_l = sx[gi * nbc + bj];
    if (grp_raw >= ngroups) return;
    const int nb = min(kGroup, nbc - gj0);

    // Derivative tables: lane l evaluates block bt = l/16 at the pairs of
    // codes +-p, p = 8(l%16) + 1 .. 8(l%16) + 8 (x = fl(s*p) and -x; code
    // -128 comes with p = 128, whose +128 entry does not exist); code 0 is
    // GELU'(0) = 1/2 exactly.  Entries are indexed by the code's raw byte.
    {
        const int bt = lane >> 4;
        const float sxt = __uint_as_float(__builtin_amdgcn_ds_bpermute(4 * (2 * bt), (int)__float_as_uint(sx_l)));
        float *tb = tables[wave][bt];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int p = 8 * (lane & 15) + j + 1;
            const float2 g = gelu_grad_pair(sxt * (float)p);
            if (p < 128) tb[p] = g.x;
            tb[256 - p] = g.y;
        }
        if ((lane & 15) == 0) tb[0] = 0.5f;
    }

    // y = fl(dy * GELU'(x)) for the lane's 64 elements, and the block max.
    const uint32_t tbase = (uint32_t)(uintptr_t)(lds_void *)tables[wave][b];
    float y[64];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t dy4[4] = {wy[i].x, wy[i].y, wy[i].z, wy[i].w};
        const uint32_t x4[4] = {wx[i].x, wx[i].y, wx[i].z, wx[i].w};
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float gp = *reinterpret_cast<const lds_f32 *>(
                    (uintptr_t)(tbase | (((x4[d] >> (8 * k)) & 0xffu) << 2)));
                const float dy = sdy_l * (float)sbyte(dy4[d], k);
                const float v = dy * gp;
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

hipError_t launch_gelu_bwd(const int8_t *qdy, int64_t lddy, const float *sdy, const int8_t *qx, int64_t ldx,
                           const float *sx, int64_t rows, int64_t cols, int8_t *qo, int64_t ldo, float *so,
                           hipStream_t stream) {
    const int64_t nbr = rows / kBlock, nbc = cols / kBlock;
    if (nbr == 0 || nbc == 0) return hipSuccess;
    const int64_t ngc = (nbc + kGroup - 1) / kGroup, ngroups = nbr * ngc;
    const int64_t grid = (ngroups + 3) / 4;
    hipLaunchKernelGGL(k_gelu_bwd_i8, dim3((unsigned)grid), dim3(256), 0, stream, qdy, lddy, sdy, qx, ldx, sx,
                       (int)nbc, (int)ngc, ngroups, qo, ldo, so);
    return hipGetLastError();
}

}  // namespace jf
