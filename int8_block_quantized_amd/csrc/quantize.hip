// quantize.hip -- per-block (32x32) INT8 quantization and requantization.
//
// Pages: Jetfire summary, one-line summary and "Approach": tensors travel as
// INT8 codes with one scale per 32x32 block, quantized on-chip.  This kernel
// is the HBM-bound entry into that data flow: fp32/bf16 in, codes + scales
// out, in one pass (4 B or 2 B read + 1 B written per element + 4 B per
// block).  jf_requant_block uses the fp32 instantiation: it is the same rule
// as the GEMM's requantizing epilogue.
//
// Mapping: one wavefront per 32x32 block, the four wavefronts of a
// workgroup on four horizontally adjacent blocks, so a workgroup reads whole
// 512-byte row segments and writes whole 128-byte code rows.  Plain (not
// non-temporal) loads and stores: measured faster here.  Within a block, lane l holds rows
// 8t + l/8 (t = 0..3), columns 4(l%8)..4(l%8)+3: each load instruction
// covers eight whole 128-byte block rows.  The block max is a DPP reduction;
// codes come from quant_codes (no division per element).
#include "jf_device.h"
#include "jf_launch.h"

namespace jf {
namespace {

constexpr int kPerWave = 1;   // blocks per wavefront (more only lowers occupancy)

template <typename T>
struct Row4;

template <>
struct Row4<float> {
    static __device__ __forceinline__ void load(const float *p, float *v) {
        const f32x4 f = *reinterpret_cast<const f32x4 *>(p);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    }
};

template <>
struct Row4<uint16_t> {
    // bfloat16 -> binary32 is exact: the 16 bits become the high half.
    static __device__ __forceinline__ void load(const uint16_t *p, float *v) {
        const u32x2 w = *reinterpret_cast<const u32x2 *>(p);
        v[0] = __uint_as_float(w.x << 16);
        v[1] = __uint_as_float(w.x & 0xffff0000u);
        v[2] = __uint_as_float(w.y << 16);
        v[3] = __uint_as_float(w.y & 0xffff0000u);
    }
};

template <typename T>
__global__ __launch_bounds__(256) void k_quantize_block(const T *__restrict__ x, int64_t ldx,
                                                        int64_t nblk, int nbc,
                                                        int8_t *__restrict__ q, int64_t ldq,
                                                        float *__restrict__ s) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t first = ((int64_t)blockIdx.x * 4 + wave_id_uniform()) * kPerWave;
    const int r0 = lane >> 3, c0 = (lane & 7) * 4;

    float v[kPerWave][16];
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
        const int64_t blk = min(first + i, nblk - 1);   // tail: re-read, never stored
        const int64_t bi = blk / nbc, bj = blk - bi * nbc;
        const T *xb = x + bi * kBlock * ldx + bj * kBlock + c0;
#pragma unroll
        for (int t = 0; t < 4; ++t) Row4<T>::load(xb + (int64_t)(8 * t + r0) * ldx, &v[i][4 * t]);
    }

#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
        const int64_t blk = first + i;
        if (blk >= nblk) break;
        const int64_t bi = blk / nbc, bj = blk - bi * nbc;
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[i][e]));
        m = wave_max_nonneg(m);
        const float sc = block_scale(m);
        int code[16];
        if (sc != 0.0f) {
            quant_codes(v[i], sc, code);
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) code[e] = 0;
        }
        int8_t *qb = q + bi * kBlock * ldq + bj * kBlock + c0;
#pragma unroll
        for (int t = 0; t < 4; ++t)
            *reinterpret_cast<uint32_t *>(qb + (int64_t)(8 * t + r0) * ldq) =
                pack4(code[4 * t], code[4 * t + 1], code[4 * t + 2], code[4 * t + 3]);
        if (lane == 0) s[blk] = sc;
    }
}

template <typename T>
hipError_t launch(const T *x, int64_t ldx, int64_t rows, int64_t cols, int8_t *q, int64_t ldq,
                  float *s, hipStream_t stream) {
    const int64_t nbr = rows / kBlock, nbc = cols / kBlock, nblk = nbr * nbc;
    if (nblk == 0) return hipSuccess;
    const int64_t per_wg = 4 * kPerWave;
    const int64_t grid = (nblk + per_wg - 1) / per_wg;
    hipLaunchKernelGGL(k_quantize_block<T>, dim3((unsigned)grid), dim3(256), 0, stream, x, ldx, nblk,
                       (int)nbc, q, ldq, s);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_f32(const float *x, int64_t ldx, int64_t rows, int64_t cols, int8_t *q,
                               int64_t ldq, float *s, hipStream_t stream) {
    return launch<float>(x, ldx, rows, cols, q, ldq, s, stream);
}

hipError_t launch_quantize_bf16(const uint16_t *x, int64_t ldx, int64_t rows, int64_t cols,
                                int8_t *q, int64_t ldq, float *s, hipStream_t stream) {
    return launch<uint16_t>(x, ldx, rows, cols, q, ldq, s, stream);
}

}  // namespace jf
