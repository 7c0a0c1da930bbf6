// dequant.hip -- per-block INT8 codes + scales back to binary32 or bfloat16.
//
// Pages: Jetfire summary, "Approach" (INT8 tensors carry one scale per 32x32
// block); the dequantized value of a code q in a block of scale s is
// x = fl(s*q) in binary32.  The bfloat16 form rounds that binary32 value to
// the nearest bfloat16, ties to even (a copy for checking and for consumers
// outside the INT8 data flow).
//
// Mapping: a thread takes kUnits units of E consecutive codes of one row,
// E = 8 for bfloat16 output and 4 for binary32, so that a unit's output is
// 16 bytes; consecutive threads take consecutive units, so every store
// instruction of a wavefront writes 1 KiB of contiguous output (whole cache
// lines, no partially written line left for another instruction) and every
// load instruction reads 64 E contiguous codes.  All of a thread's loads are
// issued before its first store.  HBM traffic per element: 1 byte in, 4
// (binary32) or 2 (bfloat16) bytes out, plus 4 bytes of scale per 1024
// elements.
#include "jf_device.h"
#include "jf_launch.h"

namespace jf {
namespace {

constexpr int kUnits = 4;
constexpr int kThreads = 256;

// Nearest bfloat16 of a finite binary32 value, ties to even: add half a
// bfloat16 ulp minus one, plus the kept part's lowest bit, and truncate.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Idx: the unit index type, 32-bit whenever the launch's unit count fits
// (the row / column split of a unit index is a division by the units per
// row, several times cheaper in 32 bits).
template <bool BF16, typename Idx>
__global__ __launch_bounds__(kThreads) void k_dequant_block(const int8_t *__restrict__ q, int64_t ldq,
                                                            const float *__restrict__ s, Idx units_per_row,
                                                            Idx nunits, void *__restrict__ y, int64_t ldy) {
    constexpr int E = BF16 ? 8 : 4;   // codes per unit (16 bytes of output)
    using In = typename std::conditional<BF16, u32x2, uint32_t>::type;
    const Idx t = (Idx)blockIdx.x * kThreads + threadIdx.x;
    const Idx stride = (Idx)gridDim.x * kThreads;
    const Idx nbc = units_per_row * E / kBlock;   // 32-column blocks per row
    Idx u[kUnits], r[kUnits], c[kUnits];
    In w[kUnits];
    float sc[kUnits];
#pragma unroll
    for (int k = 0; k < kUnits; ++k) {
        u[k] = t + k * stride;
        const Idx uc = min(u[k], nunits - 1);       // tail: re-read, never stored
        r[k] = uc / units_per_row;
        c[k] = (uc - r[k] * units_per_row) * E;     // first column of the unit
        w[k] = ld_stream(reinterpret_cast<const In *>(q + (int64_t)r[k] * ldq + c[k]));
        sc[k] = s[(r[k] / kBlock) * nbc + c[k] / kBlock];
    }
#pragma unroll
    for (int k = 0; k < kUnits; ++k) {
        if (u[k] >= nunits) break;
        uint32_t wd[E / 4];
        if constexpr (BF16) {
            wd[0] = w[k].x;
            wd[1] = w[k].y;
        } else {
            wd[0] = w[k];
        }
        float v[E];
#pragma unroll
        for (int d = 0; d < E / 4; ++d)
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * d + e] = sc[k] * (float)sbyte(wd[d], e);
        if constexpr (BF16) {
            u32x4 o;
            o.x = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
            o.y = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
            o.z = bf16_bits(v[4]) | (bf16_bits(v[5]) << 16);
            o.w = bf16_bits(v[6]) | (bf16_bits(v[7]) << 16);
            st_stream(reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(y) + (int64_t)r[k] * ldy + c[k]), o);
        } else {
            st_stream(reinterpret_cast<f32x4 *>(static_cast<float *>(y) + (int64_t)r[k] * ldy + c[k]),
                      f32x4{v[0], v[1], v[2], v[3]});
        }
    }
}

}  // namespace

hipError_t launch_dequantize(const int8_t *q, int64_t ldq, const float *s, int64_t rows, int64_t cols, bool bf16,
                             void *y, int64_t ldy, hipStream_t stream) {
    const int64_t E = bf16 ? 8 : 4, units_per_row = cols / E, nunits = rows * units_per_row;
    if (nunits == 0) return hipSuccess;
    const int64_t per_wg = (int64_t)kThreads * kUnits;
    const dim3 grid((unsigned)((nunits + per_wg - 1) / per_wg)), block(kThreads);
    // 32-bit indices when every unit index a thread forms (up to grid * per_wg) fits
    const bool narrow = (int64_t)grid.x * per_wg < (int64_t(1) << 31);
    if (bf16 && narrow)
        hipLaunchKernelGGL((k_dequant_block<true, uint32_t>), grid, block, 0, stream, q, ldq, s,
                           (uint32_t)units_per_row, (uint32_t)nunits, y, ldy);
    else if (bf16)
        hipLaunchKernelGGL((k_dequant_block<true, int64_t>), grid, block, 0, stream, q, ldq, s, units_per_row,
                           nunits, y, ldy);
    else if (narrow)
        hipLaunchKernelGGL((k_dequant_block<false, uint32_t>), grid, block, 0, stream, q, ldq, s,
                           (uint32_t)units_per_row, (uint32_t)nunits, y, ldy);
    else
        hipLaunchKernelGGL((k_dequant_block<false, int64_t>), grid, block, 0, stream, q, ldq, s, units_per_row,
                           nunits, y, ldy);
    return hipGetLastError();
}

}  // namespace jf
