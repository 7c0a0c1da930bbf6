// quantize.hip -- per-block (32x32) INT8 quantization and requantization.
//
// Pages: Jetfire summary, one-line summary and "Approach": tensors travel as
// INT8 codes with one scale per 32x32 block, quantized on-chip.  This kernel
// is the HBM-bound entry into that data flow: fp32/bf16 in, codes + scales
// out, in one pass (4 B or 2 B read + 1 B written per element + 4 B per
// block).  jf_requant_block uses the fp32 instantiation: it is the same rule
// as the GEMM's requantizing epilogue.
//
// Mapping: a wavefront takes a group of four horizontally adjacent blocks.
// Lane l holds rows 2i + l/32 (i = 0..15), elements 4(l%32)..4(l%32)+3 of the
// group row: all inside block (l%32)/8.  Each load instruction reads two whole
// group rows (2 x 512 bytes of fp32) and each store writes two whole 128-byte
// code rows, so every HBM line is touched by one instruction.  The block max
// is a DPP reduction over the block's 16 lanes plus two readlanes; codes come
// from quant_codes (no division per element).
#include "jf_device.h"
#include "jf_launch.h"

namespace jf {
namespace {

constexpr int kGroup = 4;   // horizontally adjacent blocks per wavefront

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
__global__ __launch_bounds__(256) void k_quantize_block(const T *__restrict__ x, int64_t ldx, int nbc, int ngc,
                                                        int64_t ngroups, int8_t *__restrict__ q, int64_t ldq,
                                                        float *__restrict__ s) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t grp_raw = (int64_t)blockIdx.x * 4 + wave_id_uniform();
    const int64_t grp = min(grp_raw, ngroups - 1);          // tail: re-read, never stored
    const int64_t gi = grp / ngc;
    const int gj0 = (int)(grp - gi * ngc) * kGroup;
    const int b = (lane & 31) >> 3, r2 = lane >> 5;
    const int bj = min(gj0 + b, nbc - 1);
    const int c0 = bj * kBlock + 4 * (lane & 7);

    float v[16][4];
    const T *src = x + (gi * kBlock + r2) * ldx + c0;
#pragma unroll
    for (int i = 0; i < 16; ++i) Row4<T>::load(src + 2 * i * ldx, v[i]);
    if (grp_raw >= ngroups) return;

    // Block maxima: DPP over lane bits 0-2, readlanes over bit 5.
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(v[i][e]));
    uint32_t u = __float_as_uint(m);
    u = max(u, dpp<kDppXor1>(u));
    u = max(u, dpp<kDppXor2>(u));
    u = max(u, dpp<kDppHalfMirror>(u));
    float sc_b[kGroup];
#pragma unroll
    for (int bb = 0; bb < kGroup; ++bb)
        sc_b[bb] = block_scale(__uint_as_float(max(__builtin_amdgcn_readlane(u, 8 * bb),
                                                   __builtin_amdgcn_readlane(u, 32 + 8 * bb))));
    const float sc = b == 0 ? sc_b[0] : b == 1 ? sc_b[1] : b == 2 ? sc_b[2] : sc_b[3];

    int8_t *dst = q + (gi * kBlock + r2) * ldq + c0;
    const bool store = gj0 + b < nbc;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        float xs[16];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) xs[4 * i + e] = v[4 * h + i][e];
        int code[16];
        if (sc != 0.0f) {
            quant_codes(xs, sc, code);
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) code[e] = 0;
        }
        if (store) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint32_t *>(dst + (int64_t)(2 * (4 * h + i)) * ldq) =
                    pack4(code[4 * i], code[4 * i + 1], code[4 * i + 2], code[4 * i + 3]);
        }
    }
    if (lane < kGroup && gj0 + lane < nbc) {
        const float sl = lane == 0 ? sc_b[0] : lane == 1 ? sc_b[1] : lane == 2 ? sc_b[2] : sc_b[3];
        s[gi * nbc + gj0 + lane] = sl;
    }
}

template <typename T>
hipError_t launch(const T *x, int64_t ldx, int64_t rows, int64_t cols, int8_t *q, int64_t ldq,
                  float *s, hipStream_t stream) {
    const int64_t nbr = rows / kBlock, nbc = cols / kBlock;
    if (nbr == 0 || nbc == 0) return hipSuccess;
    const int64_t ngc = (nbc + kGroup - 1) / kGroup, ngroups = nbr * ngc;
    const int64_t grid = (ngroups + 3) / 4;
    hipLaunchKernelGGL(k_quantize_block<T>, dim3((unsigned)grid), dim3(256), 0, stream, x, ldx, (int)nbc, (int)ngc,
                       ngroups, q, ldq, s);
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
