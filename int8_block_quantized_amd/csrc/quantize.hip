// quantize.hip -- per-block (32x32) INT8 quantization and requantization.
//
// Pages: Jetfire summary, one-line summary and "Approach": tensors travel as
// INT8 codes with one scale per 32x32 block, quantized on-chip.  This kernel
// is the HBM-bound entry into that data flow: fp32/bf16 in, codes + scales
// out, in one pass (4 B or 2 B read + 1 B written per element + 4 B per
// block).  jf_requant_block uses the fp32 instantiation: it is the same rule
// as the GEMM's requantizing epilogue.
//
// Mapping (a "band" workgroup).  A workgroup covers one 32-row band of
// blocks and a segment of 1 KiB per row (256 fp32 = 8 blocks, or 512 bf16 =
// 16 blocks).  Each of its W wavefronts holds L rows (W * L = 32; by default
// L = 8, four wavefronts), lane l holding the 16 bytes at offset 16 l of each
// of its rows: every load instruction reads one whole 1 KiB row segment and
// every store writes the segment's 256 or 512 code bytes.  On the MI355X this
// streams at 6.0 TB/s on a 16384 x 16384 fp32 input, against 5.4-5.5 TB/s
// for wavefronts that each hold four whole blocks (512-byte row pieces per
// load) and 5.2-5.4 TB/s for the same band with L = 2.  A block's maximum is
// reduced inside the wavefront by DPP (the lanes of a block are adjacent),
// then across the W wavefronts through LDS; codes come from quant_codes (no
// division per element).
#include <algorithm>

#include "jf_device.h"
#include "jf_launch.h"

namespace jf {
namespace {

#ifndef JF_QUANT_ROWS_PER_WAVE
#define JF_QUANT_ROWS_PER_WAVE 8
#endif
constexpr int kRowsPerWave = JF_QUANT_ROWS_PER_WAVE;   // L
constexpr int64_t kMaxGridX = 1 << 20, kMaxGridY = 1 << 15;   // workgroups per launch and grid dimension
constexpr int kWaves = kBlock / kRowsPerWave;     // W

template <typename T>
struct Seg;

template <>
struct Seg<float> {
    static constexpr int kElems = 4;              // elements per lane and row (16 bytes)
    static __device__ __forceinline__ void load(const float *p, float *v) {
        const f32x4 f = ld_stream(reinterpret_cast<const f32x4 *>(p));
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    }
    static __device__ __forceinline__ void store(int8_t *p, const int *c) {
        st_stream(reinterpret_cast<uint32_t *>(p), pack4(c[0], c[1], c[2], c[3]));
    }
};

template <>
struct Seg<uint16_t> {
    static constexpr int kElems = 8;
    // bfloat16 -> binary32 is exact: the 16 bits become the high half.
    static __device__ __forceinline__ void load(const uint16_t *p, float *v) {
        const u32x4 w = ld_stream(reinterpret_cast<const u32x4 *>(p));
        const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(d[k] << 16);
            v[2 * k + 1] = __uint_as_float(d[k] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(int8_t *p, const int *c) {
        st_stream(reinterpret_cast<u32x2 *>(p), u32x2{pack4(c[0], c[1], c[2], c[3]), pack4(c[4], c[5], c[6], c[7])});
    }
};

// Maximum over the lanes of one block (LPB adjacent lanes, LPB = 4 or 8):
// lane bits 0..log2(LPB)-1 by DPP; afterwards every lane of the block holds
// it.  Non-negative binary32 values order like their bit patterns.
template <int LPB>
__device__ __forceinline__ uint32_t block_lanes_max(uint32_t u) {
    u = max(u, dpp<kDppXor1>(u));
    u = max(u, dpp<kDppXor2>(u));
    if constexpr (LPB == 8) u = max(u, dpp<kDppHalfMirror>(u));
    return u;
}

template <typename T>
__global__ __launch_bounds__(64 * kWaves) void k_quantize_block(const T *__restrict__ x, int64_t ldx, int nbc,
                                                               int seg0, int band0, int8_t *__restrict__ q,
                                                               int64_t ldq, float *__restrict__ s) {
    using S = Seg<T>;
    constexpr int E = S::kElems, LPB = kBlock / E, NBS = kWave / LPB;   // blocks per segment
    __shared__ __attribute__((aligned(16))) float red[NBS][kWaves];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_id_uniform();
    const int seg = seg0 + blockIdx.x, band = band0 + blockIdx.y;
    const int b = lane / LPB;                        // block inside the segment
    const int bj = seg * NBS + b;                    // block column
    const bool valid = bj < nbc;
    const int64_t col = (int64_t)min(bj, nbc - 1) * kBlock + (lane % LPB) * E;
    const int64_t row0 = (int64_t)band * kBlock + wave * kRowsPerWave;

    float v[kRowsPerWave][E];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) S::load(x + (row0 + i) * ldx + col, v[i]);

    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
        for (int e = 0; e < E; ++e) m = fmaxf(m, fabsf(v[i][e]));
    const uint32_t mu = block_lanes_max<LPB>(__float_as_uint(m));
    if (lane % LPB == 0) red[b][wave] = __uint_as_float(mu);
    __syncthreads();
    uint32_t bm = 0;
#pragma unroll
    for (int w4 = 0; w4 < kWaves; w4 += 4) {
        if constexpr (kWaves >= 4) {
            const f32x4 r = *reinterpret_cast<const f32x4 *>(&red[b][w4]);
            bm = max(bm, max(max(__float_as_uint(r.x), __float_as_uint(r.y)), max(__float_as_uint(r.z), __float_as_uint(r.w))));
        } else {
#pragma unroll
            for (int k = 0; k < kWaves; ++k) bm = max(bm, __float_as_uint(red[b][k]));
        }
    }
    const float sc = block_scale(__uint_as_float(bm));

    float xs[kRowsPerWave * E];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
        for (int e = 0; e < E; ++e) xs[i * E + e] = v[i][e];
    int code[kRowsPerWave * E];
    if (sc != 0.0f) {
        quant_codes(xs, sc, code);
    } else {
#pragma unroll
        for (int e = 0; e < kRowsPerWave * E; ++e) code[e] = 0;
    }
    if (valid) {
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) S::store(q + (row0 + i) * ldq + col, &code[i * E]);
        if (wave == 0 && lane % LPB == 0) s[(int64_t)band * nbc + bj] = sc;
    }
}

template <typename T>
hipError_t launch(const T *x, int64_t ldx, int64_t rows, int64_t cols, int8_t *q, int64_t ldq,
                  float *s, hipStream_t stream) {
    constexpr int NBS = kWave / (kBlock / Seg<T>::kElems);
    const int64_t nbr = rows / kBlock, nbc = cols / kBlock;
    if (nbr == 0 || nbc == 0) return hipSuccess;
    const int64_t nseg = (nbc + NBS - 1) / NBS;
    // grid x: segments, y: bands; very large matrices take several launches
    for (int64_t b0 = 0; b0 < nbr; b0 += kMaxGridY)
        for (int64_t s0 = 0; s0 < nseg; s0 += kMaxGridX) {
            const dim3 grid((unsigned)std::min<int64_t>(kMaxGridX, nseg - s0),
                            (unsigned)std::min<int64_t>(kMaxGridY, nbr - b0));
            hipLaunchKernelGGL(k_quantize_block<T>, grid, dim3(64 * kWaves), 0, stream, x, ldx, (int)nbc, (int)s0,
                               (int)b0, q, ldq, s);
        }
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
