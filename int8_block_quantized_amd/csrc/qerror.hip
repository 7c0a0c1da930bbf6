// qerror.hip -- quantization error by scale granularity.
//
// Pages: Jetfire summary, "Measured effects": per-block quantization against
// per-token and per-channel quantization, compared by quantization error on
// activations with channel-wise outliers.  The same scale/code rule as
// jf_quantize_block (s = fl(max|x|/127), q = clamp(rne(fl(x/s)), -127, 127))
// on four group shapes: 32x32 block, token (row), channel (column), tensor;
// returns the group scales and sum (x - fl(s*q))^2 in binary64.
//
// 32x32 blocks take one pass.  Rows, columns and the tensor take three
// launches after clearing: group maxima (non-negative binary32 maxima
// combined as bit patterns with atomic integer max; column maxima walk down
// the bands, the others along them), maxima -> scales, then codes and
// errors.  Error sums are per-lane binary64, reduced per
// workgroup, one atomic add each.
//
// Element mapping: the quantizer's band workgroup.  A workgroup covers one
// 32-row band of blocks and a 1 KiB segment (256 columns, 8 blocks) of each
// row; its four wavefronts hold eight rows each, lane l the four values at
// columns 4l..4l+3 of the segment (block l/8), so every load reads a whole
// 1 KiB row segment.
#include <algorithm>

#include "jf_device.h"
#include "jf_launch.h"

namespace jf {
namespace {

constexpr int kRows = 8;                    // rows per wavefront
constexpr int kWaves = kBlock / kRows;      // 4 wavefronts
constexpr int kSegBlocks = 8;               // blocks per 1 KiB segment of fp32
constexpr int kMaxSegPerWG = 8;   // segments per workgroup, in turn (at most)
#ifndef JF_QE_BPW
#define JF_QE_BPW 4
#endif
constexpr int kMaxBandsPerWG = JF_QE_BPW;   // bands per column-maxima workgroup (at most)
constexpr int64_t kMaxGridX = 1 << 20, kMaxGridY = 1 << 15;

enum { kBlockG = 0, kToken = 1, kChannel = 2, kTensor = 3 };

struct Tile {
    float v[kRows][4];
    int64_t row0, col0;   // first row and first column of the lane's values
    int bj;               // block column of the lane (clamped)
    bool valid;           // the lane's block exists (ragged last segment)
};

__device__ __forceinline__ Tile load_tile(const float *x, int64_t ldx, int nbc, int seg, int band) {
    Tile t;
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id_uniform();
    const int bj = seg * kSegBlocks + lane / 8;
    t.valid = bj < nbc;
    t.bj = min(bj, nbc - 1);
    t.row0 = (int64_t)band * kBlock + wave * kRows;
    t.col0 = (int64_t)t.bj * kBlock + 4 * (lane & 7);
    const float *src = x + t.row0 * ldx + t.col0;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const f32x4 f = *reinterpret_cast<const f32x4 *>(src + i * ldx);
        t.v[i][0] = f.x; t.v[i][1] = f.y; t.v[i][2] = f.z; t.v[i][3] = f.w;
    }
    return t;
}

// Sum of a binary64 value over the workgroup, then one atomic add.
__device__ __forceinline__ void wg_sum_add(double acc, double *sse) {
    __shared__ double wg_sum[kWaves];
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id_uniform();
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) wg_sum[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) atomicAdd(sse, (wg_sum[0] + wg_sum[1]) + (wg_sum[2] + wg_sum[3]));
}

// Row, column or tensor maxima as uint32 bit patterns (x >= 0: IEEE order =
// unsigned order), combined with atomic max.  A workgroup takes spw (up to
// eight) segments of its band in turn, the next one's loads issued before
// the current one is reduced: every workgroup ends in atomics, and those on
// one address (the tensor maximum, the error sum) serialize in L2 at roughly
// one per 13 ns (the one-segment workgroups of a 16384 x 16384 input spent
// most of their time there), so fewer, longer workgroups keep them off the
// critical path; the launcher keeps at least 1024 workgroups.
template <int G>
__global__ __launch_bounds__(64 * kWaves) void k_qe_max(const float *__restrict__ x, int64_t ldx, int nbc, int nseg,
                                                        int spw, int sg0, int band0, uint32_t *__restrict__ mx) {
    __shared__ uint32_t wmax[kWaves];
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id_uniform();
    const int band = band0 + blockIdx.y, seg_first = (sg0 + blockIdx.x) * spw;
    float tmax = 0.0f;                                   // tensor: running maximum
    const int seg_last = min(seg_first + spw, nseg) - 1;
    Tile t = load_tile(x, ldx, nbc, min(seg_first, nseg - 1), band);
#pragma unroll 1
    for (int j = 0; j < spw && seg_first + j < nseg; ++j) {
        // the next segment's loads go out first; after the workgroup's last
        // segment they re-read it (lines still in L2: no HBM traffic)
        const Tile nt = load_tile(x, ldx, nbc, min(seg_first + j + 1, seg_last), band);
        if constexpr (G == kTensor) {
#pragma unroll
            for (int i = 0; i < kRows; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, t.valid ? fabsf(t.v[i][e]) : 0.0f);
        } else {
            static_assert(G == kToken, "column maxima: k_qe_colmax");
            // row i of the wavefront: max over the lane's 4 values, then the wavefront
#pragma unroll
            for (int i = 0; i < kRows; ++i) {
                float m = 0.0f;
#pragma unroll
                for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(t.v[i][e]));
                const uint32_t u = __float_as_uint(wave_max_nonneg(t.valid ? m : 0.0f));
                if (lane == 0) atomicMax(mx + t.row0 + i, u);
            }
        }
        t = nt;
    }
    if constexpr (G == kTensor) {
        const uint32_t wm = __float_as_uint(wave_max_nonneg(tmax));
        if (lane == 0) wmax[wave] = wm;
        __syncthreads();
        if (threadIdx.x == 0) atomicMax(mx, max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
    }
}

// Column maxima.  A workgroup takes one 1 KiB segment (256 columns) and bpw
// consecutive bands, walking down them with the next band's loads issued
// before the current one is reduced; each lane keeps the running maxima of
// its four columns over its rows, the four wavefronts combine them through
// LDS once, and the workgroup ends in one atomic per column (lane l of the
// first wavefront takes columns l, l + 64, l + 128, l + 192, so each atomic
// instruction covers 256 contiguous bytes).  Walking along the band instead
// (as the row and tensor maxima do) would cost a barrier and 256 atomics per
// segment.
__global__ __launch_bounds__(64 * kWaves) void k_qe_colmax(const float *__restrict__ x, int64_t ldx, int nbc,
                                                           int nbr, int bpw, int sg0, int bg0,
                                                           uint32_t *__restrict__ mx) {
    __shared__ uint32_t cmax[kWaves][kWave * 4];
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id_uniform();
    const int seg = sg0 + blockIdx.x, band_first = (bg0 + blockIdx.y) * bpw;
    const int band_last = min(band_first + bpw, nbr) - 1;
    float m[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    Tile t = load_tile(x, ldx, nbc, seg, band_first);
#pragma unroll 1
    for (int j = band_first; j <= band_last; ++j) {
        // the next band's loads go out first; after the last band they re-read it
        const Tile nt = load_tile(x, ldx, nbc, seg, min(j + 1, band_last));
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < kRows; ++i) m[e] = fmaxf(m[e], fabsf(t.v[i][e]));
        t = nt;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) cmax[wave][4 * lane + e] = __float_as_uint(m[e]);   // column 4 lane + e
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = lane + kWave * e;                     // column of the segment
            if (seg * kSegBlocks + c / kBlock < nbc)
                atomicMax(mx + (int64_t)seg * kSegBlocks * kBlock + c,
                          max(max(cmax[0][c], cmax[1][c]), max(cmax[2][c], cmax[3][c])));
        }
    }
}

__global__ __launch_bounds__(256) void k_qe_init(uint32_t *__restrict__ mx, int64_t n, double *__restrict__ sse) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) mx[i] = 0u;
    if (i == 0) *sse = 0.0;
}

// maxima (bit patterns) -> scales, in place
__global__ __launch_bounds__(256) void k_qe_scale(uint32_t *__restrict__ mx, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) mx[i] = __float_as_uint(block_scale(__uint_as_float(mx[i])));
}

// Codes and errors.  The code is rne of the reciprocal product t = fl(x*r),
// r = fl(1/s), redone with the IEEE quotient when t lies within 2^-15 of a
// half-integer (the quant_codes argument) or when 1/s overflows; a zero
// scale gives code 0.  The difference d = x - fl(s*q) is exact in binary32:
// for q = 0 it is x, otherwise x and fl(s*q) have the same sign and are
// within a factor of two of each other (|x - s q| <= s/2 + ulp, |s q| >= s),
// so Sterbenz's lemma applies.  d*d is then exact in binary64 (48 bits), and
// each lane adds its terms to a binary64 sum.
template <int N>
__device__ __forceinline__ void add_sq_err(const float (&x)[N], float s, double &acc) {
    const float r = 1.0f / s;
    float n[N];
    bool near = !(r < __builtin_inff());
#pragma unroll
    for (int e = 0; e < N; ++e) {
        const float t = x[e] * r;
        n[e] = __builtin_rintf(t);
        near |= fabsf(fabsf(t - n[e]) - 0.5f) < 0x1p-15f;
    }
    if (__builtin_amdgcn_ballot_w64(near) != 0) {
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const float t = x[e] * r;
            if (!(r < __builtin_inff()) || fabsf(fabsf(t - n[e]) - 0.5f) < 0x1p-15f)
                n[e] = s == 0.0f ? 0.0f : __builtin_rintf(x[e] / s);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int e = 0; e < N; ++e) {
        const float d = x[e] - s * __builtin_amdgcn_fmed3f(n[e], -127.0f, 127.0f);
        acc = fma((double)d, (double)d, acc);
    }
}

// Errors of one tile's 32 values of a lane under the given scales.
template <int G>
__device__ __forceinline__ double tile_err(const Tile &t, const float *__restrict__ s) {
    double acc = 0.0;
    if constexpr (G == kTensor) {
        const float sc = s[0];
#pragma unroll
        for (int c = 0; c < kRows / 4; ++c) {
            float v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) v[k] = t.v[4 * c + k / 4][k % 4];
            add_sq_err<16>(v, sc, acc);
        }
    } else if constexpr (G == kToken) {
#pragma unroll
        for (int i = 0; i < kRows; ++i) add_sq_err<4>(t.v[i], s[t.row0 + i], acc);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v[kRows];
#pragma unroll
            for (int i = 0; i < kRows; ++i) v[i] = t.v[i][e];
            add_sq_err<kRows>(v, s[t.col0 + e], acc);
        }
    }
    return t.valid ? acc : 0.0;
}

template <int G>
__global__ __launch_bounds__(64 * kWaves) void k_qe_err(const float *__restrict__ x, int64_t ldx, int nbc, int nseg,
                                                        int spw, int sg0, int band0, const float *__restrict__ s,
                                                        double *__restrict__ sse) {
    const int band = band0 + blockIdx.y, seg_first = (sg0 + blockIdx.x) * spw;
    double acc = 0.0;
    const int seg_last = min(seg_first + spw, nseg) - 1;
    Tile t = load_tile(x, ldx, nbc, min(seg_first, nseg - 1), band);
#pragma unroll 1
    for (int j = 0; j < spw && seg_first + j < nseg; ++j) {
        // the next segment's loads go out first; after the workgroup's last
        // segment they re-read it (lines still in L2: no HBM traffic)
        const Tile nt = load_tile(x, ldx, nbc, min(seg_first + j + 1, seg_last), band);
        acc += tile_err<G>(t, s);
        t = nt;
    }
    wg_sum_add(acc, sse);
}

// 32x32 blocks in one pass: block maxima inside the wavefront by DPP (a
// block's 8 lanes are adjacent), then across the four wavefronts through LDS
// (two buffers: one barrier per segment); scales and errors from registers.
__global__ __launch_bounds__(64 * kWaves) void k_qe_block(const float *__restrict__ x, int64_t ldx, int nbc,
                                                          int nseg, int spw, int sg0, int band0, float *__restrict__ s,
                                                          double *__restrict__ sse) {
    __shared__ __attribute__((aligned(16))) float red[2][kSegBlocks][kWaves];
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id_uniform();
    const int band = band0 + blockIdx.y, seg_first = (sg0 + blockIdx.x) * spw;
    const int b = lane / 8;
    double acc = 0.0;
    const int seg_last = min(seg_first + spw, nseg) - 1;
    Tile t = load_tile(x, ldx, nbc, min(seg_first, nseg - 1), band);
#pragma unroll 1
    for (int j = 0; j < spw && seg_first + j < nseg; ++j) {
        // the next segment's loads go out first; after the workgroup's last
        // segment they re-read it (lines still in L2: no HBM traffic)
        const Tile nt = load_tile(x, ldx, nbc, min(seg_first + j + 1, seg_last), band);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < kRows; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(t.v[i][e]));
        uint32_t u = __float_as_uint(m);
        u = max(u, dpp<kDppXor1>(u));
        u = max(u, dpp<kDppXor2>(u));
        u = max(u, dpp<kDppHalfMirror>(u));              // the 8 lanes of one block
        if ((lane & 7) == 0) red[j & 1][b][wave] = __uint_as_float(u);
        __syncthreads();
        const f32x4 r = *reinterpret_cast<const f32x4 *>(red[j & 1][b]);
        const float sc = block_scale(fmaxf(fmaxf(r.x, r.y), fmaxf(r.z, r.w)));
        if (t.valid && wave == 0 && (lane & 7) == 0) s[(int64_t)band * nbc + t.bj] = sc;
        double a = 0.0;
#pragma unroll
        for (int c = 0; c < kRows / 4; ++c) {
            float v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) v[k] = t.v[4 * c + k / 4][k % 4];
            add_sq_err<16>(v, sc, a);
        }
        acc += t.valid ? a : 0.0;
        t = nt;
    }
    wg_sum_add(acc, sse);
}

template <typename L>
void for_grid(int64_t nbr, int64_t nsg, L &&launch) {
    for (int64_t b0 = 0; b0 < nbr; b0 += kMaxGridY)
        for (int64_t s0 = 0; s0 < nsg; s0 += kMaxGridX)
            launch(b0, s0, dim3((unsigned)std::min<int64_t>(kMaxGridX, nsg - s0),
                                (unsigned)std::min<int64_t>(kMaxGridY, nbr - b0)));
}

template <int G>
hipError_t launch_g(const float *x, int64_t ldx, int64_t rows, int64_t cols, float *s, double *sse,
                    hipStream_t stream) {
    const int64_t nbr = rows / kBlock, nbc = cols / kBlock;
    const int64_t nseg = (nbc + kSegBlocks - 1) / kSegBlocks;
    // segments per workgroup: as many as keep at least 1024 workgroups
    int spw = kMaxSegPerWG;
    while (spw > 1 && nbr * ((nseg + spw - 1) / spw) < 1024) spw /= 2;
    const int64_t nsg = (nseg + spw - 1) / spw;
    const int64_t ng = G == kBlockG ? 0 : G == kToken ? rows : G == kChannel ? cols : 1;   // maxima to clear
    uint32_t *mx = reinterpret_cast<uint32_t *>(s);
    // zero the atomically combined maxima and the sum (block scales are
    // written whole by the one-pass kernel)
    hipLaunchKernelGGL(k_qe_init, dim3((unsigned)((ng + 256) / 256)), dim3(256), 0, stream, mx, ng, sse);
    if (nbr == 0 || nbc == 0) return hipGetLastError();
    if constexpr (G == kChannel) {
        // bands per workgroup: as many (up to kMaxBandsPerWG) as keep at least 1024 workgroups
        int bpw = kMaxBandsPerWG;
        while (bpw > 1 && nseg * ((nbr + bpw - 1) / bpw) < 1024) bpw /= 2;
        const int64_t nbg = (nbr + bpw - 1) / bpw;
        for_grid(nbg, nseg, [&](int64_t b0, int64_t s0, dim3 grid) {
            hipLaunchKernelGGL(k_qe_colmax, grid, dim3(64 * kWaves), 0, stream, x, ldx, (int)nbc, (int)nbr, bpw,
                               (int)s0, (int)b0, mx);
        });
    } else {
        for_grid(nbr, nsg, [&](int64_t b0, int64_t s0, dim3 grid) {
            if constexpr (G == kBlockG)
                hipLaunchKernelGGL(k_qe_block, grid, dim3(64 * kWaves), 0, stream, x, ldx, (int)nbc, (int)nseg, spw,
                                   (int)s0, (int)b0, s, sse);
            else
                hipLaunchKernelGGL(k_qe_max<G>, grid, dim3(64 * kWaves), 0, stream, x, ldx, (int)nbc, (int)nseg,
                                   spw, (int)s0, (int)b0, mx);
        });
    }
    if constexpr (G != kBlockG) {
        hipLaunchKernelGGL(k_qe_scale, dim3((unsigned)((ng + 255) / 256)), dim3(256), 0, stream, mx, ng);
        for_grid(nbr, nsg, [&](int64_t b0, int64_t s0, dim3 grid) {
            hipLaunchKernelGGL(k_qe_err<G>, grid, dim3(64 * kWaves), 0, stream, x, ldx, (int)nbc, (int)nseg, spw,
                               (int)s0, (int)b0, (const float *)s, sse);
        });
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_error(const float *x, int64_t ldx, int64_t rows, int64_t cols, int granularity, float *s,
                              double *sse, hipStream_t stream) {
    switch (granularity) {
    case kBlockG: return launch_g<kBlockG>(x, ldx, rows, cols, s, sse, stream);
    case kToken: return launch_g<kToken>(x, ldx, rows, cols, s, sse, stream);
    case kChannel: return launch_g<kChannel>(x, ldx, rows, cols, s, sse, stream);
    default: return launch_g<kTensor>(x, ldx, rows, cols, s, sse, stream);
    }
}

}  // namespace jf
