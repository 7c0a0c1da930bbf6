// qerror.hip -- quantization error by scale granularity.
//
// Pages: Jetfire summary, "Measured effects": per-block quantization against
// per-token and per-channel quantization, compared by quantization error on
// activations with channel-wise outliers.  The same scale/code rule as
// jf_quantize_block (s = fl(max|x|/127), q = clamp(rne(fl(x/s)), -127, 127))
// on four group shapes: 32x32 block, token (row), channel (column), tensor;
// returns the group scales and sum (x - fl(s*q))^2 in binary64.
//
// 32x32 blocks take one pass (a wavefront holds its blocks whole).  Rows,
// columns and the tensor take three launches after clearing: group maxima
// (non-negative binary32 maxima combined as bit patterns with atomic integer
// max), maxima -> scales, then codes and errors.  Error sums are per-lane
// binary64, reduced per workgroup, one atomic add each.  The
// element mapping is the quantize kernel's: a wavefront takes four
// horizontally adjacent blocks, lane l holding rows 2i + l/32 (i = 0..15)
// and elements 4(l%32)..4(l%32)+3 of the 128-element group row.
#include "jf_device.h"
#include "jf_launch.h"

namespace jf {
namespace {

constexpr int kGroup = 4;

enum { kBlockG = 0, kToken = 1, kChannel = 2, kTensor = 3 };

struct Tile {
    float v[16][4];
    int64_t gi, row0, col0;   // block row, first row, first column of the lane's 4 elements
    int gj0;                  // first block column of the group
    bool valid;               // the lane's block exists (tail groups)
};

__device__ __forceinline__ Tile load_tile(const float *x, int64_t ldx, int nbc, int ngc, int64_t grp) {
    Tile t;
    const int lane = threadIdx.x & (kWave - 1);
    t.gi = grp / ngc;
    t.gj0 = (int)(grp - t.gi * ngc) * kGroup;
    const int b = (lane & 31) >> 3;
    const int bj = min(t.gj0 + b, nbc - 1);
    t.valid = t.gj0 + b < nbc;
    t.row0 = t.gi * kBlock + (lane >> 5);
    t.col0 = (int64_t)bj * kBlock + 4 * (lane & 7);
    const float *src = x + t.row0 * ldx + t.col0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const f32x4 f = *reinterpret_cast<const f32x4 *>(src + 2 * i * ldx);
        t.v[i][0] = f.x; t.v[i][1] = f.y; t.v[i][2] = f.z; t.v[i][3] = f.w;
    }
    return t;
}

// Row, column or tensor maxima as uint32 bit patterns (x >= 0: IEEE order =
// unsigned order), combined with atomic max.
template <int G>
__global__ __launch_bounds__(256) void k_qe_max(const float *__restrict__ x, int64_t ldx, int nbc, int ngc,
                                                int64_t ngroups, uint32_t *__restrict__ mx) {
    __shared__ uint32_t wg_max[4];
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id_uniform();
    const int64_t grp_raw = (int64_t)blockIdx.x * 4 + wave;
    const Tile t = load_tile(x, ldx, nbc, ngc, min(grp_raw, ngroups - 1));
    const bool live = grp_raw < ngroups && t.valid;
    if constexpr (G == kTensor) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(t.v[i][e]));
        const uint32_t wm = __float_as_uint(wave_max_nonneg(live ? m : 0.0f));
        if (lane == 0) wg_max[wave] = wm;
        __syncthreads();
        if (threadIdx.x == 0) atomicMax(mx, max(max(wg_max[0], wg_max[1]), max(wg_max[2], wg_max[3])));
    } else if constexpr (G == kToken) {
        // row 2i + l/32: max over the 4 elements, then over the 32 lanes of the half-wave
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float m = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(t.v[i][e]));
            uint32_t u = live ? __float_as_uint(m) : 0u;
            u = max(u, dpp<kDppXor1>(u));
            u = max(u, dpp<kDppXor2>(u));
            u = max(u, dpp<kDppHalfMirror>(u));
            u = max(u, dpp<kDppMirror>(u));
            u = max(u, (uint32_t)__shfl_xor((int)u, 16));
            if (grp_raw < ngroups && (lane & 31) == 0) atomicMax(mx + t.row0 + 2 * i, u);
        }
    } else {
        // columns col0..col0+3: max over the 16 rows, then with lane l^32
        uint32_t u[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(t.v[i][e]));
            u[e] = live ? __float_as_uint(m) : 0u;
            u[e] = max(u[e], (uint32_t)__shfl_xor((int)u[e], 32));
        }
        if (grp_raw < ngroups && live && lane < 32)
#pragma unroll
            for (int e = 0; e < 4; ++e) atomicMax(mx + t.col0 + e, u[e]);
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

template <int G>
__global__ __launch_bounds__(256) void k_qe_err(const float *__restrict__ x, int64_t ldx, int nbc, int ngc,
                                                int64_t ngroups, const float *__restrict__ s,
                                                double *__restrict__ sse) {
    __shared__ double wg_sum[4];
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id_uniform();
    const int64_t grp_raw = (int64_t)blockIdx.x * 4 + wave;
    const Tile t = load_tile(x, ldx, nbc, ngc, min(grp_raw, ngroups - 1));
    const bool live = grp_raw < ngroups && t.valid;
    double acc = 0.0;
    if constexpr (G == kTensor) {
        const float sc = live ? s[0] : 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) v[k] = t.v[4 * c + k / 4][k % 4];
            add_sq_err<16>(v, sc, acc);
        }
    } else if constexpr (G == kToken) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float sc = live ? s[t.row0 + 2 * i] : 0.0f;
            add_sq_err<4>(t.v[i], sc, acc);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float sc = live ? s[t.col0 + e] : 0.0f;
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = t.v[i][e];
            add_sq_err<16>(v, sc, acc);
        }
    }
    if (!live) acc = 0.0;
    // wave sum, then one atomic add per workgroup
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) wg_sum[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) atomicAdd(sse, (wg_sum[0] + wg_sum[1]) + (wg_sum[2] + wg_sum[3]));
}

// 32x32 blocks in one pass: the wavefront holds its four blocks whole, so
// the block maxima, scales and errors come from registers.
__global__ __launch_bounds__(256) void k_qe_block(const float *__restrict__ x, int64_t ldx, int nbc, int ngc,
                                                  int64_t ngroups, float *__restrict__ s,
                                                  double *__restrict__ sse) {
    __shared__ double wg_sum[4];
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id_uniform();
    const int64_t grp_raw = (int64_t)blockIdx.x * 4 + wave;
    const Tile t = load_tile(x, ldx, nbc, ngc, min(grp_raw, ngroups - 1));
    const bool live = grp_raw < ngroups && t.valid;
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(t.v[i][e]));
    uint32_t u = __float_as_uint(m);
    u = max(u, dpp<kDppXor1>(u));
    u = max(u, dpp<kDppXor2>(u));
    u = max(u, dpp<kDppHalfMirror>(u));                  // the 8 lanes of one block row pair
    u = max(u, (uint32_t)__shfl_xor((int)u, 32));        // and the other half-wave's rows
    const float sc = block_scale(__uint_as_float(u));
    if (live && (lane & 39) == 0) s[t.gi * nbc + t.col0 / kBlock] = sc;   // lanes 0, 8, 16, 24
    double acc = 0.0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = t.v[4 * c + k / 4][k % 4];
        add_sq_err<16>(v, sc, acc);
    }
    if (!live) acc = 0.0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) wg_sum[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) atomicAdd(sse, (wg_sum[0] + wg_sum[1]) + (wg_sum[2] + wg_sum[3]));
}

template <int G>
hipError_t launch_g(const float *x, int64_t ldx, int64_t rows, int64_t cols, float *s, double *sse,
                    hipStream_t stream) {
    const int64_t nbr = rows / kBlock, nbc = cols / kBlock;
    const int64_t ngc = (nbc + kGroup - 1) / kGroup, ngroups = nbr * ngc;
    const int64_t ng = G == kBlockG ? 0 : G == kToken ? rows : G == kChannel ? cols : 1;   // maxima to clear
    uint32_t *mx = reinterpret_cast<uint32_t *>(s);
    // zero the atomically combined maxima and the sum (block scales are
    // written whole by the one-pass kernel)
    hipLaunchKernelGGL(k_qe_init, dim3((unsigned)((ng + 256) / 256)), dim3(256), 0, stream, mx, ng, sse);
    if (ngroups == 0) return hipGetLastError();
    const unsigned grid = (unsigned)((ngroups + 3) / 4);
    if constexpr (G == kBlockG) {
        hipLaunchKernelGGL(k_qe_block, dim3(grid), dim3(256), 0, stream, x, ldx, (int)nbc, (int)ngc, ngroups, s,
                           sse);
    } else {
        hipLaunchKernelGGL(k_qe_max<G>, dim3(grid), dim3(256), 0, stream, x, ldx, (int)nbc, (int)ngc, ngroups,
                           mx);
        hipLaunchKernelGGL(k_qe_scale, dim3((unsigned)((ng + 255) / 256)), dim3(256), 0, stream, mx, ng);
        hipLaunchKernelGGL(k_qe_err<G>, dim3(grid), dim3(256), 0, stream, x, ldx, (int)nbc, (int)ngc, ngroups,
                           (const float *)s, sse);
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
