// gelu.hip -- INT8-in / INT8-out GELU with per-block requantization.
//
// Pages: Jetfire summary, "Problem" (non-linear operators are memory-bound)
// and "Approach" (they too read and write INT8 with per-block scales).  The
// erf form of GELU is used: g(x) = x * Phi(x), Phi(x) = erfc(-x/sqrt 2) / 2.
//
// Memory mapping.  A wavefront pass covers a group of four horizontally
// adjacent 32x32 blocks: each 16-byte load or store of the wavefront spans
// eight whole 128-byte rows of the group, so every HBM line is read and
// written by one instruction.  Lane l holds rows 8i + l/8 (i = 0..3), bytes
// 16(l%8)..16(l%8)+15 of the group row: all of them inside block (l%8)/2.
// Each wavefront makes two passes, with the loads of both issued first.
//
// Per block, every element is x = fl(s*q) for one of at most 256 codes, so g
// is evaluated once per code value, not once per element:
//   1. the block's largest code c_max: packed 16-bit maxima over the lane's
//      bytes, then a max over the block's 16 lanes (two DPP steps within
//      each row of 16 lanes, two row-swapping permutes across the rows), so
//      every lane holds its own block's;
//   2. for x >= 0, g is increasing, and for x < 0, |g| < 0.16998; so when
//      c_max > 0 and g(c_max) >= 0.17 the block max |g| is g(c_max),
//      evaluated in binary64 (one call for the eight blocks of both passes,
//      with their output scales).  Otherwise (blocks with almost no positive
//      mass) every element's |g| is looked up in a table evaluated in
//      binary64;
//   3. s' = fl(max/127); lane l evaluates g for the codes +-(2l+1) and
//      +-(2l+2) in binary32 (gelu_fast's polynomial tail approximation: one
//      tail value per pair, as g(x) = x - xQ(x) and g(-x) = -xQ(x)) and turns
//      them into output codes (table_codes: exact against the binary64
//      reference, see there), bytes of the block's 256-entry code table in
//      LDS, indexed by the code's raw byte;
//   4. each element's output code is one byte read from its block's table (a
//      256-byte table spans the 64 LDS banks once, so reads of one table
//      never conflict; the four tables of a group share the banks, so one
//      instruction's reads can).
// Measured with timing-only copies: the per-block table work costs about 5%
// of the kernel's time and the lookups' bank conflicts 1-2%; the rest is the
// group structure itself (loads, code maxima, one lookup per element,
// packing, stores), about 1.12x the time of a streaming copy of its bytes.
// HBM traffic is the algorithmic 2 bytes per element plus 8 bytes per block.
#include "jf_device.h"
#include "jf_gelu.h"
#include "jf_launch.h"

namespace jf {
namespace {

// The binary64 reference value (gelu_tail: the normal-tail expansion, 67
// VALU instructions against 144 for the library erfc) as a call: one copy of
// the code instead of one per use, and its registers stay out of the
// kernel's loop.
__device__ __attribute__((noinline)) float gelu_ref_outlined(float x) { return gelu_tail(x); }

// Output codes of a lane's table entries.  g holds gelu_fast values, s2 =
// fl(m/127) with m = gelu_tail of the block's largest code, m >= 0.17, so the
// table inputs satisfy |x| >= 0.0022 or x = 0, where gelu_fast is within
// 6.51e-7 |gref| of gref = gelu_tail(x) for x >= 0 and within 2.14e-7 of it
// for x < 0.  Let r = rcp(s2) (hardware reciprocal, within one ulp, i.e.
// 2^-23 relative), t = fl(g r) and Q = fl(gref / s2), the quotient whose
// rne is the reference code.  Collecting the reciprocal's error and the two
// products' roundings (2^-24 each) with the error of g:
//   x >= 0: |t - Q| <= (6.51e-7 + 2.4e-7) |t|  <  1e-6 |t|,
//   x <  0: |t - Q| <= 2.15e-7 r + 2.4e-7 |t|  <  2.2e-7 r + 1e-6 |t|.
// So with w = 1e-6 |t| + 2.2e-7 r, rne(t) = rne(Q) whenever t is more than
// w away from the nearest half-integer (t - rne(t) is exact); the test uses
// w + 2^-20, which covers its own roundings.  The other entries (about
// 1.5e-4 of the positive ones at the bench input's scales, far fewer of the
// negative ones) are recomputed from gelu_tail with an IEEE division, one
// wavefront-wide binary64 call per round.
template <int N>
__device__ __forceinline__ void table_codes(const float (&g)[N], const float (&x)[N], float s2, int (&code)[N]) {
    const float r = __builtin_amdgcn_rcpf(s2);
    const float half_c = 0.5f - __builtin_fmaf(2.2e-7f, r, 0x1p-20f);
    float n[N];
    uint32_t near = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const float t = g[j] * r;
        n[j] = __builtin_rintf(t);
        if (fabsf(t - n[j]) > __builtin_fmaf(-1e-6f, fabsf(t), half_c)) near |= 1u << j;
    }
    while (__builtin_amdgcn_ballot_w64(near != 0) != 0) {
        if (near != 0) {
            const int k = __builtin_ctz(near);
            near &= near - 1;
            float xk = x[0];
#pragma unroll
            for (int j = 1; j < N; ++j) xk = k == j ? x[j] : xk;
            const float nk = __builtin_rintf(gelu_ref_outlined(xk) / s2);
#pragma unroll
            for (int j = 0; j < N; ++j) n[j] = k == j ? nk : n[j];
        }
    }
#pragma unroll
    for (int j = 0; j < N; ++j) code[j] = (int)__builtin_amdgcn_fmed3f(n[j], -127.0f, 127.0f);   // n is finite
}

constexpr int kGroup = 4;    // horizontally adjacent blocks per wavefront pass
constexpr int kPasses = 2;   // passes per wavefront

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const uint8_t lds_u8;

// Largest signed code among a lane's 64 bytes of one pass.  Read as two
// signed 16-bit halves, a dword orders each half by its high byte (bytes 1
// and 3); shifted left by 8 within each half, by its low byte (bytes 0 and
// 2).  Three packed instructions per dword, one reduction at the end.
__device__ __forceinline__ int max_code(const u32x4 (&w)[4]) {
    s16x2 hi = __builtin_bit_cast(s16x2, w[0].x), lo = hi << 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t wd[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
        for (int d = (i == 0 ? 1 : 0); d < 4; ++d) {
            const s16x2 v = __builtin_bit_cast(s16x2, wd[d]);
            hi = __builtin_elementwise_max(hi, v);
            lo = __builtin_elementwise_max(lo, (s16x2)(v << 8));
        }
    }
    const s16x2 m = __builtin_elementwise_max(hi, lo) >> 8;
    return max((int)m.x, (int)m.y);
}

// Maximum over the 16 lanes holding one block (lanes 8r + 2b + e): DPP over
// lane bits 0 and 3 within each row of 16 lanes, ...
__device__ __forceinline__ uint32_t group_reduce_rows(uint32_t v) {
    v = max(v, dpp<kDppXor1>(v));
    return max(v, dpp<kDppRowRor8>(v));
}
// ... then across the four rows (lane bits 5 and 4) with the row-swapping
// permutes: afterwards every lane holds the maximum of its own block.
__device__ __forceinline__ uint32_t wave_rows_max(uint32_t v) {
    const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);   // lanes l and l ^ 32
    v = max(h[0], h[1]);
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);   // lanes l and l ^ 16
    return max(r[0], r[1]);
}
// Block b's maximum for the slow path (wave-uniform), from the row maxima.
__device__ __forceinline__ uint32_t block_max_u(uint32_t v_rows, int b) {
    const uint32_t a = __builtin_amdgcn_readlane(v_rows, 2 * b), c = __builtin_amdgcn_readlane(v_rows, 16 + 2 * b);
    const uint32_t d = __builtin_amdgcn_readlane(v_rows, 32 + 2 * b), e = __builtin_amdgcn_readlane(v_rows, 48 + 2 * b);
    return max(max(a, c), max(d, e));
}

__global__ __launch_bounds__(256) void k_gelu_i8(const int8_t *__restrict__ q, int64_t ldq,
                                                 const float *__restrict__ s, int nbc, int ngc, int64_t ngroups,
                                                 int8_t *__restrict__ qo, int64_t ldqo,
                                                 float *__restrict__ so) {
    // Per wavefront: the four blocks' output-code tables (256 bytes each)
    // and one binary64-derived |g| table for the rare slow path.
    __shared__ __attribute__((aligned(256))) uint32_t tables[4][kGroup][kWave];
    __shared__ float gtab[4][256];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = wave_id_uniform();
    const int r8 = lane >> 3, b = (lane & 7) >> 1, colb = (lane & 1) * 16;
    const int64_t first = ((int64_t)blockIdx.x * 4 + wave) * kPasses;

    u32x4 w[kPasses][4];
    float scl[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int64_t grp = min(first + p, ngroups - 1);    // tail: re-read, never stored
        const int64_t gi = grp / ngc;
        const int bj = min((int)(grp - gi * ngc) * kGroup + b, nbc - 1);
        const int8_t *src = q + (gi * kBlock + r8) * ldq + (int64_t)bj * kBlock + colb;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[p][i] = ld_stream(reinterpret_cast<const u32x4 *>(src + 8 * i * ldq));
        scl[p] = s[gi * nbc + bj];
    }

    // Largest code of every block of both passes (each lane: its own
    // block's), and g of it in binary64 for all eight blocks in one call:
    // lanes 16p + 2bb hold block bb of pass p.
    static_assert(kPasses == 2, "one binary64 call serves two passes");
    int cm_all[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
        cm_all[p] = (int)wave_rows_max(group_reduce_rows((uint32_t)(max_code(w[p]) + 128))) - 128;
    const bool second = (lane & 16) != 0;
    const float xt = (second ? scl[1] : scl[0]) * (float)(second ? cm_all[1] : cm_all[0]);
    const float gt_lane = gelu_ref_outlined(xt);
    const float s2_lane = block_scale(gt_lane);   // the output scales of the fast path
    const float kf[2] = {(float)(2 * lane + 1), (float)(2 * lane + 2)};   // the lane's table magnitudes

#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int64_t grp = first + p;
        if (grp >= ngroups) break;
        const int64_t gi = grp / ngc;
        const int gj0 = (int)(grp - gi * ngc) * kGroup;
        const int nb = min(kGroup, nbc - gj0);             // blocks of this group

#pragma unroll
        for (int bb = 0; bb < kGroup; ++bb) {
            if (bb >= nb) break;
            const int cmax = __builtin_amdgcn_readlane(cm_all[p], 2 * bb);
            const float sc = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(scl[p]), 2 * bb));
            const float gtop = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(gt_lane), 16 * p + 2 * bb));
            float x[4], g[4];
            int code[4] = {0, 0, 0, 0};
            float s2;
            if (cmax > 0 && gtop >= 0.17f) {
                // Lane l takes the code pairs +-p, p = 2l+1 and 2l+2: one tail
                // value Q serves g(x) = x - xQ and g(-x) = -xQ (the same
                // arithmetic as gelu_fast on each); code 0 gives 0.  The
                // pair p = 128 only has its negative code.
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float xp = sc * kf[h];
                    const float q = gelu_tail_q(xp);
                    x[2 * h] = xp;
                    g[2 * h] = xp - xp * q;
                    x[2 * h + 1] = -xp;
                    g[2 * h + 1] = -xp * q;
                }
                s2 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(s2_lane), 16 * p + 2 * bb));
                table_codes(g, x, s2, code);
                uint8_t *tb = reinterpret_cast<uint8_t *>(tables[wave][bb]);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int pc = 2 * lane + h + 1;
                    if (pc < 128) tb[pc] = (uint8_t)code[2 * h];
                    tb[256 - pc] = (uint8_t)code[2 * h + 1];
                }
                if (lane == 0) tb[0] = 0;
            } else {
                // entries u = 4*lane + j, code (int8_t)u
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = sc * (float)(int8_t)(4 * lane + j);
                // Rare: the block's largest |g| may sit on a negative code.
                // The whole table is evaluated with the reference formula
                // and the block's elements look up their |g| in it.
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    g[j] = gelu_ref_outlined(x[j]);
                    gtab[wave][4 * lane + j] = fabsf(g[j]);
                }
                float m = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t wd[4] = {w[p][i].x, w[p][i].y, w[p][i].z, w[p][i].w};
#pragma unroll
                    for (int d = 0; d < 4; ++d)
#pragma unroll
                        for (int k = 0; k < 4; ++k) m = fmaxf(m, gtab[wave][(wd[d] >> (8 * k)) & 0xffu]);
                }
                // only the lanes of block bb count
                s2 = block_scale(__uint_as_float(block_max_u(group_reduce_rows(__float_as_uint(m)), bb)));
                if (s2 != 0.0f) quant_codes(g, s2, code);
                tables[wave][bb][lane] = pack4(code[0], code[1], code[2], code[3]);
            }
            if (lane == 0) so[gi * nbc + gj0 + bb] = s2;
        }

        // Each element's output code: one byte of its block's table.
        if (gj0 + b < nbc) {
            // LDS byte address of entry u: the table is 256-byte aligned, so
            // one byte permute puts u under the table's base address.
            const uint32_t tbase = (uint32_t)(uintptr_t)(lds_void *)tables[wave][b];
            int8_t *dst = qo + (gi * kBlock + r8) * ldqo + (int64_t)(gj0 + b) * kBlock + colb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t wd[4] = {w[p][i].x, w[p][i].y, w[p][i].z, w[p][i].w};
                uint32_t od[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uint32_t r[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        r[k] = *reinterpret_cast<const lds_u8 *>(
                            (uintptr_t)__builtin_amdgcn_perm(tbase, wd[d], 0x07060500u | (uint32_t)k));
                    od[d] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(r[3], r[2], 0x0c0c0400u),
                                                  __builtin_amdgcn_perm(r[1], r[0], 0x0c0c0400u), 0x05040100u);
                }
                st_stream(reinterpret_cast<u32x4 *>(dst + 8 * i * ldqo), u32x4{od[0], od[1], od[2], od[3]});
            }
        }
    }
}

}  // namespace

hipError_t launch_gelu(const int8_t *q, int64_t ldq, const float *s, int64_t rows, int64_t cols,
                       int8_t *qo, int64_t ldqo, float *so, hipStream_t stream) {
    const int64_t nbr = rows / kBlock, nbc = cols / kBlock;
    if (nbr == 0 || nbc == 0) return hipSuccess;
    const int64_t ngc = (nbc + kGroup - 1) / kGroup, ngroups = nbr * ngc;
    const int64_t per_wg = 4 * kPasses;
    const int64_t grid = (ngroups + per_wg - 1) / per_wg;
    hipLaunchKernelGGL(k_gelu_i8, dim3((unsigned)grid), dim3(256), 0, stream, q, ldq, s, (int)nbc, (int)ngc,
                       ngroups, qo, ldqo, so);
    return hipGetLastError();
}

}  // namespace jf
