// jf_device.h -- device helpers shared by the quantize, requantize, GEMM and
// GELU kernels of libjetfire (gfx950, wave64).
//
// The per-block rule implemented here is the library's reading of the
// per-block (32x32) quantization in "Jetfire: Efficient and Accurate
// Transformer Pretraining with INT8 Data Flow and Per-Block Quantization"
// (one-line summary and "Approach"): s = fl(max|x|/127) with one IEEE
// binary32 division, q = clamp(rne(fl(x/s)), -127, 127), q = 0 when s = 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jf {

constexpr int kBlock = 32;      // quantization block edge
constexpr int kWave = 64;       // CDNA wavefront size

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming HBM access of the memory-bound kernels: every input and output
// element is touched once, so loads and stores carry the nontemporal hint.
#ifndef JF_NT
#define JF_NT 1
#endif
template <typename T>
__device__ __forceinline__ T ld_stream(const T *p) {
    if constexpr (JF_NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <typename T>
__device__ __forceinline__ void st_stream(T *p, T v) {
    if constexpr (JF_NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Lane exchange inside rows of 16 lanes (DPP); all lanes valid.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within each 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within each 16
constexpr int kDppRowRor8 = 0x128;     // lane i <-> i^8 within each 16 (rotate by 8)

// Wave-uniform maximum of non-negative binary32 values: for them the IEEE
// order is the unsigned order of the bit patterns.  Rows of 16 reduce with
// DPP, the four row results with readlane.
__device__ __forceinline__ float wave_max_nonneg(float v) {
    uint32_t u = __float_as_uint(v);
    u = max(u, dpp<kDppXor1>(u));
    u = max(u, dpp<kDppXor2>(u));
    u = max(u, dpp<kDppHalfMirror>(u));
    u = max(u, dpp<kDppMirror>(u));
    const uint32_t a = __builtin_amdgcn_readlane(u, 0), b = __builtin_amdgcn_readlane(u, 16);
    const uint32_t c = __builtin_amdgcn_readlane(u, 32), d = __builtin_amdgcn_readlane(u, 48);
    return __uint_as_float(max(max(a, b), max(c, d)));
}

// Wave-uniform maximum of signed integers.
__device__ __forceinline__ int wave_max_int(int v) {
    v = max(v, (int)dpp<kDppXor1>((uint32_t)v));
    v = max(v, (int)dpp<kDppXor2>((uint32_t)v));
    v = max(v, (int)dpp<kDppHalfMirror>((uint32_t)v));
    v = max(v, (int)dpp<kDppMirror>((uint32_t)v));
    const int a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const int c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return max(max(a, b), max(c, d));
}

// Block scale from the block's max magnitude: one correctly rounded division
// (HIP keeps binary32 '/' IEEE-exact unless fast-math is requested).
__device__ __forceinline__ float block_scale(float absmax) { return absmax / 127.0f; }

// Code of one value under a non-zero scale: correctly rounded quotient,
// round-half-even, clamp to the symmetric INT8 range.
__device__ __forceinline__ int quant_code(float x, float s) {
    return (int)__builtin_amdgcn_fmed3f(__builtin_rintf(x / s), -127.0f, 127.0f);   // the quotient is finite
}

// Codes of N values under one non-zero scale s, without a division per value.
// With r = fl(1/s) and t = fl(x*r):  t = (x/s)(1+d1)(1+d2), |di| <= 2^-24, so
// t is within 2.5 ulp(t) <= 2.5 * 2^-17 of fl(x/s) whenever |x/s| < 128 (the
// codes' range).  rne(t) therefore equals rne(fl(x/s)) unless t lies within
// 2^-15 of a half-integer; only those values (about 6 in 10^5) are redone
// with an IEEE division, in a branch the wavefront takes only when one of its
// lanes needs it.  A scale so small that 1/s overflows takes the division
// path for every value.  Results are clamped to [-127, 127].
template <int N>
__device__ __forceinline__ void quant_codes(const float (&x)[N], float s, int (&code)[N]) {
    // The division paths go one value at a time (scheduling barriers between
    // them), so their temporaries do not add to the caller's register peak.
    const float r = 1.0f / s;
    if (!(r < __builtin_inff())) {
#pragma unroll
        for (int e = 0; e < N; ++e) {
            code[e] = quant_code(x[e], s);
            __builtin_amdgcn_sched_barrier(0);
        }
        return;
    }
    float n[N];
    bool near = false;
#pragma unroll
    for (int e = 0; e < N; ++e) {
        const float t = x[e] * r;
        n[e] = __builtin_rintf(t);
        near |= fabsf(t - n[e]) > 0.5f - 0x1p-15f;   // |t - rne(t)| <= 1/2, and the difference is exact
    }
    if (__builtin_amdgcn_ballot_w64(near) != 0) {
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const float t = x[e] * r;
            if (fabsf(t - n[e]) > 0.5f - 0x1p-15f) n[e] = __builtin_rintf(x[e] / s);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int e = 0; e < N; ++e) code[e] = (int)__builtin_amdgcn_fmed3f(n[e], -127.0f, 127.0f);   // n is finite
}

// Four codes (already in [-127,127]) packed little-endian into one dword.
__device__ __forceinline__ uint32_t pack4(int c0, int c1, int c2, int c3) {
    return (uint32_t)(c0 & 0xff) | ((uint32_t)(c1 & 0xff) << 8) | ((uint32_t)(c2 & 0xff) << 16) |
           ((uint32_t)(c3 & 0xff) << 24);
}

__device__ __forceinline__ int sbyte(uint32_t w, int k) { return (int)(int8_t)(w >> (8 * k)); }

__device__ __forceinline__ int wave_id_uniform() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

}  // namespace jf
