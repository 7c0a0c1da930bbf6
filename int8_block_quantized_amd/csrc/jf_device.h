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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, kWave));
    return v;
}

// Block scale from the block's max magnitude: one correctly rounded division
// (HIP keeps binary32 '/' IEEE-exact unless fast-math is requested).
__device__ __forceinline__ float block_scale(float absmax) { return absmax / 127.0f; }

// Code of one value under a non-zero scale: correctly rounded quotient,
// round-half-even, clamp to the symmetric INT8 range.
__device__ __forceinline__ int quant_code(float x, float s) {
    float r = __builtin_rintf(x / s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
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
