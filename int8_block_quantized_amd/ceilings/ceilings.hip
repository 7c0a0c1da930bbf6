// ceilings.hip -- measured ceilings for the benchmark (libjfceil.so).
//
// Not part of the hot path: register-only loops and streaming copies that
// bound what the library's kernels can reach on this GPU, timed with HIP
// events on the null stream.
//
//   JFC_MFMA_ONLY      v_mfma_i32_32x32x32_i8 back to back, four independent
//                      output blocks per wavefront (2 x 2 blocks sharing two
//                      A and two B fragments, as in the GEMM), four
//                      wavefronts per SIMD: the INT8 matrix-core rate.
//   JFC_MFMA_RESCALE   the same MFMAs, each followed by the GEMM's rescale of
//                      its 16 results per lane (v_cvt_f32_i32, then
//                      fma(sigma, P, acc)): the GEMM's arithmetic per
//                      (output block, k-block) with no memory traffic.
//   JFC_MFMA_BIAS      as JFC_MFMA_RESCALE with the partial converted
//                      through the MFMA's C operand (C = bits of 1.5 * 2^23,
//                      then one exact subtraction instead of the convert).
//   JFC_COPY_I8        int8 -> int8 streaming copy (the GELU's 1 + 1 bytes
//                      per element), 16-byte nontemporal loads and stores.
//   JFC_COPY_F32_I8    fp32 -> int8 narrowing stream (the quantize's 4 + 1
//                      bytes per element): 16 bytes read, 4 written per lane.
//   JFC_COPY_2I8_I8    two int8 inputs -> one int8 output (the GELU
//                      backward's and residual add's 1 + 1 + 1 bytes).
// The copies alternate between two input sets, each larger than the 256 MB
// Infinity Cache, so no launch finds its input cached.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { JFC_MFMA_ONLY = 0, JFC_MFMA_RESCALE = 1, JFC_MFMA_BIAS = 2, JFC_COPY_I8 = 3, JFC_COPY_F32_I8 = 4,
       JFC_COPY_2I8_I8 = 5 };

constexpr int kThreads = 256;   // four wavefronts, one per SIMD

template <int MODE>
__global__ __launch_bounds__(kThreads) void k_mfma_loop(int iters, float *out) {
    float acc[4][16];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][r] = 0.0f;
    v4i af[2], bf[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        af[b] = v4i{(int)threadIdx.x + b, 1, 2, 3};
        bf[b] = v4i{3, (int)threadIdx.x, 5 + b, 7};
    }
    float sigma = 1.0f + (float)threadIdx.x * 1e-7f;
    v16i bias;
#pragma unroll
    for (int r = 0; r < 16; ++r) bias[r] = 0x4B400000;
    for (int it = 0; it < iters; ++it) {
        // the operands look new every iteration, so nothing is hoisted
        asm volatile("" : "+v"(sigma), "+v"(af[0]), "+v"(af[1]), "+v"(bf[0]), "+v"(bf[1]));
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if constexpr (MODE == JFC_MFMA_ONLY) {
                const v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[b & 1], af[b >> 1], v16i{}, 0, 0, 0);
                asm volatile("" ::"v"(p));
            } else if constexpr (MODE == JFC_MFMA_RESCALE) {
                const v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[b & 1], af[b >> 1], v16i{}, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int pr = p[r];
                    acc[b][r] = __builtin_fmaf(sigma, (float)pr, acc[b][r]);
                }
            } else {
                const v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[b & 1], af[b >> 1], bias, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int pr = p[r];
                    acc[b][r] = __builtin_fmaf(sigma, __int_as_float(pr) - 12582912.0f, acc[b][r]);
                }
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[b][r];
    out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// Streaming copies (grid-stride): each thread moves kUnits 16-byte units per
// iteration, all loads issued before the stores, with nontemporal loads and
// stores (the data is touched once); the best of the layouts measured for a
// plain copy on this GPU.
constexpr int kUnits = 4;

__global__ __launch_bounds__(kThreads) void k_copy_i8(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                      int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * kThreads * kUnits;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnits + threadIdx.x; base < n16; base += stride) {
        u32x4 v[kUnits];
#pragma unroll
        for (int u = 0; u < kUnits; ++u)
            if (base + u * kThreads < n16) v[u] = __builtin_nontemporal_load(src + base + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnits; ++u)
            if (base + u * kThreads < n16) __builtin_nontemporal_store(v[u], dst + base + u * kThreads);
    }
}

// 16 bytes (four fp32 values) in, 4 bytes out per unit: the low byte of each
// value's bits (a narrowing stream without arithmetic).
__global__ __launch_bounds__(kThreads) void k_copy_f32_i8(const u32x4 *__restrict__ src, uint32_t *__restrict__ dst,
                                                          int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * kThreads * kUnits;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnits + threadIdx.x; base < n4; base += stride) {
        u32x4 v[kUnits];
#pragma unroll
        for (int u = 0; u < kUnits; ++u)
            if (base + u * kThreads < n4) v[u] = __builtin_nontemporal_load(src + base + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnits; ++u)
            if (base + u * kThreads < n4)
                __builtin_nontemporal_store((v[u].x & 0xffu) | (v[u].y & 0xffu) << 8 | (v[u].z & 0xffu) << 16 |
                                                (v[u].w & 0xffu) << 24,
                                            dst + base + u * kThreads);
    }
}

__global__ __launch_bounds__(kThreads) void k_copy_2i8_i8(const u32x4 *__restrict__ a, const u32x4 *__restrict__ b,
                                                          u32x4 *__restrict__ dst, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * kThreads * kUnits;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnits + threadIdx.x; base < n16; base += stride) {
        u32x4 v[kUnits], w[kUnits];
#pragma unroll
        for (int u = 0; u < kUnits; ++u)
            if (base + u * kThreads < n16) {
                v[u] = __builtin_nontemporal_load(a + base + u * kThreads);
                w[u] = __builtin_nontemporal_load(b + base + u * kThreads);
            }
#pragma unroll
        for (int u = 0; u < kUnits; ++u)
            if (base + u * kThreads < n16) __builtin_nontemporal_store(v[u] ^ w[u], dst + base + u * kThreads);
    }
}

}  // namespace

extern "C" {

// Runs measurement `which` (JFC_*), `reps` timed launches after one warm-up.
// MFMA loops: `size` = iterations per launch (4 MFMAs each per wavefront),
// 4 wavefronts per SIMD on 256 CUs; *rate = TOPS (2*32*32*32 ops per MFMA).
// Copies: `size` = bytes of ONE input set (multiple of 4096); the library
// allocates two input sets and one output, frees them before returning;
// *rate = GB/s of algorithmic bytes (bytes read + written per launch).
// *us = mean microseconds per launch.  Returns 0, or a hipError_t value.
__attribute__((visibility("default"))) int jfc_measure(int which, int64_t size, int reps, double *rate,
                                                       double *us) {
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return (int)hipErrorUnknown;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return (int)hipErrorUnknown;
    }
    hipError_t err = hipSuccess;
    double bytes_per_launch = 0.0, ops_per_launch = 0.0;
    void *in0 = nullptr, *in1 = nullptr, *in2 = nullptr, *in3 = nullptr, *out = nullptr;
    auto launch = [&](int rep) {
        if (which <= JFC_MFMA_BIAS) {
            const int wgs = 256 * 4;   // four wavefronts per SIMD
            if (which == JFC_MFMA_ONLY) hipLaunchKernelGGL(k_mfma_loop<JFC_MFMA_ONLY>, dim3(wgs), dim3(kThreads), 0, 0, (int)size, (float *)out);
            if (which == JFC_MFMA_RESCALE) hipLaunchKernelGGL(k_mfma_loop<JFC_MFMA_RESCALE>, dim3(wgs), dim3(kThreads), 0, 0, (int)size, (float *)out);
            if (which == JFC_MFMA_BIAS) hipLaunchKernelGGL(k_mfma_loop<JFC_MFMA_BIAS>, dim3(wgs), dim3(kThreads), 0, 0, (int)size, (float *)out);
        } else {
            const unsigned grid = 32768;
            void *a = (rep & 1) ? in1 : in0, *b = (rep & 1) ? in3 : in2;
            if (which == JFC_COPY_I8)
                hipLaunchKernelGGL(k_copy_i8, dim3(grid), dim3(kThreads), 0, 0, (const u32x4 *)a, (u32x4 *)out, size / 16);
            if (which == JFC_COPY_F32_I8)
                hipLaunchKernelGGL(k_copy_f32_i8, dim3(grid), dim3(kThreads), 0, 0, (const u32x4 *)a, (uint32_t *)out, size / 16);
            if (which == JFC_COPY_2I8_I8)
                hipLaunchKernelGGL(k_copy_2i8_i8, dim3(grid), dim3(kThreads), 0, 0, (const u32x4 *)a, (const u32x4 *)b, (u32x4 *)out, size / 16);
        }
    };
    if (which < JFC_MFMA_ONLY || which > JFC_COPY_2I8_I8 || size <= 0 || reps <= 0 || !rate || !us) {
        err = hipErrorInvalidValue;
    } else if (which <= JFC_MFMA_BIAS) {
        err = hipMalloc(&out, (size_t)256 * 4 * kThreads * sizeof(float));
        ops_per_launch = 256.0 * 4 * 4 /*waves*/ * (double)size * 4 /*MFMAs*/ * 2.0 * 32 * 32 * 32;
    } else if (size % 4096 != 0) {
        err = hipErrorInvalidValue;
    } else {
        const size_t n = (size_t)size;
        const size_t outb = which == JFC_COPY_F32_I8 ? n / 4 : n;
        err = hipMalloc(&in0, n);
        if (err == hipSuccess) err = hipMalloc(&in1, n);
        if (err == hipSuccess && which == JFC_COPY_2I8_I8) err = hipMalloc(&in2, n);
        if (err == hipSuccess && which == JFC_COPY_2I8_I8) err = hipMalloc(&in3, n);
        if (err == hipSuccess) err = hipMalloc(&out, outb);
        if (err == hipSuccess) err = hipMemset(in0, 0, n);
        if (err == hipSuccess) err = hipMemset(in1, 0, n);
        if (err == hipSuccess && in2) err = hipMemset(in2, 0, n);
        if (err == hipSuccess && in3) err = hipMemset(in3, 0, n);
        bytes_per_launch = (double)n * (which == JFC_COPY_2I8_I8 ? 2 : 1) + (double)outb;
    }
    if (err == hipSuccess) {
        launch(1);
        err = hipDeviceSynchronize();
    }
    if (err == hipSuccess) {
        err = hipEventRecord(e0, 0);
        for (int r = 0; r < reps; ++r) launch(r);
        if (err == hipSuccess) err = hipEventRecord(e1, 0);
        if (err == hipSuccess) err = hipEventSynchronize(e1);
    }
    if (err == hipSuccess) err = hipGetLastError();
    float ms = 0.0f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    if (err == hipSuccess) {
        *us = (double)ms * 1e3 / reps;
        *rate = which <= JFC_MFMA_BIAS ? ops_per_launch / (*us * 1e-6) / 1e12 : bytes_per_launch / (*us * 1e-6) / 1e9;
    }
    for (void *p : {in0, in1, in2, in3, out})
        if (p) (void)hipFree(p);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return (int)err;
}

}  // extern "C"
