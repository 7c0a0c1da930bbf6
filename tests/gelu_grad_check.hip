// Exhaustive check of the binary64 GELU' evaluation used by the INT8 GELU
// backward kernel's derivative tables (jf::gelu_grad_pair_tail, from the
// scaled normal-tail polynomial) against the same quantities written with the
// device library's binary64 erfc and exp: Phi(-z) = erfc(z/sqrt 2)/2,
// z phi(z) = z exp(-z^2/2)/sqrt(2 pi), GELU'(z) = (1 - Phi(-z)) + z phi(z),
// GELU'(-z) = Phi(-z) - z phi(z), each rounded once to binary32.  Covers
// every finite binary32 z >= 0.  Prints: number of outputs that differ, the
// largest difference in units in the last place of binary32.
// Test infrastructure: built by __graft_entry__.build(), run by
// tests/test_gpu_gelu_bwd.py.
#include <hip/hip_runtime.h>
#include <stdio.h>

#include "../int8_block_quantized_amd/csrc/jf_gelu.h"

__device__ float2 grad_pair_libm(float z) {
    const double zd = (double)z;
    const double q = 0.5 * erfc(zd * 0.70710678118654752440);
    const double zpdf = zd * (exp(-0.5 * zd * zd) * 0.39894228040143267794);
    return make_float2((float)((1.0 - q) + zpdf), (float)(q - zpdf));
}

// distance in binary32 ulps (ordered integer images of the bit patterns)
__device__ unsigned ulp_dist(float a, float b) {
    int ia = __float_as_int(a), ib = __float_as_int(b);
    ia = ia < 0 ? (int)(0x80000000u - (unsigned)ia) : ia;
    ib = ib < 0 ? (int)(0x80000000u - (unsigned)ib) : ib;
    const long long d = (long long)ia - (long long)ib;
    return (unsigned)(d < 0 ? -d : d);
}

__global__ void check(unsigned *res) {
    const unsigned base = (blockIdx.x * blockDim.x + threadIdx.x) * 128u;
    unsigned diff = 0, worst = 0;
    for (unsigned i = 0; i < 128; ++i) {
        const unsigned u = base + i;
        if (u > 0x7f7fffffu) break;                       // finite, non-negative
        const float z = __uint_as_float(u);
        const float2 f = jf::gelu_grad_pair_tail(z), r = grad_pair_libm(z);
        const unsigned dx = ulp_dist(f.x, r.x), dy = ulp_dist(f.y, r.y);
        diff += (dx != 0) + (dy != 0);
        worst = max(worst, max(dx, dy));
    }
    atomicAdd(&res[0], diff);
    atomicMax(&res[1], worst);
}

int main() {
    unsigned *d = nullptr, h[2];
    if (hipMalloc(&d, sizeof h) != hipSuccess || hipMemset(d, 0, sizeof h) != hipSuccess) return 2;
    // 2^31 patterns, 128 per thread: 65536 x 256 threads
    hipLaunchKernelGGL(check, dim3(65536), dim3(256), 0, 0, d);
    if (hipMemcpy(h, d, sizeof h, hipMemcpyDeviceToHost) != hipSuccess) return 3;
    printf("%u %u\n", h[0], h[1]);
    return 0;
}
