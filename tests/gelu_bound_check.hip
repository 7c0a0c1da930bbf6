// Exhaustive checks of the INT8 GELU kernel's two GELU evaluations.
// (1) The binary32 GELU of its code tables (jf::gelu_fast) against the
// kernel's binary64 reference (jf::gelu_tail, the normal-tail expansion) over
// every binary32 input with |x| >= 2^-10, and x = 0 (the table path only sees
// those: its block scales are at least 0.17/127).  (2) gelu_tail against the
// definition written with the device library's binary64 erfc (jf::gelu_ref)
// over every finite binary32 input.  Prints: (1) max relative error for
// x >= 0, max absolute error for x < 0, number of inputs where the two
// differ; (2) number of inputs where gelu_tail and gelu_ref differ, and the
// largest difference in binary32 ulps.
// Test infrastructure: built by __graft_entry__.build(), run by
// tests/test_gpu_gelu.py.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include "../int8_block_quantized_amd/csrc/jf_gelu.h"

// distance in binary32 ulps (ordered integer images of the bit patterns)
__device__ unsigned ulp_dist(float a, float b) {
    int ia = __float_as_int(a), ib = __float_as_int(b);
    ia = ia < 0 ? (int)(0x80000000u - (unsigned)ia) : ia;
    ib = ib < 0 ? (int)(0x80000000u - (unsigned)ib) : ib;
    const long long d = (long long)ia - (long long)ib;
    return (unsigned)(d < 0 ? -d : d);
}

__global__ void check(unsigned *res) {
    const unsigned long long base = ((unsigned long long)blockIdx.x * blockDim.x + threadIdx.x) * 256ull;
    float mrel = 0.f, mabs = 0.f;
    unsigned diff = 0, tdiff = 0, tworst = 0;
    for (int i = 0; i < 256; ++i) {
        const float x = __uint_as_float((unsigned)(base + i));
        if (!(fabsf(x) < __builtin_inff())) continue;
        const float gd = jf::gelu_tail(x);
        const unsigned du = ulp_dist(gd, jf::gelu_ref(x));
        tdiff += du != 0;
        tworst = max(tworst, du);
        if (x != 0.f && fabsf(x) < 0x1p-10f) continue;
        const float gf = jf::gelu_fast(x);
        if (gf == gd) continue;
        ++diff;
        const float d = fabsf(gf - gd);
        if (x >= 0.f) mrel = fmaxf(mrel, gd != 0.f ? d / fabsf(gd) : 1.f);
        else mabs = fmaxf(mabs, d);
    }
    atomicMax(&res[0], __float_as_uint(mrel));
    atomicMax(&res[1], __float_as_uint(mabs));
    atomicAdd(&res[2], diff);
    atomicAdd(&res[3], tdiff);
    atomicMax(&res[4], tworst);
}

int main() {
    unsigned *d = nullptr, h[5];
    if (hipMalloc(&d, sizeof h) != hipSuccess || hipMemset(d, 0, sizeof h) != hipSuccess) return 2;
    hipLaunchKernelGGL(check, dim3(65536), dim3(256), 0, 0, d);   // 2^32 inputs, 256 per thread
    if (hipMemcpy(h, d, sizeof h, hipMemcpyDeviceToHost) != hipSuccess) return 3;
    float rel, abs_;
    memcpy(&rel, &h[0], 4);
    memcpy(&abs_, &h[1], 4);
    printf("%.6e %.6e %u %u %u\n", rel, abs_, h[2], h[3], h[4]);
    return 0;
}
