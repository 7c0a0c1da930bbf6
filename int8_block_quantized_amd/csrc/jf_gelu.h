// jf_gelu.h -- the two GELU evaluations used by the INT8 GELU kernel.
//
// GELU in its erf form (the non-linear operator of the Jetfire summary's INT8
// data flow, "Approach"): g(x) = x * Phi(x) with Phi the standard normal CDF,
// written as Phi(x) = erfc(-x/sqrt 2) / 2 so the negative tail keeps its
// relative accuracy.  Also included by the exhaustive error check under
// tests/, which measures gelu_fast against gelu_ref over every finite
// binary32 input.
#pragma once

#include <hip/hip_runtime.h>

namespace jf {

// Reference value: evaluated in binary64, rounded once to binary32.
__device__ __forceinline__ float gelu_ref(float x) {
    const double xd = (double)x;
    return (float)(xd * (0.5 * erfc(-xd * 0.70710678118654752440)));
}

// The same formula in binary32.  Over every finite binary32 input its error
// against gelu_ref is at most 2.93e-7 relative for x >= 0 and 4.48e-8
// absolute for x < 0 (the kernel's tie window is derived from these).
__device__ __forceinline__ float gelu_fast(float x) {
    return x * (0.5f * erfcf(-x * 0.70710678118654752440f));
}

}  // namespace jf
