// jf_gelu.h -- the GELU and GELU' evaluations used by the INT8 GELU kernels.
//
// GELU in its erf form (the non-linear operator of the Jetfire summary's INT8
// data flow, "Approach"): g(x) = x * Phi(x) with Phi the standard normal CDF,
// written as Phi(x) = erfc(-x/sqrt 2) / 2 so the negative tail keeps its
// relative accuracy.  Also included by the exhaustive error check under
// tests/, which measures gelu_fast against gelu_ref over every finite
// binary32 input.
#pragma once

#include <hip/hip_runtime.h>

#include "jf_normal_tail.h"

namespace jf {

// Reference value: evaluated in binary64, rounded once to binary32.
__device__ __forceinline__ float gelu_ref(float x) {
    const double xd = (double)x;
    return (float)(xd * (0.5 * erfc(-xd * 0.70710678118654752440)));
}

// The same value from the normal-tail expansion (jf_normal_tail.h), with
// every constant in scalar registers: the INT8 GELU kernel evaluates it once
// per wavefront (its blocks' largest values) and in rare fallbacks, through
// a call, where the library erfc's constants cost about 60 VALU moves.
// Phi(x) = 1 - Q(x) for x >= 0 and Q(-x) for x < 0, Q(z) = e^{-z^2/2} M(z);
// z*z is exact in binary64.
__device__ __forceinline__ float gelu_tail(float x) {
    const double xd = (double)x, z = fabs(xd);
    const double q = exp_neg_s(0.5 * (z * z)) * normal_tail_scaled_s(z);
    return (float)(xd * (xd >= 0.0 ? 1.0 - q : q));
}

// GELU'(z) (.x) and GELU'(-z) (.y) for z >= 0 in binary64 from the
// normal-tail expansion of jf_normal_tail.h (one exp, one division and a
// degree-24 polynomial: about a third of the instructions of the library's
// erfc and exp), each rounded once: d = Q(z) - z phi(z) =
// exp(-z^2/2) (M(z) - z/sqrt(2 pi)) is GELU'(-z), and
// GELU'(z) = Phi(z) + z phi(z) = 1 - d.  z*z is exact in binary64.
__device__ __forceinline__ float2 gelu_grad_pair_tail(float z) {
    const double zd = (double)z;
    const double d = exp(-0.5 * (zd * zd)) * (normal_tail_scaled(zd) - zd * 0.39894228040143267794);
    return make_float2((float)(1.0 - d), (float)d);
}

// Fast binary32 GELU for the code tables.  Phi(x) = 1 - Q(x) for x >= 0 and
// Q(-x) for x < 0, where Q is the upper tail of the standard normal
// distribution, approximated by formula 26.2.17 of Abramowitz & Stegun,
// "Handbook of Mathematical Functions" (Hastings' approximation):
//   Q(z) ~ Z(z) (b1 t + b2 t^2 + b3 t^3 + b4 t^4 + b5 t^5),  t = 1/(1 + p z),
//   Z(z) = exp(-z^2/2)/sqrt(2 pi), p = 0.2316419, absolute error < 7.5e-8;
// here with b_i/sqrt(2 pi) folded into the coefficients, the hardware
// reciprocal and base-2 exponential.  Over every binary32 input with
// |x| >= 2^-10 (and x = 0) its error against gelu_ref is at most 6.51e-7
// relative for x >= 0 and 2.14e-7 absolute for x < 0 (checked exhaustively;
// the table path only evaluates such inputs).
__device__ __forceinline__ float gelu_tail_q(float z) {   // Q(z), z >= 0
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.2316419f, z, 1.0f));
    const float c1 = 0.127414796f, c2 = -0.142248368f, c3 = 0.710706871f, c4 = -0.726576013f,
                c5 = 0.530702714f;
    const float poly = t * __builtin_fmaf(t, __builtin_fmaf(t, __builtin_fmaf(t, __builtin_fmaf(t, c5, c4), c3), c2), c1);
    return __builtin_amdgcn_exp2f(-0.72134752044448170368f * z * z) * poly;   // exp(-z^2/2) = 2^(-z^2/(2 ln 2))
}
__device__ __forceinline__ float gelu_fast(float x) {
    const float q = gelu_tail_q(fabsf(x));
    return x >= 0.0f ? x - x * q : x * q;
}

}  // namespace jf
