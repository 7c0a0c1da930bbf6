// jf_normal_tail.h -- the upper normal tail Q(z) = erfc(z/sqrt 2)/2 in
// binary64, used by the INT8 GELU backward (its GELU' tables) and by the
// INT8 GELU forward (its binary64 reference for block maxima and rare
// fallbacks).  Written by gen_normal_tail.py: the Chebyshev interpolant of
// the scaled tail M(z) = Q(z) exp(z^2/2) in t = (z - 4)/(z + 4), degree
// 24 (largest relative error of M's binary64 evaluation on [0, 40]:
// 4.50e-16); for the forward GELU also exp(-u) by a Cody-Waite reduction
// with a two-part ln 2 and a degree-13 Taylor polynomial (within 1.2e-16
// relative on [0, 700]) and sreg(), which keeps binary64 constants in
// scalar registers.  Do not edit by hand.
#pragma once

#include <hip/hip_runtime.h>

namespace jf {

constexpr double kTailK = 4.0;
constexpr int kTailDegree = 24;
__device__ constexpr double kTailPoly[kTailDegree + 1] = {
    0x1.82b4bb8c94dcep-3,  // t^0
    -0x1.373e3a893c28cp-3,  // t^1
    0x1.8c6dbf2cfc2afp-4,  // t^2
    -0x1.7dff2bff68052p-5,  // t^3
    0x1.eec4cc3e4db3ep-7,  // t^4
    -0x1.ee2761054e5e1p-10,  // t^5
    -0x1.c81719d60dcdbp-11,  // t^6
    0x1.ab825ff09481bp-12,  // t^7
    0x1.17a4aec9fa29ap-15,  // t^8
    -0x1.e4a431b3465b0p-15,  // t^9
    -0x1.001f7d33a2ff5p-21,  // t^10
    0x1.26d193750d626p-17,  // t^11
    0x1.80ca2044c09bdp-23,  // t^12
    -0x1.8d64fadf80ed1p-20,  // t^13
    -0x1.523a2fde9b829p-23,  // t^14
    0x1.1319f41c90a11p-22,  // t^15
    0x1.24d40b9cf1122p-24,  // t^16
    -0x1.5739b1a22c213p-25,  // t^17
    -0x1.763bb001aa685p-26,  // t^18
    0x1.33354e7ae3599p-28,  // t^19
    0x1.7329462b6b607p-28,  // t^20
    -0x1.4b02181dd18fdp-33,  // t^21
    -0x1.04ffdbe7bdef2p-30,  // t^22
    -0x1.0236305d3fd38p-35,  // t^23
    0x1.828df1c3afaadp-34,  // t^24
};

// M(z) = Q(z) exp(z^2/2) for z >= 0 (finite): a reciprocal, Horner in t.
// w = 1/(z + K) from the hardware estimate and two Newton steps (each
// squares the relative error, so w is within an ulp of the quotient),
// not an IEEE division: a few ulps in t move M by ~1e-16 relative.
__device__ __forceinline__ double normal_tail_scaled(double z) {
    const double d = z + kTailK;
    double w = __builtin_amdgcn_rcp(d);
    w = __builtin_fma(w, __builtin_fma(-d, w, 1.0), w);
    w = __builtin_fma(w, __builtin_fma(-d, w, 1.0), w);
    const double t = (z - kTailK) * w;
    double p = kTailPoly[kTailDegree];
#pragma unroll
    for (int k = kTailDegree - 1; k >= 0; --k) p = __builtin_fma(p, t, kTailPoly[k]);
    return p * (kTailK * w);
}

// Forces a constant into scalar registers, so that a binary64 FMA takes it
// as an operand (a literal would cost two VALU moves at each use outside a
// loop the compiler can hoist it from).
__device__ __forceinline__ double sreg(double c) {
    __asm__("" : "+s"(c));
    return c;
}

constexpr double kExpLn2Hi = 0x1.62e42fee00000p-1, kExpLn2Lo = 0x1.a39ef35793c76p-33;
constexpr double kExpInvFact[14] = {   // 1/13!, 1/12!, ..., 1/1!, 1/0!
    0x1.6124613a86d09p-33,
    0x1.1eed8eff8d898p-29,
    0x1.ae64567f544e4p-26,
    0x1.27e4fb7789f5cp-22,
    0x1.71de3a556c734p-19,
    0x1.a01a01a01a01ap-16,
    0x1.a01a01a01a01ap-13,
    0x1.6c16c16c16c17p-10,
    0x1.1111111111111p-7,
    0x1.5555555555555p-5,
    0x1.5555555555555p-3,
    0x1.0000000000000p-1,
    0x1.0000000000000p+0,
    0x1.0000000000000p+0,
};

// e^{-u} for u >= 0 with the constants in scalar registers: k = rne(u / ln 2),
// r = u - k ln 2 (two FMAs), e^{-u} = 2^-k e^{-r}.  u is capped at 746, where
// e^{-u} already rounds to 0 (and k stays far inside the int range).
__device__ __forceinline__ double exp_neg_s(double u) {
    u = __builtin_fmin(u, 746.0);
    const double k = __builtin_rint(u * 1.4426950408889634074);
    const double r = __builtin_fma(-k, sreg(kExpLn2Lo), __builtin_fma(-k, sreg(kExpLn2Hi), u));
    double p = sreg(kExpInvFact[0]);
#pragma unroll
    for (int i = 1; i < 14; ++i) p = __builtin_fma(p, -r, sreg(kExpInvFact[i]));
    return __builtin_amdgcn_ldexp(p, -(int)k);
}

// normal_tail_scaled with the polynomial's constants in scalar registers
// (for a call made once per wavefront, outside any loop).
__device__ __forceinline__ double normal_tail_scaled_s(double z) {
    const double d = z + kTailK;
    double w = __builtin_amdgcn_rcp(d);
    w = __builtin_fma(w, __builtin_fma(-d, w, 1.0), w);
    w = __builtin_fma(w, __builtin_fma(-d, w, 1.0), w);
    const double t = (z - kTailK) * w;
    double p = sreg(kTailPoly[kTailDegree]);
#pragma unroll
    for (int k = kTailDegree - 1; k >= 0; --k) p = __builtin_fma(p, t, sreg(kTailPoly[k]));
    return p * (kTailK * w);
}

}  // namespace jf
