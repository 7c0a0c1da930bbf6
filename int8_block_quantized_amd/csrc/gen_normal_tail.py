"""Writes jf_normal_tail.h: the binary64 upper normal tail
Q(z) = erfc(z/sqrt 2)/2 used by the INT8 GELU backward kernel's derivative
tables (GELU'(x) = Phi(x) + x phi(x), the derivative of the erf form x Phi(x)
of the Jetfire summary's INT8 data flow, "Approach"; Phi(-z) = Q(z)) and by
the INT8 GELU forward kernel's binary64 reference (block maxima and rare
fallbacks), which also takes exp(-u) from this header (Cody-Waite reduction
by a two-part ln 2, degree-13 Taylor polynomial, within 1.2e-16 relative on
[0, 700]).

Q is written as Q(z) = M(z) exp(-z^2/2) with M(z) = Q(z) exp(z^2/2), a
smooth function that decays like 1/(z sqrt(2 pi)).  M is approximated by a
polynomial in t = (z - K)/(z + K), which maps [0, inf) onto [-1, 1) (the
change of variable Schonfelder uses for the Chebyshev expansions of erfc,
Math. Comp. 32, 1978):
    M(z) = K/(z + K) * P(t),   P(t) = sum_k a_k t^k,
with P the degree-N Chebyshev interpolant of M(z) (z + K)/K at the N + 1
Chebyshev points of t, computed here in 50-digit arithmetic (mpmath) and
converted to the power basis for Horner's rule.

Run:  python3 gen_normal_tail.py > jf_normal_tail.h   (needs mpmath; build-time
only, nothing at run time imports it).
"""
import sys

import mpmath as mp

K = 4
N = 24
mp.mp.dps = 50


def mills_scaled(z):
    z = mp.mpf(z)
    return mp.erfc(z / mp.sqrt(2)) / 2 * mp.exp(z * z / 2)


def target(t):
    z = K * (1 + t) / (1 - t)
    return mills_scaled(z) * (z + K) / K


def power_coefficients():
    nodes = [mp.cos(mp.pi * (j + mp.mpf(1) / 2) / (N + 1)) for j in range(N + 1)]
    vals = [target(t) for t in nodes]
    cheb = []
    for k in range(N + 1):
        s = sum(vals[j] * mp.cos(mp.pi * k * (j + mp.mpf(1) / 2) / (N + 1)) for j in range(N + 1))
        cheb.append(2 * s / (N + 1) if k else s / (N + 1))
    # T_k in the power basis, by T_k = 2 t T_{k-1} - T_{k-2}
    basis = [[mp.mpf(1)], [mp.mpf(0), mp.mpf(1)]]
    for k in range(2, N + 1):
        b = [mp.mpf(0)] * (k + 1)
        for i, v in enumerate(basis[k - 1]):
            b[i + 1] += 2 * v
        for i, v in enumerate(basis[k - 2]):
            b[i] -= v
        basis.append(b)
    power = [mp.mpf(0)] * (N + 1)
    for k in range(N + 1):
        for i, v in enumerate(basis[k]):
            power[i] += cheb[k] * v
    return [float(v) for v in power]


def max_rel_error(a):
    """Largest relative error of the binary64 Horner evaluation of M on
    [0, 40] (a grid plus special points), against 50-digit M."""
    worst = 0.0
    pts = [i * 2.0 / 400 for i in range(401)] + [2 + i * 38.0 / 400 for i in range(401)]
    pts += [1e-30, 1e-8, 0.75, 0.7518]
    for z in pts:
        w = 1.0 / (z + K)
        t = (z - K) * w
        p = a[-1]
        for v in reversed(a[:-1]):
            p = p * t + v
        m = p * (K * w)
        ref = mills_scaled(z)
        worst = max(worst, float(abs(mp.mpf(m) - ref) / ref))
    return worst


def main():
    a = power_coefficients()
    err = max_rel_error(a)
    out = sys.stdout
    out.write("// jf_normal_tail.h -- the upper normal tail Q(z) = erfc(z/sqrt 2)/2 in\n")
    out.write("// binary64, used by the INT8 GELU backward (its GELU' tables) and by the\n")
    out.write("// INT8 GELU forward (its binary64 reference for block maxima and rare\n")
    out.write("// fallbacks).  Written by gen_normal_tail.py: the Chebyshev interpolant of\n")
    out.write("// the scaled tail M(z) = Q(z) exp(z^2/2) in t = (z - 4)/(z + 4), degree\n")
    out.write(f"// {N} (largest relative error of M's binary64 evaluation on [0, 40]:\n")
    out.write(f"// {err:.2e}); for the forward GELU also exp(-u) by a Cody-Waite reduction\n")
    out.write("// with a two-part ln 2 and a degree-13 Taylor polynomial (within 1.2e-16\n")
    out.write("// relative on [0, 700]) and sreg(), which keeps binary64 constants in\n")
    out.write("// scalar registers.  Do not edit by hand.\n")
    out.write("#pragma once\n\n#include <hip/hip_runtime.h>\n\nnamespace jf {\n\n")
    out.write(f"constexpr double kTailK = {K}.0;\n")
    out.write(f"constexpr int kTailDegree = {N};\n")
    out.write("__device__ constexpr double kTailPoly[kTailDegree + 1] = {\n")
    for i, v in enumerate(a):
        out.write(f"    {float.hex(v)},  // t^{i}\n")
    out.write("};\n\n")
    out.write(
        "// M(z) = Q(z) exp(z^2/2) for z >= 0 (finite): a reciprocal, Horner in t.\n"
        "// w = 1/(z + K) from the hardware estimate and two Newton steps (each\n"
        "// squares the relative error, so w is within an ulp of the quotient),\n"
        "// not an IEEE division: a few ulps in t move M by ~1e-16 relative.\n"
        "__device__ __forceinline__ double normal_tail_scaled(double z) {\n"
        "    const double d = z + kTailK;\n"
        "    double w = __builtin_amdgcn_rcp(d);\n"
        "    w = __builtin_fma(w, __builtin_fma(-d, w, 1.0), w);\n"
        "    w = __builtin_fma(w, __builtin_fma(-d, w, 1.0), w);\n"
        "    const double t = (z - kTailK) * w;\n"
        "    double p = kTailPoly[kTailDegree];\n"
        "#pragma unroll\n"
        "    for (int k = kTailDegree - 1; k >= 0; --k) p = __builtin_fma(p, t, kTailPoly[k]);\n"
        "    return p * (kTailK * w);\n"
        "}\n\n")
    # e^{-u}: Cody-Waite reduction by ln 2 (a high part with 21 trailing zero
    # bits, so k * hi is exact for |k| < 2^21, and the low part), then the Taylor
    # polynomial of degree 13 on |r| <= ln2/2 (truncation below 4e-18 relative)
    hi = float.fromhex("0x1.62e42feep-1")
    lo = float(mp.log(2) - mp.mpf(hi))
    inv_fact = [float(1 / mp.factorial(n)) for n in range(13, -1, -1)]
    out.write(
        "// Forces a constant into scalar registers, so that a binary64 FMA takes it\n"
        "// as an operand (a literal would cost two VALU moves at each use outside a\n"
        "// loop the compiler can hoist it from).\n"
        "__device__ __forceinline__ double sreg(double c) {\n"
        "    __asm__(\"\" : \"+s\"(c));\n"
        "    return c;\n"
        "}\n\n")
    out.write(f"constexpr double kExpLn2Hi = {float.hex(hi)}, kExpLn2Lo = {float.hex(lo)};\n")
    out.write("constexpr double kExpInvFact[14] = {   // 1/13!, 1/12!, ..., 1/1!, 1/0!\n")
    for i, v in enumerate(inv_fact):
        out.write(f"    {float.hex(v)},\n")
    out.write("};\n\n")
    out.write(
        "// e^{-u} for u >= 0 with the constants in scalar registers: k = rne(u / ln 2),\n"
        "// r = u - k ln 2 (two FMAs), e^{-u} = 2^-k e^{-r}.  u is capped at 746, where\n"
        "// e^{-u} already rounds to 0 (and k stays far inside the int range).\n"
        "__device__ __forceinline__ double exp_neg_s(double u) {\n"
        "    u = __builtin_fmin(u, 746.0);\n"
        "    const double k = __builtin_rint(u * 1.4426950408889634074);\n"
        "    const double r = __builtin_fma(-k, sreg(kExpLn2Lo), __builtin_fma(-k, sreg(kExpLn2Hi), u));\n"
        "    double p = sreg(kExpInvFact[0]);\n"
        "#pragma unroll\n"
        "    for (int i = 1; i < 14; ++i) p = __builtin_fma(p, -r, sreg(kExpInvFact[i]));\n"
        "    return __builtin_amdgcn_ldexp(p, -(int)k);\n"
        "}\n\n"
        "// normal_tail_scaled with the polynomial's constants in scalar registers\n"
        "// (for a call made once per wavefront, outside any loop).\n"
        "__device__ __forceinline__ double normal_tail_scaled_s(double z) {\n"
        "    const double d = z + kTailK;\n"
        "    double w = __builtin_amdgcn_rcp(d);\n"
        "    w = __builtin_fma(w, __builtin_fma(-d, w, 1.0), w);\n"
        "    w = __builtin_fma(w, __builtin_fma(-d, w, 1.0), w);\n"
        "    const double t = (z - kTailK) * w;\n"
        "    double p = sreg(kTailPoly[kTailDegree]);\n"
        "#pragma unroll\n"
        "    for (int k = kTailDegree - 1; k >= 0; --k) p = __builtin_fma(p, t, sreg(kTailPoly[k]));\n"
        "    return p * (kTailK * w);\n"
        "}\n\n}  // namespace jf\n")


if __name__ == "__main__":
    main()
