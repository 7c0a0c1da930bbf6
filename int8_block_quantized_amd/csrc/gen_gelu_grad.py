"""Writes jf_gelu_grad.h: the binary64 evaluation of GELU' used by the INT8
GELU backward kernel's derivative tables.

GELU'(x) = Phi(x) + x phi(x) (the derivative of the erf form x Phi(x), the
non-linear operator of the Jetfire summary's INT8 data flow, "Approach").
For z >= 0 both GELU'(z) and GELU'(-z) follow from the upper normal tail
Q(z) = erfc(z/sqrt 2)/2 and phi(z):
    GELU'(-z) = Q(z) - z phi(z),    GELU'(z) = 1 - GELU'(-z).
Q is written as Q(z) = M(z) exp(-z^2/2) with M(z) = Q(z) exp(z^2/2), a
smooth function that decays like 1/(z sqrt(2 pi)).  M is approximated by a
polynomial in t = (z - K)/(z + K), which maps [0, inf) onto [-1, 1) (the
change of variable Schonfelder uses for the Chebyshev expansions of erfc,
Math. Comp. 32, 1978):
    M(z) = K/(z + K) * P(t),   P(t) = sum_k a_k t^k,
with P the degree-N Chebyshev interpolant of M(z) (z + K)/K at the N + 1
Chebyshev points of t, computed here in 50-digit arithmetic (mpmath) and
converted to the power basis for Horner's rule.

Run:  python3 gen_gelu_grad.py > jf_gelu_grad.h   (needs mpmath; build-time
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
    out.write("// jf_gelu_grad.h -- GELU'(z) and GELU'(-z) in binary64 for the INT8 GELU\n")
    out.write("// backward's derivative tables.  Written by gen_gelu_grad.py (Chebyshev\n")
    out.write("// interpolant of the scaled normal tail M(z) = Q(z) exp(z^2/2) in\n")
    out.write(f"// t = (z - {K})/(z + {K}), degree {N}; largest relative error of M's binary64\n")
    out.write(f"// evaluation on [0, 40]: {err:.2e}).  Do not edit by hand.\n")
    out.write("#pragma once\n\n#include <hip/hip_runtime.h>\n\nnamespace jf {\n\n")
    out.write(f"constexpr double kGradK = {K}.0;\n")
    out.write(f"constexpr int kGradDegree = {N};\n")
    out.write("__device__ constexpr double kGradPoly[kGradDegree + 1] = {\n")
    for i, v in enumerate(a):
        out.write(f"    {float.hex(v)},  // t^{i}\n")
    out.write("};\n\n")
    out.write(
        "// GELU'(z) (.x) and GELU'(-z) (.y) for z >= 0, each rounded once to\n"
        "// binary32: d = exp(-z^2/2) (M(z) - z/sqrt(2 pi)) = Q(z) - z phi(z) is\n"
        "// GELU'(-z) and 1 - d is GELU'(z).  z*z is exact in binary64 (z is a\n"
        "// binary32 value).\n"
        "__device__ __forceinline__ float2 gelu_grad_pair_fast(float z) {\n"
        "    const double zd = (double)z;\n"
        "    const double w = 1.0 / (zd + kGradK);\n"
        "    const double t = (zd - kGradK) * w;\n"
        "    double p = kGradPoly[kGradDegree];\n"
        "#pragma unroll\n"
        "    for (int k = kGradDegree - 1; k >= 0; --k) p = __builtin_fma(p, t, kGradPoly[k]);\n"
        "    const double m = p * (kGradK * w);\n"
        "    const double d = exp(-0.5 * (zd * zd)) * (m - zd * 0.39894228040143267794);\n"
        "    return make_float2((float)(1.0 - d), (float)d);\n"
        "}\n\n}  // namespace jf\n")


if __name__ == "__main__":
    main()
