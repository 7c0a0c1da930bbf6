"""CPU check of the coefficients in jf_normal_tail.h (the binary64 expansion of
the upper normal tail that the INT8 GELU backward kernel uses for GELU' and the
INT8 GELU forward kernel uses for its binary64 reference, with the header's
exp(-u)).

M(z) = Q(z) exp(z^2/2), Q the upper normal tail, is evaluated from the
header's power-basis coefficients in t = (z - K)/(z + K) with binary64
Horner as the kernel does (here with an IEEE division for 1/(z + K); the
kernel's Newton-refined reciprocal is within an ulp of it), and compared
with 50-digit mpmath: relative error below 1e-15 on [0, 40].  The GELU' pair built from it must round to the
correctly rounded binary32 values of Phi(x) + x phi(x) (50-digit mpmath) on a
seeded sample of inputs and at the special points x = 0, the zero of GELU'
near -0.7518 and the tails.
"""
import os
import re

import mpmath as mp
import numpy as np

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "int8_block_quantized_amd", "csrc", "jf_normal_tail.h")


def header_constants():
    text = open(HDR).read()
    k = float(re.search(r"kTailK = ([0-9.]+);", text).group(1))
    n = int(re.search(r"kTailDegree = (\d+);", text).group(1))
    coeffs = [float.fromhex(c) for c in re.findall(r"^\s+(-?0x[0-9a-fp.+-]+),\s+// t\^\d+$", text, re.M)]
    assert len(coeffs) == n + 1
    return k, coeffs


def m_header(z, k, a):
    w = 1.0 / (z + k)
    t = (z - k) * w
    p = a[-1]
    for v in reversed(a[:-1]):
        p = p * t + v
    return p * (k * w)


def pair_header(x, k, a):
    z = float(x)
    d = np.exp(-0.5 * (z * z)) * (m_header(z, k, a) - z * 0.39894228040143267794)
    return np.float32(1.0 - d), np.float32(d)


def grad_exact(x):
    x = mp.mpf(float(x))
    return mp.erfc(-x / mp.sqrt(2)) / 2 + x * mp.exp(-x * x / 2) / mp.sqrt(2 * mp.pi)


def to_f32(v):
    # correctly rounded binary32 of a 50-digit value (via an exact rational
    # comparison with the two binary32 neighbours of its binary64 image)
    f = np.float32(float(v))
    lo, hi = np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))
    best = min((f, lo, hi), key=lambda c: abs(mp.mpf(float(c)) - v))
    return best


def test_scaled_tail_relative_error():
    mp.mp.dps = 50
    k, a = header_constants()
    zs = list(np.linspace(0, 2, 201)) + list(np.linspace(2, 40, 191)) + [1e-30, 1e-8, 0.75, 0.7518]
    worst = 0.0
    for z in zs:
        z = float(z)
        zm = mp.mpf(z)
        ref = mp.erfc(zm / mp.sqrt(2)) / 2 * mp.exp(zm * zm / 2)
        worst = max(worst, float(abs(mp.mpf(m_header(z, k, a)) - ref) / ref))
    assert worst < 1e-15, worst


def test_pair_rounds_like_the_exact_derivative():
    mp.mp.dps = 50
    k, a = header_constants()
    g = np.random.default_rng(7)
    xs = np.concatenate([g.uniform(0, 15, 1500), 10 ** g.uniform(-7, 1.1, 500),
                         [0.0, 0.7518, 0.75183, 5.9, 14.0, 14.5, 20.0]]).astype(np.float32)
    bad = 0
    for x in xs:
        pos, neg = pair_header(x, k, a)
        bad += int(pos != to_f32(grad_exact(x))) + int(neg != to_f32(grad_exact(-x)))
    assert bad == 0, bad
    assert pair_header(np.float32(0), k, a) == (np.float32(0.5), np.float32(0.5))



def exp_constants():
    text = open(HDR).read()
    hi = float.fromhex(re.search(r"kExpLn2Hi = (-?0x[0-9a-fp.+-]+)", text).group(1))
    lo = float.fromhex(re.search(r"kExpLn2Lo = (-?0x[0-9a-fp.+-]+)", text).group(1))
    body = text[text.index("kExpInvFact[14]"):]
    body = body[:body.index("};")]
    inv = [float.fromhex(c) for c in re.findall(r"^\s+(-?0x[0-9a-fp.+-]+),$", body, re.M)]
    assert len(inv) == 14
    return hi, lo, inv


def fma(a, b, c):
    return float(mp.mpf(a) * mp.mpf(b) + mp.mpf(c))


def exp_neg_header(u, hi, lo, inv):
    u = min(u, 746.0)
    k = float(round(u * 1.4426950408889634074))      # round half to even, like rint
    r = fma(-k, lo, fma(-k, hi, u))
    p = inv[0]
    for c in inv[1:]:
        p = fma(p, -r, c)
    return float(mp.ldexp(mp.mpf(p), -int(k)))


def test_exp_reduction_constants():
    """ln 2 split (the high part with 21 trailing zero bits, so k*hi is exact
    for |k| < 2^21; k <= 1077 here), 1/n! rounded once, and e^{-u} from them within 2 binary64
    ulps of 50-digit exp on [0, 700] (FMAs emulated exactly)."""
    mp.mp.dps = 50
    hi, lo, inv = exp_constants()
    assert abs(mp.mpf(hi) + mp.mpf(lo) - mp.log(2)) < mp.mpf(2) ** -80
    assert (np.float64(hi).view(np.uint64) & np.uint64((1 << 21) - 1)) == 0   # low 21 mantissa bits zero
    for i, v in enumerate(inv):
        assert v == float(1 / mp.factorial(13 - i))
    g = np.random.default_rng(9)
    us = list(g.uniform(0, 120, 400)) + list(g.uniform(0, 1, 200)) + [0.0, 0.3465, 0.3466, 30.1656, 700.0]
    worst = max(float(abs(mp.mpf(exp_neg_header(float(u), hi, lo, inv)) - mp.exp(-mp.mpf(float(u)))) /
                      mp.exp(-mp.mpf(float(u)))) for u in us)
    assert worst < 2 * 2.0 ** -53, worst
    assert exp_neg_header(800.0, hi, lo, inv) == 0.0


def test_gelu_value_rounds_like_the_exact_value():
    """The forward kernel's binary64 reference GELU (x Phi(x) from the tail
    expansion and the exp above) rounds to the correctly rounded binary32
    value of 50-digit x Phi(x) on a seeded sample and at special points."""
    mp.mp.dps = 50
    k, a = header_constants()
    hi, lo, inv = exp_constants()
    g = np.random.default_rng(8)
    xs = np.concatenate([g.uniform(-15, 15, 1200), 10 ** g.uniform(-7, 1.1, 250),
                         -(10 ** g.uniform(-7, 1.1, 250)), [0.0, -0.7518, 5.9, -5.9, -14.0, 30.0, 1e4]]).astype(np.float32)
    bad = 0
    for x in xs:
        xd = float(x)
        z = abs(xd)
        q = exp_neg_header(0.5 * z * z, hi, lo, inv) * m_header(z, k, a)
        got = np.float32(xd * (1.0 - q if xd >= 0 else q))
        xm = mp.mpf(xd)
        bad += int(got != to_f32(xm * mp.erfc(-xm / mp.sqrt(2)) / 2))
    assert bad == 0, bad
