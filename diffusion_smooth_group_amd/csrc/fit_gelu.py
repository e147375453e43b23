"""Derives the polynomial used by the GEMM epilogue's GELU.

GELU(x) = x Phi(x) with Phi(x) = 1 - E(|x|) for x >= 0 and E(|x|) for x < 0,
where E(a) = erfc(a / sqrt2) / 2; both cases are GELU(x) = max(x, 0) - |x| E(|x|),
one fused multiply-add after E.  The epilogue evaluates

    E(a) = 2^(-a^2 log2(e) / 2 + N(a)),   N(a) = log2(erfcx(a / sqrt2) / 2),

with N a degree-7 polynomial in a on [0, 4 sqrt2] (a is clamped there; beyond
it E < 8e-9, below float32 resolution next to 1 and negligible next to the
result's other terms).  N is smooth and slowly varying, so the fit is fitted
by iteratively reweighted least squares on Chebyshev nodes (converging toward
the minimax fit).  Degree 7 keeps the relative error of E below 6e-6; degree 6
(3e-5) is below a 16-bit output's half-ulp too, but flips enough fp16
roundings of an fc1 output to move some of fc2's 4-bit codes.  One exp2 and
ten other VALU instructions per element.

Run it to print the coefficients (lowest degree first) and the largest
relative error of E and of GELU for float32 evaluation on a dense grid.  Not
part of the build.
"""
import numpy as np
from scipy.special import erfc, erfcx

A_MAX = 4.0 * np.sqrt(2.0)
DEG = 7


def target(a):
    return np.log2(0.5 * erfcx(a / np.sqrt(2.0)))


def fit(deg=DEG, n=4000, passes=40):
    a = 0.5 * A_MAX * (1.0 - np.cos(np.pi * (np.arange(n) + 0.5) / n))
    y = target(a)
    w = np.ones(n)
    for _ in range(passes):
        V = np.vander(a, deg + 1, increasing=True)
        c, *_ = np.linalg.lstsq(V * w[:, None], y * w, rcond=None)
        e = np.abs(V @ c - y)
        w = w * (1.0 + 5.0 * e / e.max())
        w /= w.max()
    return c


def gelu_f32(x, c):
    """The epilogue's arithmetic, in float32."""
    f = np.float32
    x = x.astype(f)
    a = np.minimum(np.abs(x), f(A_MAX))
    p = np.full_like(a, f(c[-1]))
    for ci in c[-2::-1]:
        p = (p * a + f(ci)).astype(f)
    arg = (a * (a * f(-np.log2(np.e) / 2.0)) + p).astype(f)
    e = np.exp2(arg.astype(np.float64)).astype(f)
    # one rounding: max(x, 0) - |x| e
    return (np.maximum(x, f(0)).astype(np.float64) - np.abs(x).astype(np.float64) * e.astype(np.float64)).astype(f)


if __name__ == "__main__":
    c = fit()
    print("coefficients (a^0 .. a^%d):" % DEG, ", ".join("%.10e" % v for v in c))
    a = np.linspace(0.0, A_MAX, 400001)
    f = np.float32
    a32 = a.astype(f)
    p = np.full_like(a32, f(c[-1]))
    for ci in c[-2::-1]:
        p = (p * a32 + f(ci)).astype(f)
    E = np.exp2((a32 * (a32 * f(-np.log2(np.e) / 2.0)) + p).astype(np.float64))
    Eref = 0.5 * erfc(a32.astype(np.float64) / np.sqrt(2.0))
    print("max relative error of E on [0, 4 sqrt2]: %.2e" % (np.abs(E - Eref) / Eref).max())
    x = np.linspace(-8.0, 8.0, 400001)
    g = gelu_f32(x, c).astype(np.float64)
    x32 = x.astype(f).astype(np.float64)
    gref = 0.5 * x32 * erfc(-x32 / np.sqrt(2.0))
    big = np.abs(gref) > 1e-6
    print("max relative error of GELU where |GELU| > 1e-6: %.2e" % (np.abs(g - gref)[big] / np.abs(gref[big])).max())
    print("max absolute error of GELU on [-8, 8]: %.2e" % np.abs(g - gref).max())
