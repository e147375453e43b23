"""Derives the erfc coefficients used by the GEMM epilogue's GELU.

erfc(z) for z >= 0 is written as t * exp(-z^2 + P(t)) with t = 1 / (1 + z/2),
which maps [0, inf) onto (0, 1]; P(t) = log(erfcx(z) / t) is smooth there
(P(0+) = -log(2 sqrt(pi)), P(1) = 0).  A degree-9 polynomial fitted by
iteratively reweighted least squares on Chebyshev nodes (converging toward
the minimax fit) keeps |P_fit - P| below 1e-7 on the whole interval, i.e. a
relative error of erfc below 1e-7.  Run it to print the coefficients, lowest
degree first, and the maximum error on a dense grid.  Not part of the build.
"""
import numpy as np
from scipy.special import erfcx


def target(t):
    z = 2.0 * (1.0 / t - 1.0)
    return np.log(erfcx(z) / t)


def fit(deg=9, n=4000, passes=60):
    x = 0.5 - 0.5 * np.cos(np.pi * (np.arange(n) + 0.5) / n)
    x = np.clip(x, 1e-6, 1.0)
    y = target(x)
    w = np.ones(n)
    for _ in range(passes):
        V = np.vander(x, deg + 1, increasing=True)
        c, *_ = np.linalg.lstsq(V * w[:, None], y * w, rcond=None)
        e = V @ c - y
        w = w * (np.abs(e) / np.abs(e).max() + 1e-3) ** 0.5
        w /= w.max()
    return c


if __name__ == "__main__":
    c = fit()
    t = np.linspace(1e-6, 1.0, 200001)
    print("coefficients (t^0 .. t^9):", ", ".join("%.10f" % v for v in c))
    print("max |P_fit - P| = %.2e" % np.abs(np.polyval(c[::-1], t) - target(t)).max())
