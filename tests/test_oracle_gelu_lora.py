"""Pins for the oracle's GELU and LoRA attach (CPU only).

GELU (the erf form x Phi(x), used for the FLUX MLP's fc1 output; the pages
do not give the activation) is checked against the standard normal
distribution computed independently -- Phi by numerical quadrature of the
Gaussian density -- and against identities that fix it: Phi(x) + Phi(-x) = 1
gives GELU(x) - GELU(-x) = x, GELU(0) = 0 with slope 1/2, GELU(x) -> x for
large x and -> 0 for very negative x, and GELU'(x) = Phi(x) + x phi(x).

LoRA attach [SVDQuant §5.2, integrating LoRA: the LoRA's factors join the
16-bit low-rank branch and the 4-bit residual is not re-quantized]: with the
LoRA attached, the layer's pre-rounding output must grow by exactly
round16(X A) round16(alpha B) -- the LoRA acting on the raw input X, not on
the smoothed X_hat -- and nothing else may change.  The expected increment
is built here with scalar exact sums (math.fsum) and numpy's own
float64 -> float16 conversion, not with the oracle's rounding routine.
"""
import math

import numpy as np
import pytest
from scipy import integrate

import oracle as o


# ------------------------------------------------------------------- GELU
def _phi_quad(x):
    """Standard normal CDF by adaptive quadrature of the density."""
    dens = lambda t: math.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)
    if x >= 0:
        v, _ = integrate.quad(dens, 0.0, x, epsabs=1e-15, epsrel=1e-14, limit=200)
        return 0.5 + v
    v, _ = integrate.quad(dens, x, 0.0, epsabs=1e-15, epsrel=1e-14, limit=200)
    return 0.5 - v


def test_gelu_closed_values():
    # Phi(1) = 0.8413447460685429..., Phi(-1) = 0.15865525393145707...
    g = o.gelu_erf(np.array([1.0, -1.0, 0.0, -0.0]))
    assert abs(g[0] - 0.8413447460685429) < 1e-15
    assert abs(g[1] - (-0.15865525393145707)) < 1e-15
    assert g[2] == 0.0 and g[3] == 0.0


def test_gelu_matches_quadrature_of_the_density():
    xs = np.concatenate([np.linspace(-6.0, 6.0, 97), [-0.3, 0.01, 0.7071067811865476, 2.5, -3.75]])
    g = o.gelu_erf(xs)
    ref = np.array([x * _phi_quad(x) for x in xs])
    assert np.max(np.abs(g - ref)) < 1e-13


def test_gelu_odd_part_is_identity():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(2000) * 3, rng.uniform(-40, 40, 200)])
    d = o.gelu_erf(x) - o.gelu_erf(-x)
    assert np.max(np.abs(d - x) / np.maximum(1.0, np.abs(x))) < 1e-14


def test_gelu_slope_at_zero_and_derivative():
    h = 1e-6
    s0 = (o.gelu_erf(np.array([h]))[0] - o.gelu_erf(np.array([-h]))[0]) / (2 * h)
    assert abs(s0 - 0.5) < 1e-9
    for x in (-2.0, -0.5, 0.8, 1.9, 3.1):
        num = (o.gelu_erf(np.array([x + h]))[0] - o.gelu_erf(np.array([x - h]))[0]) / (2 * h)
        ana = _phi_quad(x) + x * math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)
        assert abs(num - ana) < 1e-8


def test_gelu_tails():
    # 1 - Phi(10) is about 7.6e-24, far below half an ulp of 10
    g = o.gelu_erf(np.array([10.0, 40.0, -10.0, -40.0]))
    assert g[0] == 10.0 and g[1] == 40.0
    assert -1e-21 < g[2] <= 0.0 and g[3] == 0.0


# ------------------------------------------------------------------- LoRA
def _f16(x):
    """float64 -> fp16 value (numpy's correctly rounded conversion)."""
    return np.float64(np.float16(x))


def _lora_layer(alpha, seed=5):
    rng = np.random.default_rng(seed)
    M, K, N, r, rL = 5, 128, 12, 3, 2
    X = rng.standard_normal((M, K)) * 0.5
    X[:, 7] *= 20.0                               # an outlier channel, so lambda != 1
    W = rng.standard_normal((K, N)) * 0.05
    A = rng.standard_normal((K, rL)) * 0.3
    B = rng.standard_normal((rL, N)) * 0.3
    bits = lambda a: a.astype(np.float16).view(np.uint16)
    Xb, Wb, Ab, Bb = bits(X), bits(W), bits(A), bits(B)
    base = o.pack(Wb, o.F16, o.activation_absmax(o.decode16(Xb, o.F16)), r, o.INT4)
    assert np.any(base["lam"] != 1.0)
    with_l = o.attach_lora(base, Ab, Bb, alpha)
    return Xb, Ab, Bb, base, with_l


def _expected_increment(Xb, Ab, Bb, alpha):
    """round16(X A) round16(alpha B), scalar exact sums."""
    X = Xb.view(np.float16).astype(np.float64)
    A = Ab.view(np.float16).astype(np.float64)
    B = Bb.view(np.float16).astype(np.float64)
    M, K = X.shape
    rL, N = B.shape
    T = np.array([[_f16(math.fsum(X[m, k] * A[k, j] for k in range(K))) for j in range(rL)] for m in range(M)])
    Bq = np.array([[_f16(alpha * B[j, n]) for n in range(N)] for j in range(rL)])
    return np.array([[math.fsum(T[m, j] * Bq[j, n] for j in range(rL)) for n in range(N)] for m in range(M)])


@pytest.mark.parametrize("alpha", [1.0, 0.3, -1.7])
def test_lora_adds_exactly_its_own_product_on_raw_x(alpha):
    Xb, Ab, Bb, base, with_l = _lora_layer(alpha)
    _, p0 = o.forward(base, Xb, return_parts=True)
    _, p1 = o.forward(with_l, Xb, return_parts=True)
    inc = p1["Y64"] - p0["Y64"]
    ref = _expected_increment(Xb, Ab, Bb, alpha)
    scale = max(1.0, np.abs(p0["Y64"]).max())
    assert np.max(np.abs(inc - ref)) < 1e-13 * scale
    assert np.max(np.abs(ref)) > 1e-2            # the LoRA is not negligible here


def test_lora_leaves_residual_and_branch_untouched():
    Xb, Ab, Bb, base, with_l = _lora_layer(0.3)
    r = base["L1x"].shape[1]
    assert np.array_equal(with_l["qw"], base["qw"]) and np.array_equal(with_l["sw"], base["sw"])
    assert np.array_equal(with_l["L1x"][:, :r], base["L1x"]) and np.array_equal(with_l["L2q"][:r], base["L2q"])
    assert np.array_equal(with_l["lam"], base["lam"]) and np.array_equal(with_l["invlam"], base["invlam"])
    # the 4-bit product and the rank-r part of the branch are unchanged
    _, p0 = o.forward(base, Xb, return_parts=True)
    _, p1 = o.forward(with_l, Xb, return_parts=True)
    assert np.array_equal(p0["Ymain"], p1["Ymain"]) and np.array_equal(p0["qx"], p1["qx"])
    assert np.array_equal(p1["T"][:, :r], p0["T"])
