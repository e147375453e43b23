"""Pins of the oracle's iterative low-rank refinement [SVDQuant §4.2, the
closing remark on the low-rank branch]: the split error is checked against
a scalar brute force written independently here; the refinement loop is
checked to decompose W_hat - deq(Q(R)) (not W_hat - R, which would return
the one-shot split again) and to keep the smallest error."""
import math

import numpy as np
import pytest

import oracle as o
from diffusion_smooth_group_amd import workloads as wl

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _layer(K, N, dtype, fmt, seed, w_out=3):
    spec = wl.small_spec("r", 64, K, N, dtype, fmt, 8, x_outliers=3, w_outliers=w_out, seed=(seed, 0))
    d = wl.generate(spec)
    a = o.activation_absmax(o.decode16(d["X"], dtype))
    return d, a


def _scalar16(bits, dtype):
    b = int(bits)
    if dtype == o.BF16:
        return float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0])
    return float(np.array([b], dtype=np.uint16).view(np.float16)[0])


@pytest.mark.parametrize("fmt", [o.INT4, o.MXFP4])
def test_split_error_matches_scalar_brute_force(fmt):
    K, N, dt, r = 128, 6, o.BF16, 3
    d, a = _layer(K, N, dt, fmt, 5)
    p = o.pack(d["W"], dt, a, r, fmt)
    err = o.split_error(d["W"], dt, p["lam"], p["L1x"], p["L2q"], p["qw"], p["sw"], fmt)
    G = o.GROUP[fmt]
    ref = 0.0
    for j in range(K):
        lj = float(p["lam"][j])
        for n in range(N):
            w = _scalar16(d["W"][j, n], dt)
            lr = sum(_scalar16(p["L1x"][j, k], dt) * _scalar16(p["L2q"][k, n], dt) for k in range(r))
            if fmt == o.INT4:
                deq = int(p["qw"][j, n]) * _scalar16(p["sw"][j // G, n], o.F16)
            else:
                c = int(p["qw"][j, n])
                deq = (-1.0 if c & 8 else 1.0) * E2M1[c & 7] * math.ldexp(1.0, int(p["sw"][j // G, n]) - 127)
            dd = lj * w - lj * lr - deq
            ref += dd * dd
    assert abs(err - ref) <= 1e-9 * ref


@pytest.mark.parametrize("fmt", [o.INT4, o.MXFP4])
def test_refinement_decomposes_the_quantized_remainder_and_keeps_the_minimum(fmt):
    K, N, dt, r = 256, 192, o.BF16, 8
    d, a = _layer(K, N, dt, fmt, 11)
    out = o.refine_split(d["W"], dt, a, r, fmt, 3)
    rounds = out["rounds"]
    one = o.pack(d["W"], dt, a, r, fmt)
    # round 0 is the one-shot split
    assert np.array_equal(rounds[0]["L1x"], one["L1x"]) and np.array_equal(rounds[0]["qw"], one["qw"])
    # round 1 splits W_hat - deq(Q(R0)): a different target, so different factors
    # (splitting W_hat - R0 = diag(lambda) L1x L2q would give round 0's back)
    assert not np.array_equal(rounds[1]["L1x"], rounds[0]["L1x"])
    What = o.smoothed_weight(o.decode16(d["W"], dt), out["lam"])
    B1 = What - o.dequant_weight(rounds[0]["qw"], rounds[0]["sw"], fmt)
    L1, L2, _ = o.truncated_svd(B1, r)
    assert np.array_equal(o.runtime_factors(L1, L2, out["invlam"], dt)[0], rounds[1]["L1x"])
    errs = [x["err"] for x in rounds]
    assert out["best"] == int(np.argmin(errs))
    # on an outlier-heavy weight the refinement lowers the error
    assert min(errs) < errs[0]
