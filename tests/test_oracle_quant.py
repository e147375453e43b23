"""Pins for the oracle's number formats and group quantizers (CPU only).

Each check compares the oracle with something other than itself: numpy /
torch conversions, hand-worked examples from the quantizer definition of
the SVDQuant paper (§3, §5.1; fixtures under tests/golden/), and scalar
re-derivations that use a different formulation (Python's round-half-even,
binade-wise rounding).
"""
import os
import struct

import numpy as np
import pytest
import torch

import oracle as o

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_pairs(name):
    hdr, pairs = [], []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = line.split()
        if len(parts) == 1:
            hdr.append(parts[0])
        else:
            pairs.append((float(parts[0]), parts[1]))
    return hdr, pairs


# ---------------------------------------------------------------- 16-bit types
def test_round16_f16_matches_numpy_double_to_half():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
        (rng.integers(-3000, 3000, 2000) + 0.5) * 2.0 ** -24,      # subnormal ties
        (rng.integers(1, 2000, 2000) * 2 + 1) * 2.0 ** -11,        # ties at 1.x
        np.array([65504.0, 65519.99, 65520.0, -65520.0, 1e6, 2.0 ** -25, 3 * 2.0 ** -26, -0.0, 0.0]),
    ])
    got = o.round16(x, o.F16)
    ref = x.astype(np.float16).view(np.uint16)   # numpy converts double->half directly
    assert np.array_equal(got, ref)


def test_round16_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    x32 = (rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000)).astype(np.float32)
    x32[:100] = (np.arange(100, dtype=np.float32) + 0.5) * np.float32(2.0 ** -7) + 1   # ties
    got = o.round16(x32.astype(np.float64), o.BF16)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_round16_bf16_direct_from_double_no_double_rounding():
    # 1 + 2^-8 + 2^-30 is above the bf16 tie; rounding through fp32 first
    # would drop the 2^-30 and land on the tie (-> 1.0).
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8])
    got = o.decode16(o.round16(x, o.BF16), o.BF16)
    assert list(got) == [1 + 2.0 ** -7, 1.0, 1 + 2.0 ** -6]


# ------------------------------------------------------------------- INT4 g64
def test_int4_worked_example():
    hdr, pairs = _read_pairs("int4_g64_ties.txt")
    v = np.zeros(64, np.float32)
    for i, (x, _) in enumerate(pairs):
        v[i] = x
    q, s = o.quant_int4_g64(v)
    assert int(s) == int(hdr[0], 16)
    assert [int(c) for _, c in pairs] == list(q[:len(pairs)])
    assert not q[len(pairs):].any()


def _int4_scalar(v):
    """Scalar restatement: numpy fp32 scalars for the two fp32 operations,
    struct 'e' for the fp16 scale, Python round() (half-even) for rint."""
    m = max(abs(float(x)) for x in v)
    s = float(np.float32(m) / np.float32(7.0))
    s = min(s, 65504.0)
    sh = struct.unpack("<e", struct.pack("<e", s))[0]
    if sh == 0.0:
        return [0] * len(v), sh
    out = []
    for x in v:
        r = float(np.float32(x) / np.float32(sh))
        out.append(max(-7, min(7, round(r))))
    return out, sh


@pytest.mark.parametrize("scale", [1.0, 1e-3, 3e-7, 1e-9, 37.0, 5e4, 1e6])
def test_int4_against_scalar_restatement(scale):
    rng = np.random.default_rng(int(scale * 1e9) % 2 ** 31)
    v = (rng.standard_normal((40, 64)) * scale).astype(np.float32)
    v[0, :] = 0
    v[1, 5] = np.float32(7 * scale)
    v[1, :5] = np.float32(2.5 * scale)   # ties near 2.5 when 7*scale/7 == scale
    q, s = o.quant_int4_g64(v)
    for i in range(v.shape[0]):
        ref_q, ref_s = _int4_scalar(v[i])
        assert s[i].view(np.float16) == np.float16(ref_s)
        assert list(q[i]) == ref_q, i


def test_int4_error_bound_and_range():
    rng = np.random.default_rng(3)
    v = (rng.standard_t(3, (500, 64)) * 0.3).astype(np.float32)
    q, s = o.quant_int4_g64(v)
    assert np.abs(q).max() <= 7
    d = o.dequant_int4(q, s)
    sh = s.view(np.float16).astype(np.float64)
    # no clipping: |v/s| <= 7 up to the fp16 rounding of s, so error <= s/2
    # plus the part of max|v| above 7*s
    excess = np.maximum(np.abs(v).max(1) - 7 * sh, 0)
    assert np.all(np.abs(d - v).max(1) <= sh / 2 * (1 + 1e-6) + excess)


def test_int4_fp16_scale_clamp():
    v = np.zeros(64, np.float32)
    v[0] = 1e6          # 1e6/7 > 65504 -> scale clamps, codes saturate at 7
    v[1] = -1e6
    v[2] = 65504.0 * 3
    q, s = o.quant_int4_g64(v)
    assert s.view(np.float16) == np.float16(65504.0)
    assert q[0] == 7 and q[1] == -7 and q[2] == 3


# ------------------------------------------------------------------ MXFP4 g32
def test_e2m1_table():
    rows = [l.split() for l in open(os.path.join(GOLD, "e2m1_table.txt")) if l.strip() and not l.startswith("#")]
    for code_hex, val in rows:
        c = np.array([[int(code_hex, 16)] + [0] * 31], np.uint8)
        d = o.dequant_mxfp4(c, np.array([127], np.uint8))
        assert d[0, 0] == float(val) and np.signbit(d[0, 0]) == val.startswith("-")


@pytest.mark.parametrize("fname", ["mxfp4_g32_ties.txt", "mxfp4_g32_scale_up.txt"])
def test_mxfp4_worked_examples(fname):
    hdr, pairs = _read_pairs(fname)
    v = np.zeros(32, np.float32)
    for i, (x, _) in enumerate(pairs):
        v[i] = x
    c, e = o.quant_mxfp4_g32(v)
    assert int(e) == int(hdr[0])
    assert [int(h, 16) for _, h in pairs] == list(c[:len(pairs)])
    assert not c[len(pairs):].any()


def _e2m1_binade(a):
    """Independent RNE onto E2M1 by binade: step 0.5 below 2, 1 in [2,4),
    2 in [4,8); saturate at 6.  Python round() is half-even."""
    a = float(a)
    if a < 2.0:
        r = round(a * 2.0) / 2.0
    elif a < 4.0:
        r = float(round(a))
    else:
        r = round(a / 2.0) * 2.0
    return min(r, 6.0)


def _mx_scalar(v):
    m = max(abs(float(x)) for x in v)
    t = float(np.float32(m) / np.float32(6.0))
    if t == 0.0:
        e = 0
    else:
        fr, ex = np.frexp(t)          # t = fr * 2^ex, fr in [0.5, 1)
        e = int(ex) - 1 + 127 + (1 if fr != 0.5 else 0)
        e = max(e, 1) if t < 2.0 ** -126 else e
        e = min(e, 254)
    codes = []
    grid = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
    for x in v:
        u = float(np.ldexp(np.float32(x), 127 - e))
        mag = grid[_e2m1_binade(abs(u))]
        codes.append(mag | (8 if np.signbit(np.float32(x)) else 0))
    return codes, e


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -20, 3e-3, 7.0, 1e5, 1e-38, 1e30])
def test_mxfp4_against_scalar_restatement(scale):
    rng = np.random.default_rng(11)
    v = (rng.standard_normal((50, 32)) * scale).astype(np.float32)
    v[0] = 0
    v[1, :] = -0.0
    v[2, :4] = np.float32([6 * scale, 0.25 * scale, 0.75 * scale, 5 * scale])
    c, e = o.quant_mxfp4_g32(v)
    for i in range(v.shape[0]):
        rc, re = _mx_scalar(v[i])
        assert int(e[i]) == re, (i, e[i], re)
        assert list(c[i]) == rc, i


def test_mxfp4_scale_is_smallest_power_of_two_covering():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((2000, 32)) * 10.0 ** rng.integers(-8, 8, (2000, 1))).astype(np.float32)
    c, e = o.quant_mxfp4_g32(v)
    t = (np.abs(v).max(1) / np.float32(6)).astype(np.float32).astype(np.float64)
    s = np.ldexp(1.0, e.astype(np.int64) - 127)
    assert np.all(s >= t) and np.all(s / 2 < t)
    d = o.dequant_mxfp4(c, e)
    # every element within half a grid step of its value (no saturation needed)
    u = np.abs(v) / s[:, None]
    step = np.where(u < 2, 0.5, np.where(u < 4, 1.0, 2.0))
    assert np.all(np.abs(d - v) <= step / 2 * s[:, None] * (1 + 1e-12))


def test_group_axis_is_k():
    # per-token groups along K for activations; per-column groups along K for weights
    rng = np.random.default_rng(8)
    X = rng.standard_normal((3, 128)).astype(np.float32)
    X[1, 70] = 100.0
    q, s, _ = o.quantize_activations(X, np.ones(128, np.float32), o.INT4)
    assert s.shape == (3, 2)
    big = s.view(np.float16).astype(np.float32)
    assert big[1, 1] > 10 * big[1, 0] and big[0, 1] < 1
    R = rng.standard_normal((128, 5)).astype(np.float32)
    R[70, 3] = 100.0
    qw, sw = o.quantize_weight(R, o.MXFP4)
    assert sw.shape == (4, 5)
    assert sw[2, 3] > sw[2, 2] + 4 and sw[0, 3] < sw[2, 3]
