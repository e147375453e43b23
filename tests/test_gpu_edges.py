"""GPU parity on crafted activations that reach every rounding edge of the
quantizers [SVDQuant §3: Q(x) = round(x / s), s = max|x| / q_max; §5.1
implementation details: INT4 group 64 with 16-bit scales, FP4 group 32 with
8-bit power-of-two (MX) scales].

Random inputs with lambda != 1 almost never land on a tie, so this file packs
with no calibration maxima (lambda = 1, x_hat = x) and builds rows whose
quotients x / s sit exactly on the half-integers (INT4) or on the midpoints
of the E2M1 grid (MXFP4), quotients that only a correctly rounded division
puts on a tie, groups past the fp16 scale clamp, all-zero and -0.0 groups,
and groups small enough to take the quantizers' tiny-value paths.  Codes and
scales must match the oracle bit for bit, and the output must pass the usual
gate, row by row (the rows span many orders of magnitude).
"""
import numpy as np
import pytest

import oracle as o
from diffusion_smooth_group_amd import svdq as S
from tests import gpu_common as G

pytestmark = pytest.mark.gpu

K = 512
N = 256


def _pattern(vals, G_):
    """One group: the values cycled with alternating sign, the group's
    maximum placed last."""
    v = np.array([vals[i % len(vals)] * (1 if (i // len(vals)) % 2 == 0 else -1) for i in range(G_ - 1)])
    return v


def _int4_rows(dtype):
    rows = []
    halves = [0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5, 1.0, 3.0, 7.0]
    # max 7: s = 1, every half-integer a tie (ties to even)
    rows.append(np.concatenate([np.append(_pattern(halves, 64), 7.0) for _ in range(K // 64)]))
    # max 3.5: s = 0.5, ties at odd multiples of 0.25
    rows.append(np.concatenate([np.append(_pattern([h / 2 for h in halves], 64), -3.5) for _ in range(K // 64)]))
    # max 21: s = 3, x = 3 (k + 1/2) is a tie only through the exact division
    # (x * fl(1/3) lands just above it)
    thr = [3 * h for h in (0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5)]
    rows.append(np.concatenate([np.append(_pattern(thr, 64), 21.0) for _ in range(K // 64)]))
    # max 77: s = 11, again ties only through the division
    el = [11 * h for h in (0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5)]
    rows.append(np.concatenate([np.append(_pattern(el, 64), -77.0) for _ in range(K // 64)]))
    # an all-zero group, a group of -0.0, then mixed zeros
    z = np.zeros(K)
    z[64:128] = -0.0
    z[128:192] = np.where(np.arange(64) % 2 == 0, -0.0, 0.0)
    z[192:256] = np.where(np.arange(64) % 3 == 0, 2.5, -0.0)
    z[255] = 7.0
    rows.append(z)
    if dtype == o.BF16:
        # max |x| beyond 7 x 65504: the fp16 scale saturates at 65504 and the
        # codes clamp at +-7
        big = np.array([2.0 ** 20, -786432.0, 491520.0, 458752.0, -458752.0, 131072.0, 32768.0, -2048.0] * 8)
        rows.append(np.concatenate([big for _ in range(K // 64)]))
        # max below 7 x 2^-25: the fp16 scale rounds to zero, codes 0
        rows.append(np.concatenate([np.append(_pattern([2.0 ** -30, 3 * 2.0 ** -30, -2.0 ** -27], 64), 2.0 ** -26)
                                    for _ in range(K // 64)]))
    else:
        # fp16 inputs: maxima at the top of the range, and scales in fp16's
        # subnormal range
        rows.append(np.concatenate([np.append(_pattern([1000.0, 3.0e4, 49152.0, 6.0e4], 64), 65504.0)
                                    for _ in range(K // 64)]))
        rows.append(np.concatenate([np.append(_pattern([0.5, 1.5, 2.5, 6.5], 64) * 2.0 ** -20, 7 * 2.0 ** -20)
                                    for _ in range(K // 64)]))
    return rows


def _mx_rows(dtype):
    rows = []
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 3.0, 4.0]
    # max 6: e8m0 = 127 (scale 1), every E2M1 midpoint a tie (ties to even)
    rows.append(np.concatenate([np.append(_pattern(mids, 32), 6.0) for _ in range(K // 32)]))
    # max 12: t = 2 exactly, scale 2, the midpoints doubled
    rows.append(np.concatenate([np.append(_pattern([2 * m for m in mids], 32), -12.0) for _ in range(K // 32)]))
    # max 7: t = 7/6 rounds up to scale 2; midpoints of x / 2
    rows.append(np.concatenate([np.append(_pattern([2 * m for m in mids[:6]], 32), 7.0) for _ in range(K // 32)]))
    # zeros: an all-zero block, an all -0.0 block, mixed signed zeros next to a tie
    z = np.zeros(K)
    z[32:64] = -0.0
    z[64:96] = np.where(np.arange(32) % 2 == 0, -0.0, 0.0)
    z[96:128] = np.where(np.arange(32) % 3 == 0, 0.25, -0.0)
    z[127] = 6.0
    rows.append(z)
    if dtype == o.BF16:
        # tiny blocks: t = max / 6 below the smallest normal fp32 (the
        # exponent comes from the division), and bf16 subnormal inputs
        tiny = 6.0 * 2.0 ** -130
        rows.append(np.concatenate([np.append(_pattern([m * 2.0 ** -130 for m in mids], 32), tiny)
                                    for _ in range(K // 32)]))
        rows.append(np.concatenate([np.append(_pattern([2.0 ** -133, 3 * 2.0 ** -133, 2.0 ** -128], 32), 2.0 ** -127)
                                    for _ in range(K // 32)]))
        # large exponents (the output must stay finite, so not the very top)
        rows.append(np.concatenate([np.append(_pattern([2.0 ** 96, 3 * 2.0 ** 97, 2.0 ** 100], 32), 1.5 * 2.0 ** 100)
                                    for _ in range(K // 32)]))
    else:
        rows.append(np.concatenate([np.append(_pattern([m * 2.0 ** -14 for m in mids], 32), 6 * 2.0 ** -14)
                                    for _ in range(K // 32)]))
        rows.append(np.concatenate([np.append(_pattern([2.0 ** -24, 3 * 2.0 ** -24], 32), 2.0 ** -22)
                                    for _ in range(K // 32)]))
        rows.append(np.concatenate([np.append(_pattern([1000.0, 3.0e4, 49152.0], 32), 65504.0) for _ in range(K // 32)]))
    return rows


def _inputs(fmt, dtype, M, seed):
    rng = np.random.default_rng(seed)
    crafted = _int4_rows(dtype) if fmt == o.INT4 else _mx_rows(dtype)
    X = rng.standard_t(3, (M, K))
    for i, r in enumerate(crafted):
        X[i] = r
    # the crafted rows once more, shuffled in place among random rows, so
    # they also sit in the second token tile
    for i, r in enumerate(crafted):
        X[M - 1 - i] = r[::-1]
    for i, r in enumerate(crafted):
        assert np.array_equal(o.decode16(_bits(r[None, :], dtype), dtype)[0], r), f"row {i} is not exact in {dtype}"
    # fp16 rows reach 65504, so the fp16 weights are smaller: the products,
    # T and Y must stay finite for the output gate
    W = rng.standard_normal((K, N)) * (0.02 if dtype == o.BF16 else 0.02 / 64)
    bias = rng.standard_normal(N) * 0.02
    return _bits(X, dtype), _bits(W, dtype), _bits(bias, dtype), len(crafted)


def _bits(x, dtype):
    x = np.asarray(x, dtype=np.float64)
    if dtype == o.F16:
        return x.astype(np.float16).view(np.uint16)
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _run(fmt, dtype, M, seed, gelu=False):
    import torch
    Xb, Wb, bb, ncraft = _inputs(fmt, dtype, M, seed)
    dev = G.device()
    lin = S.SVDQLinear.pack(Wb, G.DTS[dtype], None, 16, G.FMTS[fmt], bb, rank_capacity=16)
    Xd = S.bits_to_device(Xb, G.DTS[dtype], dev)
    Y = lin.forward(Xd, gelu=gelu)
    torch.cuda.synchronize()
    Yb = S.device_to_bits(Y)
    ex = lin.export()
    assert np.all(ex["lam"] == 1.0) and np.all(ex["invlam"] == 1.0)
    wx = lin.workspace_export(M)
    qx, sx, _ = o.quantize_activations(o.decode16(Xb, dtype), ex["invlam"], fmt)
    assert np.array_equal(wx["codes"].astype(np.int64), np.asarray(qx, np.int64)), "activation codes"
    assert np.array_equal(wx["scales"], sx), "activation scales"
    layer = G.oracle_layer_from_export(ex, Wb, dtype, fmt, 16, bb)
    Yr = o.forward(layer, Xb, gelu=gelu)
    for m in range(M):
        G.compare_outputs(Yb[m:m + 1], Yr[m:m + 1], dtype, what=f"{fmt} {dtype} row {m}")
    return qx, sx, ncraft


@pytest.mark.parametrize("dtype", [o.BF16, o.F16])
def test_int4_ties_clamp_zeros(dtype):
    qx, sx, n = _run(o.INT4, dtype, 45, 1)
    # the crafted rows do reach the edges they were built for
    assert list(qx[0, :7]) == [0, 2, 2, 4, 4, 6, 6]                 # 0.5 .. 6.5 at s = 1
    assert list(qx[2, :7]) == [0, 2, 2, 4, 4, 6, 6]                 # 1.5 .. 19.5 at s = 3
    assert np.all(qx[4, :192] == 0) and np.all(sx[4, :3] == 0)
    if dtype == o.BF16:
        assert np.all(sx[5] == 0x7BFF)                              # fp16 65504: the clamp
        assert list(qx[5, :8]) == [7, -7, 7, 7, -7, 2, 1, 0]
        assert np.all(sx[6] == 0) and np.all(qx[6] == 0)
    else:
        assert np.all((sx[6] > 0) & (sx[6] < 0x0400))               # fp16 subnormal scales


@pytest.mark.parametrize("dtype", [o.BF16, o.F16])
def test_mxfp4_ties_zeros_tiny(dtype):
    qx, sx, n = _run(o.MXFP4, dtype, 45, 2)
    assert np.all(sx[0] == 127)
    # 0.25 0.75 1.25 1.75 2.5 3.5 5 -> 0 1 1 2 2 4 4 (E2M1 codes 0 2 2 4 4 6 6)
    assert list(qx[0, :7]) == [0, 2, 2, 4, 4, 6, 6]
    assert np.all(sx[1] == 128) and list(qx[1, :7]) == [0, 2, 2, 4, 4, 6, 6]
    assert np.all(sx[2] == 128)
    assert sx[3, 0] == 0 and np.all(qx[3, :32] == 0)                # all-zero block
    assert sx[3, 1] == 0 and np.all(qx[3, 32:64] == 8)              # -0.0 keeps its sign bit
    if dtype == o.BF16:
        assert np.all(sx[4] == 1) and np.all(sx[5] == 1)            # t below the smallest normal
        assert np.all(sx[6] == 225)


def test_mxfp4_edges_gelu_more_rows():
    # the same crafted rows among 300 tokens (two token tiles of the GEMM,
    # ragged), GELU in the epilogue
    _run(o.MXFP4, o.BF16, 300, 3, gelu=True)


def test_int4_edges_gelu_more_rows():
    _run(o.INT4, o.BF16, 300, 4, gelu=True)


@pytest.mark.parametrize("scale", [1e-36, 1e-38, 2.0 ** -130])
def test_int8_tiny_token_scales(scale):
    # the 8-bit setting's per-token scale max|x| / 127 falls below 2^-128 (its
    # reciprocal overflows fp32) or into fp32's subnormal range
    import torch
    rng = np.random.default_rng(9)
    M = 40
    X = rng.standard_t(3, (M, K))
    X[3] *= scale
    X[17] = X[17] * scale * 0.01
    X[20] = 0.0
    Xb = _bits(X, o.BF16)
    Wb = _bits(rng.standard_normal((K, N)) * 0.02, o.BF16)
    bb = _bits(rng.standard_normal(N) * 0.02, o.BF16)
    lin = S.SVDQLinear.pack(Wb, S.BF16, None, 16, S.FMT_INT8_W8A8, bb, rank_capacity=16)
    Y = lin.forward(S.bits_to_device(Xb, S.BF16, G.device()))
    torch.cuda.synchronize()
    ex = lin.export()
    wx = lin.workspace_export(M)
    qx, sx, _ = o.quantize_activations(o.decode16(Xb, o.BF16), ex["invlam"], o.INT8)
    assert np.array_equal(wx["codes"].astype(np.int64), np.asarray(qx, np.int64)), "activation codes"
    assert np.array_equal(np.asarray(wx["scales"], np.float32).reshape(-1).view(np.uint32),
                          np.asarray(sx, np.float32).reshape(-1).view(np.uint32)), "activation scales"
    assert np.abs(qx[3]).max() == 127
    layer = G.oracle_layer_from_export(ex, Wb, o.BF16, o.INT8, 16, bb)
    Yr = o.forward(layer, Xb)
    Yb = S.device_to_bits(Y)
    for m in range(M):
        G.compare_outputs(Yb[m:m + 1], Yr[m:m + 1], o.BF16, what=f"int8 row {m}")
